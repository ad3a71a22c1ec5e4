"""GPU parity: the HIP library through its C ABI against the float64 oracle on
the same seeded inputs.  Floating point within 2e-2 * max|ref| per tensor;
slots, positions and untouched KV bit-exact."""
import numpy as np
import pytest

from chunked_prefill_hybrid_rmsnorm_amd import binding as B
from chunked_prefill_hybrid_rmsnorm_amd.inputs import (bf16_to_f32,
    MISTRAL_7B, TINY, LayerShape, bf16_bits, make_hybrid_batch, make_prompt_sequence,
    mistral_batch, tiny_batch)
from oracle import layer_forward, rmsnorm, silu
from tests.gpu_helpers import (TOL, assert_close, check_layer, require_gpu, run_gpu, run_oracle,
                               tap_f64)
from tests.oracle_inputs import oracle_weights, widen

pytestmark = pytest.mark.gpu

# small shapes exercising head_dim 128 and a group of 8 at tiny sizes
D128 = LayerShape(512, 4, 1, 128, 1024)
G8 = LayerShape(512, 8, 1, 64, 512)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _flush(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- addressing
@pytest.mark.parametrize("which", ["tiny", "mistral"])
def test_slot_mapping_bit_exact(which):
    import torch
    hb = tiny_batch(seed=1) if which == "tiny" else mistral_batch(seed=1, prior_kv="none")
    db = B.DeviceBatch(hb)
    pos = torch.empty(db.M, dtype=torch.int32, device="cuda")
    slot = torch.empty(db.M, dtype=torch.int32, device="cuda")
    B.hl_slot_mapping(db.cfg, db.chunks, db.dec, hb.num_pages, pos, slot)
    torch.cuda.synchronize()
    from oracle import slot_of
    P = hb.shape.page_size
    want_pos, want_slot = [], []
    for c in hb.chunks:
        for i in range(c.length):
            want_pos.append(c.start_pos + i)
            want_slot.append(slot_of(c.start_pos + i, c.block_table, P))
    for j, cl in enumerate(hb.decodes.ctx_lens):
        want_pos.append(int(cl))
        want_slot.append(slot_of(int(cl), hb.decodes.block_tables[j], P))
    np.testing.assert_array_equal(pos.cpu().numpy(), want_pos)
    np.testing.assert_array_equal(slot.cpu().numpy(), want_slot)


# ---------------------------------------------------------------- single steps
def test_rmsnorm_step():
    import torch
    rng = np.random.default_rng(3)
    x = bf16_bits(rng.standard_normal((37, 4096)).astype(np.float32) * 3)
    g = bf16_bits(rng.uniform(0.5, 1.5, 4096).astype(np.float32))
    y = torch.empty((48, 4096), dtype=torch.bfloat16, device="cuda")
    B.hl_rmsnorm(B.bits_to_device(x), B.bits_to_device(g), y, 37, 48, 4096, 1e-5)
    torch.cuda.synchronize()
    got = tap_f64(y, 48)
    assert_close("rmsnorm", got[:37], rmsnorm(widen(x), widen(g), 1e-5))
    assert np.all(got[37:] == 0)


@pytest.mark.parametrize("m,mp,n,k,split", [(68, 80, 512, 256, False),
                                            (288, 288, 6144, 4096, False),
                                            (288, 288, 6144, 4096, True),
                                            (1, 16, 256, 1024, False),
                                            (257, 272, 4096, 14336, False),
                                            (257, 272, 4096, 14336, True),
                                            # 288-row ping-pong tile with one k-step, and
                                            # with two splits of 8 k-steps; ragged last
                                            # column tile
                                            (200, 208, 320, 64, False),
                                            (150, 160, 320, 1024, True),
                                            # small-batch row tiles (64 and 32 rows)
                                            (40, 48, 384, 1024, True),
                                            (25, 32, 256, 2048, False),
                                            # two 256-row tiles (fewer padded rows than 288)
                                            (500, 512, 384, 1024, True),
                                            # 256-weight-row tiles with two stages (two row
                                            # tiles, long k loop): ragged rows, 4 K splits
                                            (300, 304, 8192, 16384, True),
                                            # one-wave-per-SIMD tiles: 160 columns (QKV-like),
                                            # split in two and, without a workspace, unsplit
                                            (560, 576, 10240, 8192, True),
                                            (560, 576, 10240, 8192, False),
                                            # 128 columns (O-like), plain and residual
                                            (570, 576, 8192, 8192, True),
                                            # 128 columns on 256-row tiles, 4 K splits
                                            (500, 512, 4096, 4096, True),
                                            # 224 columns (plain only)
                                            (570, 576, 13440, 2048, True),
                                            # small batches, split counts that are not
                                            # powers of two for the plain epilogue: 5
                                            # (48 column tiles), 3 (80) and 7 (36)
                                            (60, 64, 6144, 4096, True),
                                            (50, 64, 10240, 8192, True),
                                            (30, 32, 4608, 4096, True)])
def test_gemm_step(m, mp, n, k, split):
    """Without a workspace K is not split (one launch, the long-k tile with two
    k-groups for the 288-row shapes); with one the partials are reduced."""
    import torch
    rng = np.random.default_rng(m + n)
    a = np.zeros((mp, k), np.uint16)
    a[:m] = bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    w = bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    r = bf16_bits(rng.standard_normal((m, n)).astype(np.float32))
    ad, wd, rd = B.bits_to_device(a), B.bits_to_device(w), B.bits_to_device(r)
    ws, nbytes = None, 0
    if split:
        nbytes = B.hl_gemm_workspace_bytes(mp, n, k)
        assert nbytes > 0
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    c = torch.empty((mp, n), dtype=torch.bfloat16, device="cuda")
    B.hl_gemm_bf16(ad, wd, c, None, m, mp, n, k, ws, nbytes)
    c2 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    B.hl_gemm_bf16(ad, wd, c2, rd, m, mp, n, k, ws, nbytes)
    torch.cuda.synchronize()
    ref = widen(a) @ widen(w).T
    got = tap_f64(c, mp)
    assert_close("gemm", got, ref)
    assert np.all(got[m:] == 0)
    assert_close("gemm+residual", tap_f64(c2, m), ref[:m] + widen(r))


@pytest.mark.parametrize("mp,f,k", [(32, 1024, 512), (64, 1024, 512), (96, 1024, 512),
                                    (272, 1024, 4096),
                                    # 256-weight-row tiles (128 outputs each) over two row
                                    # tiles; the last column tile is half empty
                                    (560, 14272, 4096)])
def test_swiglu_step(mp, f, k):
    import torch
    rng = np.random.default_rng(5)
    a = bf16_bits(rng.standard_normal((mp, k)).astype(np.float32))
    wg = bf16_bits((rng.standard_normal((f, k)) * 0.05).astype(np.float32))
    wu = bf16_bits((rng.standard_normal((f, k)) * 0.05).astype(np.float32))
    act = torch.empty((mp, f), dtype=torch.bfloat16, device="cuda")
    B.hl_gemm_swiglu(B.bits_to_device(a), B.bits_to_device(wg), B.bits_to_device(wu), act, mp, f, k)
    torch.cuda.synchronize()
    A = widen(a)
    ref = silu(A @ widen(wg).T) * (A @ widen(wu).T)
    assert_close("swiglu", tap_f64(act, mp), ref)


# ---------------------------------------------------------------- whole layer
def test_layer_tiny():
    _flush("tiny: H=256 4/2 heads d64, Lp=64 after 64 cached + 4 decodes")
    hb = tiny_batch(seed=0)
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))


def test_layer_mistral_full_size():
    _flush("mistral-shaped: Lp=256 after 768 cached + 32 decodes ctx U[128,2048]")
    hb = mistral_batch(seed=0, random_gains=True)
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))


EDGE = {
    "decode_only": dict(chunk_lens=[], chunk_starts=[], n_decodes=5, ctx_range=(1, 90)),
    "prefill_only_ragged": dict(chunk_lens=[37], chunk_starts=[0], n_decodes=0),
    "ctx_zero_decodes": dict(chunk_lens=[16], chunk_starts=[16], ctx_lens=[0, 0, 15, 16, 31]),
    "single_row": dict(chunk_lens=[], chunk_starts=[], ctx_lens=[7]),
    "single_chunk_row": dict(chunk_lens=[1], chunk_starts=[100], n_decodes=0),
    "two_chunks": dict(chunk_lens=[20, 45], chunk_starts=[0, 70], n_decodes=3),
    "three_chunks_ragged": dict(chunk_lens=[3, 17, 29], chunk_starts=[5, 0, 33], n_decodes=2),
    "long_decode_multi_partition": dict(chunk_lens=[8], chunk_starts=[0], ctx_lens=[255, 256, 700, 1300]),
    # few chunk rows after a long prefix: the key range is split over workgroups and merged
    "long_prior_chunk_key_split": dict(chunk_lens=[40], chunk_starts=[1000], n_decodes=2),
    "two_long_chunks_key_split": dict(chunk_lens=[33, 7], chunk_starts=[700, 1500], ctx_lens=[31, 32]),
    # the most chunks one call takes (HL_MAX_CHUNKS), ragged lengths and starts
    "sixteen_chunks_max": dict(chunk_lens=[1, 2, 3, 5, 8, 13, 4, 7, 9, 2, 6, 11, 1, 3, 5, 16],
                               chunk_starts=[0, 30, 7, 64, 3, 0, 90, 12, 40, 5, 77, 20, 130, 1, 9, 48],
                               n_decodes=4),
    # more decodes than one wave scans at a time (64): slice search and merge
    # walk several 64-decode blocks
    "many_decodes": dict(chunk_lens=[5], chunk_starts=[3], n_decodes=150, ctx_range=(0, 70)),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_layer_edge_cases(name):
    _flush(f"edge case {name}")
    hb = make_hybrid_batch(TINY, seed=21, random_gains=True, **EDGE[name])
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))


@pytest.mark.parametrize("prefix,ctx", [(6000, 4000), (20000, 8000)], ids=["one_round", "two_pass"])
@pytest.mark.parametrize("shape", [TINY, D128], ids=["d64", "d128"])
def test_merge_of_many_parts(shape, prefix, ctx):
    """A 16-row chunk after a long cached prefix beside one long decode.  With
    6000 cached tokens (21 or 23 key segments) and a 4000-token decode (31
    slices) the rows have 17 to 32 parts, which the merge loads in one round
    with one lane per part; with 20000 (40 or 64 segments) and 8000 (62
    slices) they have more than 32 and take its two-pass path."""
    _flush(f"merge of many parts, head dim {shape.head_dim}, prefix {prefix}, decode ctx {ctx}")
    hb = make_hybrid_batch(shape, chunk_lens=[16], chunk_starts=[prefix], ctx_lens=[ctx, 9],
                           seed=23, random_gains=True)
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))


@pytest.mark.parametrize("shape", [D128, G8], ids=["d128", "group8"])
def test_layer_other_head_shapes(shape):
    hb = make_hybrid_batch(shape, chunk_lens=[40], chunk_starts=[30], n_decodes=3,
                           ctx_range=(200, 600), seed=22, random_gains=True, weight_std=0.03)
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))


@pytest.mark.parametrize("pad", [48, 128, 256])
def test_tile_padding_changes_nothing(pad):
    """Dummy pad rows must not change any real row.  While the padded row count
    keeps the same GEMM tiles (<= 128 rows: the 128-row tile) the results are
    bit-exact; with 256 rows the 288-row tile (and for narrow outputs two
    k-groups, a different fp32 summation order) is used, so the rows match to
    the parity tolerance; pad rows stay zero either way."""
    hb = make_hybrid_batch(TINY, chunk_lens=[57], chunk_starts=[16], n_decodes=3, seed=23)
    _, g16 = run_gpu(hb, pad=16)
    _, gp = run_gpu(hb, pad=pad)
    if pad <= 128:
        np.testing.assert_array_equal(g16["out"], gp["out"])
        np.testing.assert_array_equal(g16["kv"], gp["kv"])
    else:
        assert_close("out (pad 256 vs 16)", gp["out"].astype(np.float64),
                     g16["out"].astype(np.float64))
        # KV bits: only rounding-level flips (<= 2 bf16 ulps) in a few elements
        diff = g16["kv"] != gp["kv"]
        assert diff.mean() < 0.01
        a = bf16_to_f32(g16["kv"][diff]).astype(np.float64)
        b = bf16_to_f32(gp["kv"][diff]).astype(np.float64)
        assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)))
    for k in ("xn2", "act"):
        assert np.all(gp["pad_rows"][k] == 0)


def test_repeat_is_deterministic():
    hb = tiny_batch(seed=24)
    _, a = run_gpu(hb)
    _, b = run_gpu(hb)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["kv"], b["kv"])


# ---------------------------------------------------------------- invariants on the GPU
def _gpu_prompt_in_chunks(seq, n_chunks):
    """Prefill the prompt chunk by chunk through the library; the pages carry
    the state between calls."""
    import torch
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import Chunk, Decodes, HybridBatch
    s = seq.shape
    wt = B.upload_weights(seq.weights)
    kv_t = B.bits_to_device(B.kv_to_library_layout(seq.kv_pages))
    outs = []
    for k in range(n_chunks):
        c = seq.chunk(k)
        hb = HybridBatch(s, seq.weights, seq.chunk_rows(k), [c],
                         Decodes(np.zeros(0, np.int32), np.zeros((0, 0), np.int32)), seq.kv_pages)
        db = B.DeviceBatch(hb, weights=wt)
        db.kv_t = kv_t
        db.kv = B.hl_kv(kv_t.data_ptr(), seq.kv_pages.shape[0])
        db.forward()
        torch.cuda.synchronize()
        outs.append(tap_f64(db.out, db.M))
    kv = B.kv_from_library_layout(B.device_to_bits(kv_t), s.n_kv_heads, s.page_size, s.head_dim)
    return np.concatenate(outs), kv


@pytest.mark.parametrize("n_chunks", [2, 4, 8])
def test_chunked_prefill_equals_unchunked_gpu(n_chunks):
    seq = make_prompt_sequence(TINY, 256, n_chunks, seed=25, random_gains=True)
    whole = make_prompt_sequence(TINY, 256, 1, seed=25, random_gains=True)
    out_c, kv_c = _gpu_prompt_in_chunks(seq, n_chunks)
    out_1, kv_1 = _gpu_prompt_in_chunks(whole, 1)
    w = oracle_weights(whole.weights)
    ref = layer_forward(TINY, w, widen(whole.x_prompt), [(256, 0, whole.block_table)], [], [],
                        widen(whole.kv_pages))
    assert_close("chunked vs oracle", out_c, ref.out)
    assert_close("unchunked vs oracle", out_1, ref.out)
    # rows are computed independently of how the prompt was cut
    np.testing.assert_array_equal(out_c, out_1)
    np.testing.assert_array_equal(kv_c, kv_1)


def test_hybrid_equals_each_request_alone_gpu():
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import Decodes, HybridBatch
    hb = tiny_batch(seed=26)
    _, full = run_gpu(hb, taps=False)
    Lp = hb.chunks[0].length
    alone_c = HybridBatch(hb.shape, hb.weights, hb.x[:Lp], hb.chunks,
                          Decodes(np.zeros(0, np.int32), np.zeros((0, 0), np.int32)), hb.kv_pages)
    _, gc = run_gpu(alone_c, taps=False)
    np.testing.assert_array_equal(full["out"][:Lp], gc["out"])
    for j in range(hb.decodes.n):
        dj = Decodes(hb.decodes.ctx_lens[j:j + 1], hb.decodes.block_tables[j:j + 1])
        one = HybridBatch(hb.shape, hb.weights, hb.x[Lp + j:Lp + j + 1], [], dj, hb.kv_pages)
        _, gd = run_gpu(one, taps=False)
        np.testing.assert_array_equal(full["out"][Lp + j], gd["out"][0])


def test_validate_metadata():
    hb = tiny_batch(seed=27)
    db = B.DeviceBatch(hb)
    assert B.hl_validate_metadata(db.cfg, db.chunks, db.dec, hb.num_pages) == 0
    # a page id past the pool
    assert B.hl_validate_metadata(db.cfg, db.chunks, db.dec, 3) == -6
    # two requests sharing a page
    import torch
    bad = db.dbt_t.clone()
    bad[1, 0] = int(hb.chunks[0].block_table[0])
    dec = B.hl_decodes(db.dec.n, db.dec.ctx_lens, bad.data_ptr(), db.dec.max_blocks, db.dec.max_ctx)
    assert B.hl_validate_metadata(db.cfg, db.chunks, dec, hb.num_pages) == -6


def test_timed_forward_matches_plain_forward():
    """The stage-event variant runs the same kernels: identical output and KV."""
    import torch
    hb = mistral_batch(seed=3, prior_kv="random")
    db = B.DeviceBatch(hb)
    db.forward()
    torch.cuda.synchronize()
    out_plain = db.out.clone()
    kv_plain = db.kv_t.clone()
    db.kv_t.copy_(B.bits_to_device(B.kv_to_library_layout(hb.kv_pages)))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(B.N_STAGES + 1)]
    for e in evs:
        e.record()
    B.hl_layer_forward_timed(db.cfg, db.weights, db.x, db.chunks, db.dec, db.kv, db.out, db.ws,
                             db.ws_bytes, db.pad, evs)
    torch.cuda.synchronize()
    assert torch.equal(db.out.view(torch.int16), out_plain.view(torch.int16))
    assert torch.equal(db.kv_t.view(torch.int16), kv_plain.view(torch.int16))
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(B.N_STAGES)]
    assert all(t >= 0 for t in times)
    names = B.stage_names()
    assert len(set(names)) == B.N_STAGES and names[-1] == "gemm_down_reduce"
    # this batch splits K in the QKV, O and down projections and splits keys
    # in attention: every slot holds a kernel, except the gate/up reduce (the
    # full FFN width fills the CUs without splitting K)
    assert all(t > 0 for n, t in zip(names, times) if n != "gemm_gate_up_reduce")


def test_prefill_attention_without_split_long_prefix():
    """Standalone prefill attention with no workspace (no key split): one
    wave walks > 1024 keys, refilling its block-table window."""
    import torch
    hb = make_hybrid_batch(TINY, chunk_lens=[32], chunk_starts=[2500], n_decodes=0, seed=28,
                           random_gains=True)
    db, gpu = run_gpu(hb)
    ref = run_oracle(hb)
    attn = torch.zeros((db.Mp, TINY.n_q_heads * TINY.head_dim), dtype=torch.bfloat16,
                       device="cuda")
    B.hl_prefill_attention(db.cfg, db.tap_t["qkv"], db.chunks, db.kv, attn)
    torch.cuda.synchronize()
    assert_close("attn (unsplit)", tap_f64(attn, db.M), ref.taps["attn"])
    assert_close("attn (layer)", gpu["attn"], ref.taps["attn"])


def test_layer_head_dim64_four_wave_attention():
    """Head dim 64 with a chunk of 256 row groups (1024 rows x 32 kv heads)
    beside decodes: the attention runs four-wave workgroups (no key split
    inside a workgroup), the path the Llama-70B-shaped batch takes at d = 128."""
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import LayerShape
    _flush("head dim 64, 1024-row chunk x 32 kv heads + 3 decodes (four-wave attention)")
    shape = LayerShape(2048, 32, 32, 64, 1024)
    hb = make_hybrid_batch(shape, chunk_lens=[1024], chunk_starts=[0], n_decodes=3,
                           ctx_range=(30, 200), seed=31, random_gains=True)
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))


def test_layer_llama70_full_size():
    _flush("llama2-70b-shaped: Lp=512 after 3584 cached + 64 decodes ctx U[512,4096]")
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import llama70_batch
    hb = llama70_batch(seed=0, random_gains=True)
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))


@pytest.mark.parametrize("which", ["llama70_tp8", "mistral_tp4"])
def test_layer_tensor_parallel_share_full_size(which):
    """One GPU's share of a tensor-parallel layer at full size (heads and FFN
    columns split, hidden size whole): 1 or 2 kv heads with G = 8."""
    from chunked_prefill_hybrid_rmsnorm_amd import inputs as I
    _flush(f"{which}: tensor-parallel share of the layer, full size")
    hb = getattr(I, f"{which}_batch")(seed=0, random_gains=True)
    _, gpu = run_gpu(hb)
    check_layer(hb, gpu, run_oracle(hb))



def _random_batch_args(seed):
    """Seeded draw of one batch layout: 0-3 chunks with ragged lengths and
    starts, 0-40 decodes with contexts up to 900 tokens, one of the small
    shapes and a padding granularity; at least one row."""
    rng = np.random.default_rng(1000 + seed)
    shape = (TINY, D128, G8)[seed % 3]
    n_chunks = int(rng.integers(0, 4))
    chunk_lens = [int(v) for v in rng.integers(1, 201, size=n_chunks)]
    chunk_starts = [int(v) for v in rng.integers(0, 601, size=n_chunks)]
    n_dec = int(rng.integers(0 if n_chunks else 1, 41))
    ctx_lens = [int(v) for v in rng.integers(0, 901, size=n_dec)]
    pad = (16, 32, 128)[int(rng.integers(0, 3))]
    return shape, dict(chunk_lens=chunk_lens, chunk_starts=chunk_starts, ctx_lens=ctx_lens), pad


@pytest.mark.parametrize("seed", range(24))
def test_layer_random_batches(seed):
    """Seeded random hybrid batches (chunk count, lengths, prefixes, decode
    contexts, shape and padding all drawn) against the oracle."""
    shape, args, pad = _random_batch_args(seed)
    _flush(f"random batch {seed}: {shape} pad={pad} {args}")
    hb = make_hybrid_batch(shape, seed=seed, random_gains=True, **args)
    _, gpu = run_gpu(hb, pad=pad)
    check_layer(hb, gpu, run_oracle(hb))

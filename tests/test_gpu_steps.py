"""Per-step GPU parity of the stand-alone entry points that the layer call
does not route through: hl_rope_kv_append and hl_decode_attention, each
through the C ABI against the oracle's pieces on seeded inputs; and the
streaming-read measurement aid against a host XOR.

Floating point within 2e-2 * max|ref| per tensor; copied bf16 values (V) and
every KV slot or output row the step must not touch bit-exact."""
import numpy as np
import pytest

from chunked_prefill_hybrid_rmsnorm_amd import binding as B
from chunked_prefill_hybrid_rmsnorm_amd.inputs import (
    LLAMA2_70B, MISTRAL_7B, SENTINEL_BF16, TINY, LayerShape, Weights, bf16_bits, make_hybrid_batch,
    pages_for)
from oracle import attention_row, rope_rotate
from oracle.layer import gather_request_kv
from tests.gpu_helpers import assert_close, require_gpu, tap_f64
from tests.oracle_inputs import widen

pytestmark = pytest.mark.gpu

D128 = LayerShape(512, 4, 1, 128, 1024)
G8 = LayerShape(512, 8, 1, 64, 512)
SHAPES = {"tiny": TINY, "d128": D128, "g8": G8, "mistral": MISTRAL_7B}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _no_weights():
    z = np.zeros(1, np.uint16)
    return Weights(z, z, z, z, z, z, z)


# ---------------------------------------------------------------- RoPE + KV append
@pytest.mark.parametrize("name", ["tiny", "d128", "g8", "mistral"])
def test_rope_kv_append_step(name):
    """Rows at scattered positions (0 included) and distinct slots of a
    shuffled pool; one row with slot -1 and one naming a page past the pool
    rotate but write nothing."""
    import torch
    s = SHAPES[name]
    print(f"rope_kv_append step: {name} shape", flush=True)
    rng = np.random.default_rng(21)
    P, nq, nkv, d = s.page_size, s.n_q_heads, s.n_kv_heads, s.head_dim
    rows, num_pages = 53, 24
    qkv = bf16_bits(rng.standard_normal((rows, s.qkv_rows)).astype(np.float32))
    pos = rng.integers(0, 5000, size=rows)
    pos[0] = 0
    slots = rng.permutation(num_pages * P)[:rows].astype(np.int64)
    slots[7] = -1
    slots[11] = num_pages * P + 5  # page num_pages: outside the pool
    kv0 = np.full((num_pages, 2, nkv, P, d), SENTINEL_BF16, dtype=np.uint16)
    kv0[rng.random(kv0.shape) < 0.3] = 0x3F80  # some slots hold 1.0

    qkv_t = B.bits_to_device(qkv)
    kv_t = B.bits_to_device(B.kv_to_library_layout(kv0))
    kv = B.hl_kv(kv_t.data_ptr(), num_pages)
    B.hl_rope_kv_append(B.make_config(s), qkv_t, B.int32_to_device(pos), B.int32_to_device(slots),
                        rows, kv)
    torch.cuda.synchronize()
    got = tap_f64(qkv_t, rows)
    got_bits = B.device_to_bits(qkv_t)
    kv_after = B.kv_from_library_layout(B.device_to_bits(kv_t), nkv, P, d)

    u = widen(qkv)
    want_q = np.stack([np.concatenate([rope_rotate(u[r, h * d:(h + 1) * d], pos[r], s.rope_theta)
                                       for h in range(nq)]) for r in range(rows)])
    kq0 = nq * d
    want_k = np.stack([np.concatenate([rope_rotate(u[r, kq0 + g * d:kq0 + (g + 1) * d], pos[r],
                                                   s.rope_theta) for g in range(nkv)])
                       for r in range(rows)])
    assert_close("q (rotated)", got[:, :kq0], want_q)
    assert_close("k (rotated)", got[:, kq0:kq0 + nkv * d], want_k)
    vq0 = (nq + nkv) * d
    np.testing.assert_array_equal(got_bits[:, vq0:], qkv[:, vq0:])  # V is not rotated
    # position 0 turns nothing: q and k come back bit for bit
    np.testing.assert_array_equal(got_bits[0, :vq0], qkv[0, :vq0])

    written = np.zeros(kv0.shape, dtype=bool)
    for r in range(rows):
        if slots[r] < 0 or slots[r] >= num_pages * P:
            continue
        page, off = divmod(int(slots[r]), P)
        assert_close(f"K row {r}", widen(kv_after[page, 0, :, off]).reshape(-1),
                     want_k[r], tol=2e-2)
        # the cached K is the rotated k the step wrote back into qkv
        np.testing.assert_array_equal(kv_after[page, 0, :, off].reshape(-1),
                                      got_bits[r, kq0:kq0 + nkv * d])
        np.testing.assert_array_equal(kv_after[page, 1, :, off].reshape(-1), qkv[r, vq0:])
        written[page, :, :, off] = True
    np.testing.assert_array_equal(kv_after[~written], kv0[~written])


# ---------------------------------------------------------------- decode attention
def _decode_case(shape, ctx_lens, seed):
    """Decodes only; every cached key plus the decode's own key (position
    ctx) holds N(0, 1) bf16 values, as after the layer's append step."""
    hb = make_hybrid_batch(shape, chunk_lens=[], chunk_starts=[], ctx_lens=ctx_lens, seed=seed,
                           weights=_no_weights())
    rng = np.random.default_rng(seed + 1)
    P = shape.page_size
    kv = hb.kv_pages.copy()
    for j, c in enumerate(hb.decodes.ctx_lens):
        page = hb.decodes.block_tables[j][int(c) // P]
        kv[page, :, :, int(c) % P, :] = bf16_bits(
            rng.standard_normal((2, shape.n_kv_heads, shape.head_dim)).astype(np.float32))
    return hb, kv


@pytest.mark.parametrize("name,ctx", [
    ("tiny", [16, 0, 128, 77, 1]),
    ("d128", [0, 31, 32, 33, 500, 1500]),
    ("g8", [5, 1023, 1024, 1025, 2100]),
    # many decodes of the Mistral shape: slices cover several short decodes
    ("mistral", list(np.random.default_rng(3).integers(0, 2048, size=40))),
    # Llama-2-70B shape (group 8, 64 decodes): long contexts cross block-table windows
    ("llama70", list(np.random.default_rng(4).integers(512, 4096, size=64))),
])
def test_decode_attention_step(name, ctx):
    import torch
    s = LLAMA2_70B if name == "llama70" else SHAPES[name]
    print(f"decode_attention step: {name} shape, {len(ctx)} decodes, max ctx {max(ctx)}", flush=True)
    hb, kv_bits = _decode_case(s, ctx, seed=31)
    nq, nkv, d, P = s.n_q_heads, s.n_kv_heads, s.head_dim, s.page_size
    G = nq // nkv
    n, row0 = hb.decodes.n, 3
    rows = row0 + n + 2
    rng = np.random.default_rng(32)
    qkv = bf16_bits(rng.standard_normal((rows, s.qkv_rows)).astype(np.float32))
    cfg = B.make_config(s)
    ctx_t = B.int32_to_device(hb.decodes.ctx_lens)
    bt_t = B.int32_to_device(hb.decodes.block_tables)
    dec = B.hl_decodes(n, ctx_t.data_ptr(), bt_t.data_ptr(), hb.decodes.max_blocks,
                       hb.decodes.max_ctx)
    kv_t = B.bits_to_device(B.kv_to_library_layout(kv_bits))
    kv_before = kv_t.clone()
    kv = B.hl_kv(kv_t.data_ptr(), hb.num_pages)
    fill = np.full((rows, nq * d), 0x7FA5, np.uint16)
    attn = B.bits_to_device(fill)
    ws_bytes = B.hl_decode_workspace_bytes(cfg, n, hb.decodes.max_ctx)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    B.hl_decode_attention(cfg, B.bits_to_device(qkv), row0, dec, kv, attn, ws, ws_bytes)
    torch.cuda.synchronize()

    got_bits = B.device_to_bits(attn)
    np.testing.assert_array_equal(got_bits[:row0], fill[:row0])
    np.testing.assert_array_equal(got_bits[row0 + n:], fill[row0 + n:])
    assert torch.equal(kv_t.view(torch.int16), kv_before.view(torch.int16)), "pages changed"

    kv64 = widen(kv_bits)
    q = widen(qkv)
    want = np.zeros((n, nq * d))
    for j, c in enumerate(hb.decodes.ctx_lens):
        K, V = gather_request_kv(kv64, hb.decodes.block_tables[j], int(c) + 1, P)
        for h in range(nq):
            qh = q[row0 + j, h * d:(h + 1) * d]
            want[j, h * d:(h + 1) * d] = attention_row(qh, K[h // G], V[h // G])
    got = tap_f64(attn, rows)[row0:row0 + n]
    assert_close("decode attn", got, want)
    # ctx = 0: the decode attends its own key only, so it returns its own v
    for j, c in enumerate(hb.decodes.ctx_lens):
        if c == 0:
            page = hb.decodes.block_tables[j][0]
            for h in range(nq):
                np.testing.assert_allclose(got[j, h * d:(h + 1) * d], kv64[page, 1, h // G, 0],
                                           rtol=2 ** -8, atol=0)


# ---------------------------------------------------------------- streaming read (measurement aid)
def test_read_stream_reads_every_word_once():
    """hl_read_stream leaves one XOR per workgroup: over 512 MiB of seeded
    random words the XOR of the 8192 results equals the XOR of the buffer
    computed on the host, and every word of the result array is written."""
    import torch
    print("streaming read over 512 MiB", flush=True)
    n = (512 << 20) // 4
    g = torch.Generator(device="cpu").manual_seed(7)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (n,), dtype=torch.int32, generator=g)
    buf = host.to("cuda")
    sink = torch.full((8192 + 1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    B.hl_read_stream(buf, n * 4, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    assert int(np.bitwise_xor.reduce(got[:8192])) == want
    assert got[8192] == 0x5A5A5A5A, "wrote past the 8192 results"

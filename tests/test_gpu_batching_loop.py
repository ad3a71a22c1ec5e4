"""The batching loop around the layers on the GPU (stall-free batching,
Sarathi-Serve digest, Algorithm 3).

* the embedding gather and the greedy choice, kernel by kernel;
* a tiny two-layer model run by the loop: with the GPU's own tokens fed back
  (teacher forcing), the oracle replays every iteration, and each sampled
  row's logits match it; every generated id is the argmax of its row's
  logits, ties to the lowest id (the generated ids themselves are compared
  only through that rule: a near-tie may legitimately flip)."""
import numpy as np
import pytest

from chunked_prefill_hybrid_rmsnorm_amd import binding as B
from chunked_prefill_hybrid_rmsnorm_amd.inputs import TINY, bf16_bits, bf16_to_f32, draw_weights
from oracle import greedy, model_batch
from tests.gpu_helpers import assert_close, require_gpu
from tests.oracle_inputs import oracle_weights, widen

pytestmark = pytest.mark.gpu


def test_embed_rows_gathers_and_clamps():
    import torch
    require_gpu()
    rng = np.random.default_rng(40)
    V, H = 50, 64
    table = bf16_bits(rng.standard_normal((V, H)).astype(np.float32))
    last = np.array([7, 49, 0], dtype=np.int32)
    ids = np.array([3, -1, 0, -3, 49, 60, -9, -2], dtype=np.int32)
    out = torch.empty((len(ids), H), dtype=torch.bfloat16, device="cuda")
    B.hl_embed_rows(B.bits_to_device(table), V, H, B.int32_to_device(ids),
                    B.int32_to_device(last), len(ids), out)
    torch.cuda.synchronize()
    # -1 -> slot 0, -3 -> slot 2, 60 -> clamped to 49, -9 -> slot clamped to 2
    want = [3, 7, 0, 0, 49, 49, 0, 49]
    np.testing.assert_array_equal(B.device_to_bits(out), table[want])


def test_argmax_rows_ties_and_skips():
    import torch
    require_gpu()
    V = 700
    lg = np.full((4, V), -3.0, dtype=np.float32)
    lg[0, [5, 300, 699]] = 2.0          # tie: lowest id wins
    lg[1, 650] = 1.0
    lg[1, 10] = np.nan                  # NaN never wins
    lg[2, 3] = 9.0                      # row not sampled
    lg[3, 123] = 0.5
    bits = bf16_bits(lg)
    sreq = np.array([0, 1, -1, 5], dtype=np.int32)   # slot 5 is out of range: skipped
    spos = np.array([2, 9, 0, 1], dtype=np.int32)
    last = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    outt = torch.full((10,), -7, dtype=torch.int32, device="cuda")
    B.hl_argmax_rows(B.bits_to_device(bits), 4, V, B.int32_to_device(sreq),
                     B.int32_to_device(spos), last, outt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(last.cpu().numpy(), [5, 650, -7])
    o = outt.cpu().numpy()
    assert o[2] == 5 and o[9] == 650 and (np.delete(o, [2, 9]) == -7).all()


def test_loop_matches_oracle_under_teacher_forcing():
    import torch
    from chunked_prefill_hybrid_rmsnorm_amd.batching_loop import BatchingLoop, Model
    require_gpu()
    print("tiny 2-layer model, 5 requests, budget 16, 4 generated tokens each", flush=True)
    rng = np.random.default_rng(41)
    V, L, gen = 512, 2, 4
    layers = [draw_weights(rng, TINY, 0.05, True) for _ in range(L)]
    table = bf16_bits(rng.standard_normal((V, TINY.hidden)).astype(np.float32))
    lm = bf16_bits((rng.standard_normal((V, TINY.hidden)) * 0.05).astype(np.float32))
    gfin = bf16_bits(rng.uniform(0.5, 1.5, TINY.hidden).astype(np.float32))
    prompts = [rng.integers(0, V, size=n).astype(np.int32) for n in (5, 17, 30, 9, 12)]
    model = Model.from_host(TINY, layers, table, lm, gfin)
    loop = BatchingLoop(model, prompts, gen, budget=16, seed=42)
    stats, records = loop.run(record=True)
    toks = loop.tokens()
    assert (toks >= 0).all() and (toks < V).all()
    assert stats.iterations == len(records)
    assert any(len(r.chunks) > 1 for r in records), "no multi-chunk batch in this schedule"
    assert any(r.chunks and r.decodes for r in records), "no hybrid batch in this schedule"

    ow = [oracle_weights(w) for w in layers]
    s = TINY
    kv = [np.zeros((loop.num_pages, 2, s.n_kv_heads, s.page_size, s.head_dim))
          for _ in range(L)]
    for it, rec in enumerate(records):
        ids = []
        for rid, start, length in rec.chunks:
            ids += list(prompts[rid][start:start + length])
        for rid, ctx in zip(rec.decodes, rec.ctx_lens):
            ids.append(int(toks[rid, ctx - len(prompts[rid])]))
        chunks = [(length, start, loop.bt[rid][:loop.n_blocks[rid]])
                  for rid, start, length in rec.chunks]
        bts = loop.bt[rec.decodes] if rec.decodes else np.zeros((0, loop.max_blocks), np.int32)
        logits, kv = model_batch(s, ow, widen(table), widen(lm), widen(gfin), ids, chunks,
                                 rec.ctx_lens, bts, kv)
        rows = [r for r, _, _ in rec.samples]
        assert_close(f"iteration {it} logits", rec.logits.astype(np.float64), logits[rows])
        got = greedy(rec.logits)
        for i, (_, rid, k) in enumerate(rec.samples):
            assert toks[rid, k] == got[i], (it, rid, k)


def test_loop_mistral_shape_matches_oracle_under_teacher_forcing():
    """The loop's real shapes: Mistral-7B-shaped layers (4 of the 32), vocabulary
    32000, 32 requests with prompts U{50..500}, budget 512.  The first two
    iterations -- many prompt chunks in one batch, then decodes piggybacked on
    chunks -- replayed by the oracle with the GPU's own tokens."""
    from chunked_prefill_hybrid_rmsnorm_amd.batching_loop import BatchingLoop, Model, cfg5_prompts
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import MISTRAL_7B
    require_gpu()
    print("mistral-shaped 4-layer model, vocab 32000, 32 requests, budget 512, 2 iterations",
          flush=True)
    rng = np.random.default_rng(43)
    V, L, gen, s = 32000, 4, 100, MISTRAL_7B
    layers = [draw_weights(rng, s, 0.02, True) for _ in range(L)]
    table = bf16_bits(rng.standard_normal((V, s.hidden), dtype=np.float32))
    lm = bf16_bits(rng.standard_normal((V, s.hidden), dtype=np.float32) * np.float32(0.02))
    gfin = bf16_bits(rng.uniform(0.5, 1.5, s.hidden).astype(np.float32))
    prompts = cfg5_prompts(32, V, seed=44)
    model = Model.from_host(s, layers, table, lm, gfin)
    loop = BatchingLoop(model, prompts, gen, budget=512, seed=45)
    _, records = loop.run(record=True, max_iterations=2)
    toks = loop.tokens()
    assert len(records) == 2
    assert len(records[0].chunks) > 1, "first batch should hold several prompt chunks"
    assert records[1].chunks and records[1].decodes, "second batch should be hybrid"
    print("oracle replay ...", flush=True)
    ow = [oracle_weights(w) for w in layers]
    kv = [np.zeros((loop.num_pages, 2, s.n_kv_heads, s.page_size, s.head_dim))
          for _ in range(L)]
    tab64, lm64, g64 = widen(table), widen(lm), widen(gfin)
    for it, rec in enumerate(records):
        ids = []
        for rid, start, length in rec.chunks:
            ids += list(prompts[rid][start:start + length])
        for rid, ctx in zip(rec.decodes, rec.ctx_lens):
            ids.append(int(toks[rid, ctx - len(prompts[rid])]))
        assert len(ids) <= 512
        chunks = [(length, start, loop.bt[rid][:loop.n_blocks[rid]])
                  for rid, start, length in rec.chunks]
        bts = loop.bt[rec.decodes] if rec.decodes else np.zeros((0, loop.max_blocks), np.int32)
        logits, kv = model_batch(s, ow, tab64, lm64, g64, ids, chunks, rec.ctx_lens, bts, kv)
        rows = [r for r, _, _ in rec.samples]
        assert_close(f"iteration {it} logits ({len(ids)} rows, {len(rows)} sampled)",
                     rec.logits.astype(np.float64), logits[rows])
        got = greedy(rec.logits)
        for i, (_, rid, k) in enumerate(rec.samples):
            assert toks[rid, k] == got[i], (it, rid, k)

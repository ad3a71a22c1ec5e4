"""Stall-free batching (host logic, CPU): the iteration rules of the
Sarathi-Serve digest's Algorithm 3 checked as invariants over whole runs."""
import numpy as np
import pytest

from chunked_prefill_hybrid_rmsnorm_amd.scheduler import StallFreeScheduler


def run(prompts, gen_len, budget):
    s = StallFreeScheduler(prompts, gen_len, budget)
    log = []
    while True:
        b = s.next_batch()
        if b is None:
            break
        running_decoders = [r for r in s.running if s.reqs[r].prefill_done and r not in
                            [c.rid for c in b.chunks]]
        ctx = {r: s.decode_context(r) for r in b.decodes}
        log.append((b, sorted(running_decoders), ctx))
        s.commit(b)
        assert len(log) < 10000
    return s, log


@pytest.mark.parametrize("prompts,gen_len,budget", [
    ([5, 17, 30, 9, 12], 4, 16),
    ([50, 500, 120, 7, 333, 64], 10, 128),
    (list(np.random.default_rng(3).integers(50, 500, size=32)), 100, 512),
])
def test_iteration_rules(prompts, gen_len, budget):
    s, log = run(prompts, gen_len, budget)
    admitted = []
    for b, decoders, ctx in log:
        # every request past its prompt decodes in every iteration until done
        assert sorted(b.decodes) == decoders
        # the budget bounds the rows whenever the decodes alone fit in it
        if len(b.decodes) <= budget:
            assert b.n_rows <= budget
        # new requests come in arrival order; at most one chunk continues a prompt
        for c in b.chunks:
            if c.start == 0 and c.rid not in admitted:
                admitted.append(c.rid)
        assert sum(1 for c in b.chunks if c.start > 0) <= 1
        # decode rows sit at the position after the prompt and the earlier tokens
        for r in b.decodes:
            req = s.reqs[r]
            assert ctx[r] >= req.prompt_len
    assert admitted == list(range(len(prompts)))


@pytest.mark.parametrize("prompts,gen_len,budget", [([5, 17, 30, 9, 12], 4, 16),
                                                    ([50, 500, 120, 7], 10, 64)])
def test_every_token_once_in_order(prompts, gen_len, budget):
    s, log = run(prompts, gen_len, budget)
    prefilled = {i: 0 for i in range(len(prompts))}
    tokens = {i: [] for i in range(len(prompts))}
    for b, _, _ in log:
        for c in b.chunks:
            # each prompt is prefilled contiguously from its start
            assert c.start == prefilled[c.rid]
            prefilled[c.rid] += c.length
        rows = b.n_rows
        for row, rid, k in b.samples:
            assert 0 <= row < rows
            tokens[rid].append(k)
    for i, p in enumerate(prompts):
        assert prefilled[i] == p
        assert tokens[i] == list(range(gen_len))
    assert all(r.done for r in s.reqs)


def test_chunk_sample_is_its_last_row_and_decodes_follow_chunks():
    s = StallFreeScheduler([3, 4], 2, 16)
    b = s.next_batch()
    assert [(c.rid, c.start, c.length) for c in b.chunks] == [(0, 0, 3), (1, 0, 4)]
    assert b.samples == [(2, 0, 0), (6, 1, 0)]
    s.commit(b)
    b = s.next_batch()
    assert b.chunks == [] and b.decodes == [0, 1]
    assert b.samples == [(0, 0, 1), (1, 1, 1)]
    assert [s.decode_context(r) for r in b.decodes] == [3, 4]
    s.commit(b)
    assert s.next_batch() is None


def test_long_prompt_is_chunked_beside_decodes():
    # request 0 decodes while request 1's long prompt is cut to the budget left
    s = StallFreeScheduler([2, 40], 5, 8)
    b = s.next_batch()
    assert [(c.rid, c.start, c.length) for c in b.chunks] == [(0, 0, 2), (1, 0, 6)]
    s.commit(b)
    b = s.next_batch()
    assert b.decodes == [0] and [(c.rid, c.start, c.length) for c in b.chunks] == [(1, 6, 7)]
    assert b.n_rows == 8


def test_bad_arguments():
    with pytest.raises(ValueError):
        StallFreeScheduler([3, 0], 2, 16)
    with pytest.raises(ValueError):
        StallFreeScheduler([3], 2, 0)


def test_chunk_count_capped_at_the_layer_limit():
    """Many short prompts: a batch never holds more chunks than one layer call
    takes (16), and every prompt is still admitted in arrival order."""
    from chunked_prefill_hybrid_rmsnorm_amd.binding import HL_MAX_CHUNKS
    prompts = [3] * 40
    s, log = run(prompts, 2, 512)
    assert max(len(b.chunks) for b, _, _ in log) == HL_MAX_CHUNKS
    order = [c.rid for b, _, _ in log for c in b.chunks if c.start == 0]
    assert order == list(range(len(prompts)))
    s2 = StallFreeScheduler(prompts, 2, 512, max_chunks=5)
    b = s2.next_batch()
    assert len(b.chunks) == 5 and b.n_rows == 15


def test_max_batch_capacity_formula():
    """B = floor((MG - MS) / (L * mkv)) (intelliparadigm.com article, section
    4.1), pinned on hand-computed values."""
    from chunked_prefill_hybrid_rmsnorm_amd.scheduler import kv_bytes_per_token_model, max_batch
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import MISTRAL_7B
    # one token of a 32-layer Mistral-7B-shaped model: 2 (K, V) x 8 kv heads x 128 x 2 B x 32
    mkv = kv_bytes_per_token_model(MISTRAL_7B, 32)
    assert mkv == 131072
    # 288 GB card, 14.5 GB of bf16 parameters, 4096-token sequences:
    # (288e9 - 14.5e9) / (4096 * 131072) = 509.4... -> 509
    assert max_batch(288 * 10**9, 145 * 10**8, 4096, mkv) == 509
    # exact multiples land on the boundary, one byte less drops one request
    assert max_batch(10 * 4096 * mkv, 0, 4096, mkv) == 10
    assert max_batch(10 * 4096 * mkv - 1, 0, 4096, mkv) == 9
    # a fifth kept free: (0.8 * 288e9 - 14.5e9) / 536870912 = 402.1... -> 402
    assert max_batch(288 * 10**9, 145 * 10**8, 4096, mkv, reserve=0.2) == 402
    # parameters filling the card leave no room (never negative)
    assert max_batch(10**9, 2 * 10**9, 4096, mkv) == 0


def test_max_batch_rejects_bad_sizes():
    import pytest
    from chunked_prefill_hybrid_rmsnorm_amd.scheduler import max_batch
    with pytest.raises(ValueError):
        max_batch(100, 0, 0, 8)
    with pytest.raises(ValueError):
        max_batch(100, 0, 8, 8, reserve=1.0)

"""Pins of the batching-loop oracle (CPU): the embedding gather, the greedy
tie rule, and invariants of the layer stack (a prompt prefilled in two calls
equals one call; rows of a batch are independent)."""
import numpy as np

from chunked_prefill_hybrid_rmsnorm_amd.inputs import TINY, bf16_bits, draw_weights, pages_for
from oracle import embed, greedy, model_batch
from tests.oracle_inputs import oracle_weights, widen

V, L = 64, 2


def test_embed_is_one_hot_product():
    rng = np.random.default_rng(0)
    table = rng.standard_normal((V, 16))
    ids = [3, 0, 63, 3, 17]
    onehot = np.zeros((len(ids), V))
    onehot[np.arange(len(ids)), ids] = 1.0
    np.testing.assert_array_equal(embed(table, ids), onehot @ table)


def test_greedy_ties_go_to_the_lowest_id():
    logits = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -1.0, -3.0]])
    np.testing.assert_array_equal(greedy(logits), [1, 0, 0])


def _model(seed=0):
    rng = np.random.default_rng(seed)
    layers = [oracle_weights(draw_weights(rng, TINY, 0.05, True)) for _ in range(L)]
    table = widen(bf16_bits(rng.standard_normal((V, TINY.hidden)).astype(np.float32)))
    lm = widen(bf16_bits((rng.standard_normal((V, TINY.hidden)) * 0.05).astype(np.float32)))
    g = widen(bf16_bits(rng.uniform(0.5, 1.5, TINY.hidden).astype(np.float32)))
    return layers, table, lm, g


def _pools(n_pages):
    P, s = TINY.page_size, TINY
    return [np.zeros((n_pages, 2, s.n_kv_heads, P, s.head_dim)) for _ in range(L)]


def test_prompt_in_two_calls_equals_one_call():
    layers, table, lm, g = _model(1)
    ids = list(np.random.default_rng(2).integers(0, V, size=21))
    bt = list(range(pages_for(21, TINY.page_size)))
    one, _ = model_batch(TINY, layers, table, lm, g, ids, [(21, 0, bt)], [], [], _pools(len(bt)))
    kv = _pools(len(bt))
    a, kv = model_batch(TINY, layers, table, lm, g, ids[:8], [(8, 0, bt)], [], [], kv)
    b, kv = model_batch(TINY, layers, table, lm, g, ids[8:], [(13, 8, bt)], [], [], kv)
    np.testing.assert_allclose(np.concatenate([a, b]), one, rtol=1e-9, atol=1e-9)


def test_rows_of_a_batch_are_independent():
    layers, table, lm, g = _model(3)
    rng = np.random.default_rng(4)
    p_ids = list(rng.integers(0, V, size=9))
    # request 1 already holds 5 cached tokens (written by an earlier call)
    hist = list(rng.integers(0, V, size=5))
    bt0, bt1 = [0], [1]
    kv = _pools(2)
    _, kv = model_batch(TINY, layers, table, lm, g, hist, [(5, 0, bt1)], [], [], kv)
    both, _ = model_batch(TINY, layers, table, lm, g, p_ids + [7], [(9, 0, bt0)], [5],
                          np.array([bt1]), [k.copy() for k in kv])
    alone_p, _ = model_batch(TINY, layers, table, lm, g, p_ids, [(9, 0, bt0)], [], [],
                             [k.copy() for k in kv])
    alone_d, _ = model_batch(TINY, layers, table, lm, g, [7], [], [5], np.array([bt1]),
                             [k.copy() for k in kv])
    np.testing.assert_allclose(both, np.concatenate([alone_p, alone_d]), rtol=1e-9, atol=1e-9)
    assert greedy(both).shape == (10,)


def test_model_batch_equals_dense_torch_stack():
    """The whole composition against library routines: embedding rows, each
    layer as a dense torch layer (contiguous K/V, causal SDPA), then
    F.rms_norm with the final gain and F.linear with the LM head.  Dropping
    the final norm, its gain or its eps, or transposing the head, fails."""
    import torch
    import torch.nn.functional as F
    from tests.test_oracle_layer import dense_layer_torch

    layers, table, lm, g = _model(5)
    ids = list(np.random.default_rng(6).integers(0, V, size=19))
    bt = list(range(pages_for(19, TINY.page_size)))
    logits, _ = model_batch(TINY, layers, table, lm, g, ids, [(19, 0, bt)], [], [],
                            _pools(len(bt)))
    x = table[np.asarray(ids)]
    for w in layers:
        x, _, _ = dense_layer_torch(TINY, w, x)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    xn = F.rms_norm(t(x), (TINY.hidden,), t(g), eps=TINY.rms_eps)
    ref = F.linear(xn, t(lm)).numpy()
    np.testing.assert_allclose(logits, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
    # the pin is sensitive to the final norm: without it (or its gain) the
    # logits move far beyond the tolerance above
    no_norm = F.linear(t(x), t(lm)).numpy()
    no_gain = F.linear(F.rms_norm(t(x), (TINY.hidden,), eps=TINY.rms_eps), t(lm)).numpy()
    for wrong in (no_norm, no_gain):
        assert np.abs(wrong - logits).max() > 1e-3 * np.abs(ref).max()

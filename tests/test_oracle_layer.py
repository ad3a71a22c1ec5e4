"""Layer-level pins of the oracle (CPU only).

* brute-force dense layer from library routines (contiguous K/V, explicit
  causal attention, no pages) on a single prompt;
* chunked prefill equals unchunked prefill (the chunk must keep cross-chunk
  attention correct: intelliparadigm.com section 3.1; Sarathi-Serve digest
  section 2 Q2 item 1);
* a hybrid batch equals running each request alone (a mismatch between the
  two is the pages' own symptom of a wrong mask, broken position continuity
  or a missing sync: intelliparadigm.com section 6.1);
* a decode step equals the last row of a full prefill of the same tokens;
* the prior-KV reads of N chunk calls sum to the N(N-1)/2 closed form
  (Sarathi-Serve digest, section 4, check 4);
* only the expected KV slots change.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from chunked_prefill_hybrid_rmsnorm_amd.inputs import (
    TINY, LayerShape, make_hybrid_batch, make_prompt_sequence, tiny_batch)
from oracle import layer_forward, prefix_reread_loads, slot_of
from tests.oracle_inputs import oracle_args, oracle_weights, widen


def dense_layer_torch(shape, w, x):
    """Pre-norm GQA layer over one prompt at positions 0..T-1, written with
    torch library routines and contiguous K/V."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    H, nq, nkv, d = shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    T = x.shape[0]
    xn = F.rms_norm(t(x), (H,), t(w["g_attn"]), eps=shape.rms_eps)
    qkv = F.linear(xn, t(w["w_qkv"]))
    q = qkv[:, :nq * d].reshape(T, nq, d)
    k = qkv[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d)
    v = qkv[:, (nq + nkv) * d:].reshape(T, nkv, d)
    half = d // 2
    freq = torch.pow(torch.tensor(shape.rope_theta, dtype=torch.float64),
                     -torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * freq[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def rope(u):
        z = torch.complex(u[..., :half], u[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                       v.transpose(0, 1)[None], is_causal=True,
                                       enable_gqa=True)[0].transpose(0, 1).reshape(T, nq * d)
    h = t(x) + F.linear(o, t(w["w_o"]))
    hn = F.rms_norm(h, (H,), t(w["g_ffn"]), eps=shape.rms_eps)
    act = F.silu(F.linear(hn, t(w["w_gate"]))) * F.linear(hn, t(w["w_up"]))
    out = h + F.linear(act, t(w["w_down"]))
    return out.numpy(), k.reshape(T, nkv * d).numpy(), v.reshape(T, nkv * d).numpy()


def run_chunks(seq, n_calls, decodes=None):
    """Prefill ``seq`` chunk by chunk through the oracle; returns the
    stacked outputs, the final pages and the summed prior-KV reads."""
    w = oracle_weights(seq.weights)
    kv = widen(seq.kv_pages)
    outs, loads = [], 0
    for k in range(n_calls):
        c = seq.chunk(k)
        r = layer_forward(seq.shape, w, widen(seq.chunk_rows(k)),
                          [(c.length, c.start_pos, c.block_table)], [], [], kv)
        kv = r.kv_pages
        outs.append(r.out)
        loads += r.prior_loads
    return np.concatenate(outs), kv, loads


def test_dense_brute_force_single_prompt():
    seq = make_prompt_sequence(TINY, 40, 1, seed=11, random_gains=True)
    w = oracle_weights(seq.weights)
    out, kv, _ = run_chunks(seq, 1)
    ref, k_ref, v_ref = dense_layer_torch(TINY, w, widen(seq.x_prompt))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())
    # the cached K (rotated) and V of every position
    P = TINY.page_size
    for pos in range(40):
        page, off = divmod(slot_of(pos, seq.block_table, P), P)
        np.testing.assert_allclose(kv[page, 0, :, off].reshape(-1), k_ref[pos], rtol=1e-10,
                                   atol=1e-12)
        np.testing.assert_allclose(kv[page, 1, :, off].reshape(-1), v_ref[pos], rtol=1e-10,
                                   atol=1e-12)


def test_dense_brute_force_gqa_group8():
    shape = LayerShape(128, 8, 1, 32, 256)
    seq = make_prompt_sequence(shape, 24, 1, seed=12, random_gains=True, weight_std=0.1)
    out, _, _ = run_chunks(seq, 1)
    ref, _, _ = dense_layer_torch(shape, oracle_weights(seq.weights), widen(seq.x_prompt))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


@pytest.mark.parametrize("n_chunks", [2, 4, 8])
def test_chunked_equals_unchunked(n_chunks):
    seq = make_prompt_sequence(TINY, 128, n_chunks, seed=13, random_gains=True)
    whole = make_prompt_sequence(TINY, 128, 1, seed=13, random_gains=True)
    out_c, kv_c, _ = run_chunks(seq, n_chunks)
    out_1, kv_1, _ = run_chunks(whole, 1)
    scale = np.abs(out_1).max()
    np.testing.assert_allclose(out_c, out_1, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(kv_c, kv_1, rtol=0, atol=1e-12, equal_nan=True)


@pytest.mark.parametrize("n_chunks", [1, 2, 4, 8, 16])
def test_prior_kv_reads_match_closed_form(n_chunks):
    seq = make_prompt_sequence(TINY, 128, n_chunks, seed=14)
    _, _, loads = run_chunks(seq, n_chunks)
    C = 128 // n_chunks
    assert loads == prefix_reread_loads(C, n_chunks, TINY.n_kv_heads)
    # sum over chunks of the chunks before each one
    assert loads == C * TINY.n_kv_heads * sum(k - 1 for k in range(1, n_chunks + 1))


def test_closed_form_values():
    # N(N-1)/2 for N = 1..6, and the Mistral-shaped 2048-token prompt in bytes
    assert [prefix_reread_loads(1, n, 1) for n in range(1, 7)] == [0, 1, 3, 6, 10, 15]
    kvB_per_head = 2 * 128 * 2
    mb = [prefix_reread_loads(2048 // n, n, 8) * kvB_per_head / 2 ** 20 for n in (1, 2, 4, 8, 16)]
    np.testing.assert_allclose(mb, [0, 4.0, 12.0, 28.0, 60.0])


def test_hybrid_equals_each_request_alone():
    hb = tiny_batch(seed=15)
    r = layer_forward(*oracle_args(hb))
    shape, w, x, chunks, ctx, bts, kv0 = oracle_args(hb)
    Lp = hb.chunks[0].length
    alone = layer_forward(shape, w, x[:Lp], chunks, [], [], kv0)
    scale = np.abs(r.out).max()
    np.testing.assert_allclose(r.out[:Lp], alone.out, rtol=0, atol=1e-12 * scale)
    kv_union = alone.kv_pages
    for j in range(len(ctx)):
        one = layer_forward(shape, w, x[Lp + j:Lp + j + 1], [], [ctx[j]], bts[j:j + 1], kv0)
        np.testing.assert_allclose(r.out[Lp + j], one.out[0], rtol=0, atol=1e-12 * scale)
        changed = ~np.isclose(one.kv_pages, kv0, rtol=0, atol=0, equal_nan=True)
        kv_union = np.where(changed, one.kv_pages, kv_union)
    np.testing.assert_allclose(r.kv_pages, kv_union, rtol=0, atol=1e-12, equal_nan=True)


def test_decode_equals_last_row_of_prefill():
    seq = make_prompt_sequence(TINY, 33, 1, seed=16, random_gains=True)
    w = oracle_weights(seq.weights)
    x = widen(seq.x_prompt)
    kv = widen(seq.kv_pages)
    full = layer_forward(TINY, w, x, [(33, 0, seq.block_table)], [], [], kv)
    pre = layer_forward(TINY, w, x[:32], [(32, 0, seq.block_table)], [], [], kv)
    dec = layer_forward(TINY, w, x[32:], [], [32], [seq.block_table], pre.kv_pages)
    np.testing.assert_allclose(dec.out[0], full.out[32], rtol=0,
                               atol=1e-12 * np.abs(full.out).max())
    np.testing.assert_allclose(dec.kv_pages, full.kv_pages, rtol=0, atol=1e-12, equal_nan=True)


def test_decode_with_empty_context_returns_own_value():
    # ctx = 0: the token attends only to itself, so attention returns its v
    hb = make_hybrid_batch(TINY, chunk_lens=[], chunk_starts=[], ctx_lens=[0, 0, 5], seed=17,
                           random_gains=True)
    r = layer_forward(*oracle_args(hb))
    G = TINY.n_q_heads // TINY.n_kv_heads
    d = TINY.head_dim
    for row in range(2):
        v = r.taps["v"][row].reshape(TINY.n_kv_heads, d)
        a = r.taps["attn"][row].reshape(TINY.n_q_heads, d)
        for h in range(TINY.n_q_heads):
            np.testing.assert_allclose(a[h], v[h // G], rtol=1e-14)


def test_only_expected_slots_change():
    hb = tiny_batch(seed=18)
    args = oracle_args(hb)
    r = layer_forward(*args)
    kv0 = args[-1]
    P = TINY.page_size
    # brute-force list of the slots this batch appends to
    expect = []
    for c in hb.chunks:
        expect += [slot_of(c.start_pos + i, c.block_table, P) for i in range(c.length)]
    for j, c in enumerate(hb.decodes.ctx_lens):
        expect.append(slot_of(int(c), hb.decodes.block_tables[j], P))
    np.testing.assert_array_equal(r.slots, expect)
    assert len(set(expect)) == len(expect)
    flat_old = kv0.transpose(0, 3, 1, 2, 4).reshape(-1, 2 * TINY.n_kv_heads * TINY.head_dim)
    flat_new = r.kv_pages.transpose(0, 3, 1, 2, 4).reshape(flat_old.shape)
    same = np.all((flat_old == flat_new) | (np.isnan(flat_old) & np.isnan(flat_new)), axis=1)
    assert sorted(np.nonzero(~same)[0].tolist()) == sorted(expect)

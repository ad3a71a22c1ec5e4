"""Pins of the oracle's building blocks against closed forms, special cases
and independent library routines (CPU only)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention_row, rmsnorm, rope_rotate, silu, slot_of, swiglu_ffn


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_hand_values():
    # row (3, 4): mean of squares 12.5, root 3.5355339059; eps 0, unit gain
    out = rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    np.testing.assert_allclose(out, [[0.848528137423857, 1.131370849898476]], rtol=1e-14)
    # constant-magnitude row maps to +-g exactly (eps 0)
    out = rmsnorm(np.array([[2.0, -2.0, 2.0, -2.0]]), np.array([1.0, 2.0, 3.0, 4.0]), 0.0)
    np.testing.assert_allclose(out, [[1.0, -2.0, 3.0, -4.0]], rtol=1e-15)


def test_rmsnorm_eps_inside_root():
    # all-ones row: mean square 1, so the output is g / sqrt(1 + eps)
    eps = 0.25
    out = rmsnorm(np.ones((1, 8)), np.full(8, 3.0), eps)
    np.testing.assert_allclose(out, np.full((1, 8), 3.0 / math.sqrt(1.25)), rtol=1e-15)


def test_rmsnorm_properties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    g = np.ones(64)
    y = rmsnorm(x, g, 1e-12)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-9)
    np.testing.assert_allclose(rmsnorm(7.5 * x, g, 1e-12), y, rtol=1e-9)


def test_rmsnorm_vs_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 96))
    g = rng.uniform(0.5, 1.5, 96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(rmsnorm(x, g, 1e-5), ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    u = np.random.default_rng(3).standard_normal(64)
    np.testing.assert_array_equal(rope_rotate(u, 0, 1e4), u)


def test_rope_hand_values():
    # d = 4, theta = 1e4: pair (0, 2) turns at 1 rad per position, pair (1, 3)
    # at theta^(-1/2) = 0.01 rad per position.
    out = rope_rotate(np.array([1.0, 0.0, 0.0, 0.0]), 1, 1e4)
    np.testing.assert_allclose(out, [math.cos(1), 0, math.sin(1), 0], atol=1e-15)
    out = rope_rotate(np.array([0.0, 1.0, 0.0, 0.0]), 100, 1e4)
    np.testing.assert_allclose(out, [0, math.cos(1), 0, math.sin(1)], atol=1e-12)
    # second element of a pair: (0, b) -> (-b sin, b cos)
    out = rope_rotate(np.array([0.0, 0.0, 2.0, 0.0]), 1, 1e4)
    np.testing.assert_allclose(out, [-2 * math.sin(1), 0, 2 * math.cos(1), 0], atol=1e-15)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    r = rope_rotate(q, 777, 1e4)
    # each pair keeps its length
    np.testing.assert_allclose(np.hypot(r[:64], r[64:]), np.hypot(q[:64], q[64:]), rtol=1e-12)
    # the score depends only on the position difference
    s1 = rope_rotate(q, 50, 1e4) @ rope_rotate(k, 20, 1e4)
    s2 = rope_rotate(q, 1030, 1e4) @ rope_rotate(k, 1000, 1e4)
    assert abs(s1 - s2) < 1e-9 * abs(s1) + 1e-12


def test_rope_vs_complex_multiplication():
    # the same rotation written as complex numbers a + ib times e^{i angle}
    rng = np.random.default_rng(5)
    u = rng.standard_normal(64)
    pos, theta = 333, 1e4
    half = 32
    z = torch.complex(torch.from_numpy(u[:half]), torch.from_numpy(u[half:]))
    freq = torch.pow(torch.tensor(theta, dtype=torch.float64),
                     -torch.arange(0, 64, 2, dtype=torch.float64) / 64)
    rot = z * torch.polar(torch.ones(half, dtype=torch.float64), pos * freq)
    ref = torch.cat([rot.real, rot.imag]).numpy()
    np.testing.assert_allclose(rope_rotate(u, pos, theta), ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- SiLU / FFN
def test_silu_values():
    assert silu(np.array(0.0)) == 0.0
    np.testing.assert_allclose(silu(np.array([50.0])), [50.0], rtol=1e-15)
    assert abs(silu(np.array(-50.0))) < 1e-19
    # silu(1) = 1 / (1 + e^-1)
    np.testing.assert_allclose(silu(np.array(1.0)), 0.7310585786300049, rtol=1e-15)
    z = np.random.default_rng(6).standard_normal(100) * 4
    np.testing.assert_allclose(silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13)


def test_swiglu_ffn_vs_torch():
    rng = np.random.default_rng(7)
    hn = rng.standard_normal((3, 16))
    wg, wu, wd = (rng.standard_normal((40, 16)), rng.standard_normal((40, 16)),
                  rng.standard_normal((16, 40)))
    act, y = swiglu_ffn(hn, wg, wu, wd)
    t = lambda a: torch.from_numpy(a)
    ref_act = F.silu(F.linear(t(hn), t(wg))) * F.linear(t(hn), t(wu))
    np.testing.assert_allclose(act, ref_act.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, F.linear(ref_act, t(wd)).numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- attention
def test_attention_special_cases():
    rng = np.random.default_rng(8)
    v = rng.standard_normal((7, 8))
    q = rng.standard_normal(8)
    same_keys = np.tile(rng.standard_normal(8), (7, 1))
    np.testing.assert_allclose(attention_row(q, same_keys, v), v.mean(axis=0), rtol=1e-13)
    # a single key returns its value exactly
    np.testing.assert_array_equal(attention_row(q, same_keys[:1], v[:1]), v[0])


def test_attention_vs_sdpa():
    rng = np.random.default_rng(9)
    q = rng.standard_normal(64)
    K = rng.standard_normal((50, 64))
    V = rng.standard_normal((50, 64))
    t = lambda a: torch.from_numpy(a)
    ref = F.scaled_dot_product_attention(t(q)[None, None, None], t(K)[None, None],
                                         t(V)[None, None])[0, 0, 0].numpy()
    np.testing.assert_allclose(attention_row(q, K, V), ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- addressing
def test_slot_of_brute_force():
    rng = np.random.default_rng(10)
    P = 16
    perm = rng.permutation(40)
    bt = perm[:10]
    # enumerate the request's slots page by page, in order
    enumerated = [int(p) * P + o for p in bt for o in range(P)]
    for pos in range(160):
        assert slot_of(pos, bt, P) == enumerated[pos]


def test_attention_large_scores_stay_finite():
    # scores in the hundreds: the softmax must shift by the maximum score
    q = np.full(16, 12.0)
    K = np.stack([np.full(16, 30.0), np.full(16, -30.0), np.full(16, 29.0)])
    V = np.eye(3, 16)
    o = attention_row(q, K, V)
    assert np.all(np.isfinite(o))
    # score gap between key 0 and key 2 is 12*16/4 = 48: key 0 takes ~all weight
    np.testing.assert_allclose(o[:3], [1.0, 0.0, math.exp(-48.0)], rtol=1e-9, atol=1e-300)

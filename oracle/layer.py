"""Float64 oracle of one decoder-layer forward over a hybrid batch.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* A hybrid batch stacks the rows of one (or more) prefill chunks and the
  single new token of each piggybacked decode into one ``[Lp+Bd, H]`` matrix;
  the linear layers run once on the stacked matrix, attention is split by
  request (SARATHI paper summary on gitcode.csdn.net, part 2 item 3, the
  "merge / split / merge" operator scheduling; intelliparadigm.com article
  section 3.3).
* A chunk's tokens attend to every earlier token of the prompt, the KV of
  earlier chunks included, and causally within the chunk (intelliparadigm.com
  section 3.1; Sarathi-Serve digest section 2 Q2 item 1).
* Positions continue across chunks: every chunk keeps its own position ids
  (intelliparadigm.com section 6.1).
* Decodes read their history from paged KV (PagedAttention,
  intelliparadigm.com section 3.3).
* The pages give no layer internals beyond "LayerNorm" (intelliparadigm.com
  section 6.1) and "decoder-only transformer, GQA" (Sarathi-Serve digest,
  appendix Table 1).  The layer shape taken here is the usual pre-norm GQA
  block with RMSNorm, rotary position embedding and a SwiGLU FFN, as the
  workload description names them.

Readings where the pages are silent (each one is a choice, not a fact of
the pages):

* RMSNorm: ``x / sqrt(mean(x^2) + eps) * g`` (eps inside the root, gain
  after the normalisation).
* RoPE: "rotate-half" pairing of element ``i`` with ``i + d/2``, angle
  ``pos * theta^(-2i/d)``; applied to q and k, not v; K is cached after the
  rotation.
* A decode whose request has ``c`` cached tokens sits at position ``c``,
  appends its own K/V there, and attends ``c + 1`` keys.
* q head ``h`` reads kv head ``h // (n_q_heads / n_kv_heads)``; scores are
  scaled by ``1/sqrt(head_dim)``; full causal masking, no sliding window.
* Every K/V append of the batch happens before any attention read.

Parity status: every function here is pinned by the CPU tests (closed forms,
special cases reducing to library routines, invariants the pages fix); the
absolute choice of RoPE pairing and norm placement is a reading, so those
two are "parity unpinned" as choices, while their arithmetic is pinned.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np


# ------------------------------------------------------------------ pieces
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMS normalisation with gain: ``x / sqrt(mean(x^2) + eps) * g``."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope_rotate(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate one head vector ``u`` (length d) to position ``pos``.

    Element i (i < d/2) pairs with element i + d/2; the pair turns by the
    angle ``pos * theta**(-2 i / d)``.
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    angle = float(pos) * np.power(float(theta), -2.0 * i / d)
    c, s = np.cos(angle), np.sin(angle)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """``z * sigmoid(z)`` written as ``z / (1 + exp(-z))``."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(hn: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
               w_down: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """``act = silu(hn W_gate^T) * (hn W_up^T)``; returns ``(act, act W_down^T)``."""
    act = silu(hn @ w_gate.T) * (hn @ w_up.T)
    return act, act @ w_down.T


def slot_of(pos: int, block_table: Sequence[int], page_size: int) -> int:
    """PagedAttention addressing: the token at position ``pos`` of a request
    lives in page ``block_table[pos // page_size]`` at offset
    ``pos % page_size``; its flat slot number is ``page * page_size + offset``."""
    return int(block_table[pos // page_size]) * page_size + pos % page_size


def attention_row(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Softmax attention of one query over ``keys``/``values`` ([T, d]).

    Scores ``q.k / sqrt(d)``; the softmax subtracts the maximum score before
    exponentiating.
    """
    d = q.shape[-1]
    s = keys @ q / math.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ values


def gather_request_kv(kv: np.ndarray, block_table: Sequence[int], n_tokens: int,
                      page_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Contiguous K and V ([n_kv, n_tokens, d]) of a request's first
    ``n_tokens`` positions, read through its block table."""
    t = np.arange(n_tokens)
    pages = np.asarray(block_table, dtype=np.int64)[t // page_size]
    offs = t % page_size
    K = kv[pages, 0, :, offs]          # [n_tokens, n_kv, d]
    V = kv[pages, 1, :, offs]
    return K.transpose(1, 0, 2), V.transpose(1, 0, 2)


def prefix_reread_loads(chunk_len: int, n_chunks: int, n_kv_heads: int) -> int:
    """Closed form of the chunked-prefill KV re-read (Sarathi-Serve digest,
    section 4, check 4): chunk k of N (1-based) reloads the KV of the k-1
    earlier chunks, so the whole prompt reloads chunk KV sum_{k=1}^{N}(k-1)
    = N(N-1)/2 times; in (token, kv head) loads that is
    ``chunk_len * N(N-1)/2 * n_kv_heads``."""
    return chunk_len * n_chunks * (n_chunks - 1) // 2 * n_kv_heads


# ------------------------------------------------------------------ layer
@dataclass
class OracleResult:
    out: np.ndarray            # [M, H]
    kv_pages: np.ndarray       # updated copy, float64
    slots: np.ndarray          # int64 [M]
    positions: np.ndarray      # int64 [M]
    taps: Dict[str, np.ndarray] = field(default_factory=dict)
    # distinct (token, kv head) pairs read from before each chunk's first
    # position, summed over the chunks of the call
    prior_loads: int = 0


def _row_requests(chunks, ctx_lens, block_tables, page_size):
    """(position, block_table, chunk_start) for each row, chunk rows first."""
    rows = []
    for (length, start, bt) in chunks:
        for i in range(length):
            rows.append((start + i, bt, start))
    for j, c in enumerate(ctx_lens):
        rows.append((int(c), block_tables[j], int(c)))
    return rows


def layer_forward(shape, w: Dict[str, np.ndarray], x: np.ndarray,
                  chunks: Sequence[Tuple[int, int, Sequence[int]]],
                  ctx_lens: Sequence[int], block_tables: Sequence[Sequence[int]],
                  kv_pages: np.ndarray) -> OracleResult:
    """One decoder-layer forward over a hybrid batch.

    ``shape`` has fields hidden, n_q_heads, n_kv_heads, head_dim, ffn,
    page_size, rms_eps, rope_theta.  ``w`` maps w_qkv [(nq+2nkv)d, H], w_o
    [H, nq d], w_gate/w_up [F, H], w_down [H, F], g_attn/g_ffn [H] to float
    arrays.  ``chunks`` lists (length, start_pos, block_table); decode j has
    ``ctx_lens[j]`` cached tokens and block table ``block_tables[j]``.
    ``kv_pages`` is [num_pages, 2, n_kv, page_size, head_dim]; a copy is
    updated and returned.

    Steps, in order: row positions and KV slots; RMSNorm; the fused QKV
    projection on the stacked rows; RoPE on q and k; append K/V of every
    row; attention of every row over its request's keys 0..pos; O
    projection plus residual; RMSNorm; SwiGLU FFN plus residual.
    """
    H, nq, nkv, d = shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    P = shape.page_size
    G = nq // nkv
    x = np.asarray(x, dtype=np.float64)
    M = x.shape[0]
    kv = np.array(kv_pages, dtype=np.float64, copy=True)

    rows = _row_requests(chunks, ctx_lens, block_tables, P)
    assert len(rows) == M, "x must have one row per chunk token and per decode"
    positions = np.array([r[0] for r in rows], dtype=np.int64)
    slots = np.array([slot_of(r[0], r[1], P) for r in rows], dtype=np.int64)

    # RMSNorm before attention
    xn1 = rmsnorm(x, w["g_attn"], shape.rms_eps)

    # fused QKV projection on the stacked rows
    qkv = xn1 @ np.asarray(w["w_qkv"], dtype=np.float64).T
    q = qkv[:, :nq * d].reshape(M, nq, d)
    k = qkv[:, nq * d:(nq + nkv) * d].reshape(M, nkv, d)
    v = qkv[:, (nq + nkv) * d:].reshape(M, nkv, d)

    # RoPE at each row's own position
    q = np.stack([np.stack([rope_rotate(q[r, h], positions[r], shape.rope_theta)
                            for h in range(nq)]) for r in range(M)]) if M else q
    k = np.stack([np.stack([rope_rotate(k[r, g], positions[r], shape.rope_theta)
                            for g in range(nkv)]) for r in range(M)]) if M else k

    # append K (rotated) and V of every row before any attention
    for r in range(M):
        page, off = divmod(int(slots[r]), P)
        kv[page, 0, :, off] = k[r]
        kv[page, 1, :, off] = v[r]

    # attention: each row over keys 0..pos of its own request
    attn = np.zeros((M, nq, d))
    # per chunk: which (token, kv head) pairs before the chunk's first
    # position were read by any of its rows
    prior_read = [np.zeros((start, nkv), dtype=bool) for (_, start, _) in chunks]
    chunk_of_row = [ci for ci, (length, _, _) in enumerate(chunks) for _ in range(length)]
    for r, (pos, bt, start) in enumerate(rows):
        K, V = gather_request_kv(kv, bt, pos + 1, P)
        for h in range(nq):
            g = h // G
            attn[r, h] = attention_row(q[r, h], K[g], V[g])
            if r < len(chunk_of_row) and start > 0:
                prior_read[chunk_of_row[r]][:min(pos + 1, start), g] = True
    prior_loads = int(sum(m.sum() for m in prior_read))

    attn2 = attn.reshape(M, nq * d)
    h_res = x + attn2 @ np.asarray(w["w_o"], dtype=np.float64).T

    # RMSNorm before the FFN, then SwiGLU FFN with residual
    xn2 = rmsnorm(h_res, w["g_ffn"], shape.rms_eps)
    act, ffn = swiglu_ffn(xn2, np.asarray(w["w_gate"], dtype=np.float64),
                          np.asarray(w["w_up"], dtype=np.float64),
                          np.asarray(w["w_down"], dtype=np.float64))
    out = h_res + ffn

    taps = {
        "xn1": xn1,
        "q": q.reshape(M, nq * d),
        "k": k.reshape(M, nkv * d),
        "v": v.reshape(M, nkv * d),
        "attn": attn2,
        "h": h_res,
        "xn2": xn2,
        "act": act,
    }
    return OracleResult(out, kv, slots, positions, taps, prior_loads)

"""Seeded synthetic inputs for one hybrid-batch decoder-layer call.

This module only draws numbers and lays them out; it holds none of the
layer's arithmetic.  Both the CPU oracle (through the tests) and the HIP
library consume exactly the arrays produced here, so bf16 values are
handed over as raw ``uint16`` bit patterns.

Workload shapes follow the pages:

* the hybrid batch is one prefill chunk of ``Lp`` tokens followed by ``Bd``
  decode tokens, stacked into a ``[Lp+Bd, H]`` activation matrix
  (SARATHI paper summary, gitcode.csdn.net, part 2 "underlying operator
  scheduling": linear layers on the concatenated matrix);
* a long prompt is cut into fixed-size chunks computed over several calls,
  each chunk attending to the KV of the earlier ones (intelliparadigm.com
  article, section 3.1; Sarathi-Serve digest, section 2 Q2 item 1);
* the KV cache is paged, 16 tokens per page, one block table per request
  (PagedAttention for the decodes, intelliparadigm.com section 3.3).

Drawing order for one layer (fixed, so every consumer sees the same bytes):
W_qkv, W_o, W_gate, W_up, W_down, g_attn, g_ffn, x, decode context lengths,
page permutation, pre-existing KV values.  Normal draws are fp32 from
``numpy.random.default_rng(seed)`` (PCG64) rounded to bf16 with
round-to-nearest-even.  "N(0, s)" means standard deviation ``s``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

PAGE_SIZE = 16
# bf16 quiet-NaN with a payload: fills every KV slot that holds no token, so
# a stray read or write of such a slot shows up in a comparison.
SENTINEL_BF16 = np.uint16(0x7FA5)


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    page_size: int = PAGE_SIZE
    rms_eps: float = 1e-5
    rope_theta: float = 1e4

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def kv_bytes_per_token(self) -> int:
        """K and V of one token for every kv head, bf16."""
        return 2 * self.n_kv_heads * self.head_dim * 2


# Tiny layer: H=256, 4 q heads / 2 kv heads, head_dim 64, SwiGLU FFN 1024.
TINY = LayerShape(256, 4, 2, 64, 1024)
# Mistral-7B-shaped layer: H=4096, 32 q / 8 kv heads, head_dim 128, FFN 14336.
MISTRAL_7B = LayerShape(4096, 32, 8, 128, 14336)
# Llama-2-70B-shaped layer: H=8192, 64 q / 8 kv heads, head_dim 128, FFN 28672.
LLAMA2_70B = LayerShape(8192, 64, 8, 128, 28672)
# One GPU's share of a tensor-parallel layer (heads and FFN columns split T
# ways, hidden size whole): the per-GPU kernel shapes of Llama-2-70B at T = 8
# and Mistral-7B at T = 4.
LLAMA2_70B_TP8 = LayerShape(8192, 8, 1, 128, 3584)
MISTRAL_7B_TP4 = LayerShape(4096, 8, 2, 128, 3584)


# ---------------------------------------------------------------- bf16 bits
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the bits."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- containers
@dataclass
class Weights:
    """Layer weights as bf16 bits, every matrix ``[out, in]`` row-major.

    ``w_qkv`` stacks the q heads, then the k heads, then the v heads, each
    head's ``head_dim`` rows contiguous.
    """
    w_qkv: np.ndarray
    w_o: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    g_attn: np.ndarray
    g_ffn: np.ndarray

    def as_dict(self):
        return {k: getattr(self, k) for k in
                ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")}

    @property
    def nbytes(self) -> int:
        return sum(v.nbytes for v in self.as_dict().values())


@dataclass
class Chunk:
    """One prefill chunk: ``length`` rows at positions start_pos .. start_pos+length-1."""
    length: int
    start_pos: int
    block_table: np.ndarray  # int32 [n_blocks], covers positions [0, start_pos+length)


@dataclass
class Decodes:
    """Piggybacked decode tokens, one per request.

    Decode j has ``ctx_lens[j]`` tokens cached; its new token sits at
    position ``ctx_lens[j]`` and attends ``ctx_lens[j] + 1`` keys.
    """
    ctx_lens: np.ndarray      # int32 [Bd]
    block_tables: np.ndarray  # int32 [Bd, max_blocks]; unused entries 0

    @property
    def n(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1]) if self.block_tables.ndim == 2 else 0

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_lens.max()) if self.n else 0


@dataclass
class HybridBatch:
    shape: LayerShape
    weights: Weights
    x: np.ndarray             # bf16 bits [M, H]; chunk rows first, then decode rows
    chunks: List[Chunk]
    decodes: Decodes
    kv_pages: np.ndarray      # bf16 bits [num_pages, 2, n_kv, page_size, head_dim]

    @property
    def n_rows(self) -> int:
        return int(self.x.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.kv_pages.shape[0])

    @property
    def n_chunk_rows(self) -> int:
        return sum(c.length for c in self.chunks)


# ---------------------------------------------------------------- drawing
def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_bits(a)


def draw_weights(rng: np.random.Generator, shape: LayerShape, std: float,
                 random_gains: bool) -> Weights:
    H, F = shape.hidden, shape.ffn
    nqd = shape.n_q_heads * shape.head_dim
    w_qkv = _normal_bf16(rng, (shape.qkv_rows, H), std)
    w_o = _normal_bf16(rng, (H, nqd), std)
    w_gate = _normal_bf16(rng, (F, H), std)
    w_up = _normal_bf16(rng, (F, H), std)
    w_down = _normal_bf16(rng, (H, F), std)
    if random_gains:
        g_attn = bf16_bits(rng.uniform(0.5, 1.5, size=H).astype(np.float32))
        g_ffn = bf16_bits(rng.uniform(0.5, 1.5, size=H).astype(np.float32))
    else:
        g_attn = bf16_bits(np.ones(H, np.float32))
        g_ffn = bf16_bits(np.ones(H, np.float32))
    return Weights(w_qkv, w_o, w_gate, w_up, w_down, g_attn, g_ffn)


def pages_for(n_tokens: int, page_size: int = PAGE_SIZE) -> int:
    return -(-n_tokens // page_size)


def make_hybrid_batch(shape: LayerShape, *, chunk_lens: Sequence[int],
                      chunk_starts: Sequence[int], ctx_lens: Optional[Sequence[int]] = None,
                      n_decodes: int = 0, ctx_range=(16, 128), seed: int = 0,
                      weight_std: float = 0.02, random_gains: bool = False,
                      weights: Optional[Weights] = None, spare_frac: float = 0.25,
                      prior_kv: str = "random") -> HybridBatch:
    """Draw one hybrid batch.

    ``chunk_lens``/``chunk_starts`` give each chunk's ``Lp`` and the position
    of its first token (tokens before it are already cached).  Decode
    contexts are either given or drawn uniformly from the inclusive integer
    range ``ctx_range``.  The page pool holds ``ceil((1+spare_frac) *
    needed)`` pages, handed out by one seeded permutation in request order
    (chunks first, then decodes); spare pages and every slot without a
    cached token hold the sentinel.  With ``prior_kv="random"`` the cached
    tokens' K and V are N(0, 1) bf16.
    """
    rng = np.random.default_rng(seed)
    P = shape.page_size
    if weights is None:
        weights = draw_weights(rng, shape, weight_std, random_gains)
    n_chunk_rows = int(sum(chunk_lens))
    if ctx_lens is None:
        ctx = rng.integers(ctx_range[0], ctx_range[1], size=n_decodes, endpoint=True)
    else:
        ctx = np.asarray(ctx_lens, dtype=np.int64)
        n_decodes = int(ctx.shape[0])
    M = n_chunk_rows + n_decodes
    x = _normal_bf16(rng, (M, shape.hidden), 1.0)

    need_chunk = [pages_for(s + l, P) for l, s in zip(chunk_lens, chunk_starts)]
    need_dec = [pages_for(int(c) + 1, P) for c in ctx]
    needed = sum(need_chunk) + sum(need_dec)
    num_pages = max(1, int(math.ceil((1.0 + spare_frac) * needed)))
    perm = rng.permutation(num_pages).astype(np.int32)

    chunks: List[Chunk] = []
    cursor = 0
    for l, s, nb in zip(chunk_lens, chunk_starts, need_chunk):
        chunks.append(Chunk(int(l), int(s), perm[cursor:cursor + nb].copy()))
        cursor += nb
    max_blocks = max(need_dec) if need_dec else 0
    bts = np.zeros((n_decodes, max_blocks), dtype=np.int32)
    for j, nb in enumerate(need_dec):
        bts[j, :nb] = perm[cursor:cursor + nb]
        cursor += nb
    decodes = Decodes(ctx.astype(np.int32), bts)

    kv = np.full((num_pages, 2, shape.n_kv_heads, P, shape.head_dim), SENTINEL_BF16,
                 dtype=np.uint16)
    if prior_kv == "random":
        # cached tokens of every request, in request order
        for c in chunks:
            _fill_cached(rng, kv, c.block_table, c.start_pos, P)
        for j in range(n_decodes):
            _fill_cached(rng, kv, bts[j], int(ctx[j]), P)
    elif prior_kv != "none":
        raise ValueError(prior_kv)

    return HybridBatch(shape, weights, x, chunks, decodes, kv)


def _fill_cached(rng, kv, block_table, n_cached, P):
    if n_cached <= 0:
        return
    n_kv, d = kv.shape[2], kv.shape[4]
    vals = _normal_bf16(rng, (n_cached, 2, n_kv, d), 1.0)
    for t in range(n_cached):
        page = block_table[t // P]
        kv[page, :, :, t % P, :] = vals[t]


# ---------------------------------------------------------------- presets
def tiny_batch(seed: int = 0, random_gains: bool = True) -> HybridBatch:
    """Tiny layer: chunk 2 of a 128-token prompt (Lp=64 after 64 cached
    tokens) plus 4 decodes with contexts drawn from U{16..128}."""
    return make_hybrid_batch(TINY, chunk_lens=[64], chunk_starts=[64], n_decodes=4,
                             ctx_range=(16, 128), seed=seed, weight_std=0.02,
                             random_gains=random_gains)


def mistral_batch(seed: int = 0, random_gains: bool = False, **kw) -> HybridBatch:
    """Mistral-7B-shaped layer: chunk 4 of a 1024-token prompt (Lp=256 after
    768 cached tokens) plus 32 decodes with contexts from U{128..2048}."""
    args = dict(chunk_lens=[256], chunk_starts=[768], n_decodes=32, ctx_range=(128, 2048),
                seed=seed, weight_std=0.02, random_gains=random_gains)
    args.update(kw)
    return make_hybrid_batch(MISTRAL_7B, **args)


def llama70_batch(seed: int = 0, random_gains: bool = False, **kw) -> HybridBatch:
    """Llama-2-70B-shaped layer: the last 512-token chunk of a 4096-token
    prompt (3584 cached) plus 64 decodes with contexts from U{512..4096}."""
    args = dict(chunk_lens=[512], chunk_starts=[3584], n_decodes=64, ctx_range=(512, 4096),
                seed=seed, weight_std=0.01, random_gains=random_gains)
    args.update(kw)
    return make_hybrid_batch(LLAMA2_70B, **args)


def llama70_tp8_batch(seed: int = 0, random_gains: bool = False, **kw) -> HybridBatch:
    """The Llama-2-70B batch on one GPU's tensor-parallel share (T = 8)."""
    args = dict(chunk_lens=[512], chunk_starts=[3584], n_decodes=64, ctx_range=(512, 4096),
                seed=seed, weight_std=0.01, random_gains=random_gains)
    args.update(kw)
    return make_hybrid_batch(LLAMA2_70B_TP8, **args)


def mistral_tp4_batch(seed: int = 0, random_gains: bool = False, **kw) -> HybridBatch:
    """The Mistral-7B batch on one GPU's tensor-parallel share (T = 4)."""
    args = dict(chunk_lens=[256], chunk_starts=[768], n_decodes=32, ctx_range=(128, 2048),
                seed=seed, weight_std=0.02, random_gains=random_gains)
    args.update(kw)
    return make_hybrid_batch(MISTRAL_7B_TP4, **args)


def sweep_batch(lp: int, bd: int, seed: int = 0, **kw) -> HybridBatch:
    """Token-budget sweep point on the Mistral-7B shape: a fresh chunk
    (start_pos 0) of ``lp`` tokens plus ``bd`` decodes from U{128..4096}."""
    chunk_lens = [lp] if lp > 0 else []
    chunk_starts = [0] if lp > 0 else []
    args = dict(chunk_lens=chunk_lens, chunk_starts=chunk_starts, n_decodes=bd,
                ctx_range=(128, 4096), seed=seed, weight_std=0.02)
    args.update(kw)
    return make_hybrid_batch(MISTRAL_7B, **args)


@dataclass
class PromptSequence:
    """A prompt of ``prompt_len`` tokens to be prefilled in ``n_chunks``
    equal chunks over successive calls sharing one block table."""
    shape: LayerShape
    weights: Weights
    x_prompt: np.ndarray     # bf16 bits [prompt_len, H]
    block_table: np.ndarray  # int32 [pages_for(prompt_len)]
    kv_pages: np.ndarray     # bf16 bits, all sentinel
    chunk_len: int
    n_chunks: int

    def chunk(self, k: int) -> Chunk:
        """Chunk k (0-based) of the prompt."""
        return Chunk(self.chunk_len, k * self.chunk_len, self.block_table)

    def chunk_rows(self, k: int) -> np.ndarray:
        return self.x_prompt[k * self.chunk_len:(k + 1) * self.chunk_len]


def make_prompt_sequence(shape: LayerShape, prompt_len: int, n_chunks: int, seed: int = 0,
                         weight_std: float = 0.02, random_gains: bool = False,
                         spare_frac: float = 0.25) -> PromptSequence:
    if prompt_len % n_chunks:
        raise ValueError("prompt_len must split into equal chunks")
    rng = np.random.default_rng(seed)
    weights = draw_weights(rng, shape, weight_std, random_gains)
    x = _normal_bf16(rng, (prompt_len, shape.hidden), 1.0)
    need = pages_for(prompt_len, shape.page_size)
    num_pages = max(1, int(math.ceil((1.0 + spare_frac) * need)))
    perm = rng.permutation(num_pages).astype(np.int32)
    kv = np.full((num_pages, 2, shape.n_kv_heads, shape.page_size, shape.head_dim),
                 SENTINEL_BF16, dtype=np.uint16)
    return PromptSequence(shape, weights, x, perm[:need].copy(), kv,
                          prompt_len // n_chunks, n_chunks)


def empty_decodes() -> Decodes:
    return Decodes(np.zeros(0, np.int32), np.zeros((0, 0), np.int32))

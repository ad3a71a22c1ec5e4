"""Roofline cost model of one hybrid-batch layer call (host-side arithmetic).

The model is the pages' own: an operator's time is ``max(T_math, T_mem)``,
because a matmul kernel overlaps its memory traffic with its arithmetic, so
the slower of the two decides (Sarathi-Serve digest, section 4, roofline
equation; the worked example of the SARATHI summary on gitcode.csdn.net,
part 3, prices each batch the same way).  Kernels on one stream run back to
back, so a layer's time at roofline is the sum over its kernels.

Algorithmic work per operation (real rows only unless stated):

* GEMM ``[M,K] x [K,N]``: ``2*Mp*K*N`` flops (``Mp`` = rows after padding,
  what the hardware computes) and ``K*N*2 + M*K*2 + M*N*2`` bytes (weights
  read once, activations in and out once; residual GEMMs add ``M*N*2``).
* chunk-prefill attention: ``4*d*nq*(Lp*P0 + Lp*(Lp+1)/2)`` flops; bytes =
  K/V of all ``P0+Lp`` keys read once per kv head plus q in / out.
* decode attention: bytes ``sum_j (c_j+1) * kvB`` plus q in / out; flops
  ``4*d*nq*sum_j(c_j+1)``.
* RMSNorm, RoPE/append: bytes only.

MI355X figures used (vendor-published dense peaks): 2.5e15 bf16 flop/s,
8.0e12 B/s HBM3E.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Iterable, List, Sequence, Tuple

PEAK_BF16_FLOPS = 2.5e15
PEAK_HBM_BPS = 8.0e12
PEAK_FP32_VALU_FLOPS = 157.3e12


def roofline_time(t_math: float, t_mem: float) -> float:
    """Execution time of one operator under the roofline model."""
    return max(t_math, t_mem)


def schedule_time(batches: Iterable[Tuple[int, float, float]]) -> float:
    """Total time of a schedule given ``(count, t_math, t_mem)`` per batch kind."""
    return sum(n * roofline_time(tm, tb) for n, tm, tb in batches)


def tiles_needed(rows: int, tile: int) -> int:
    """Row tiles a GEMM must launch for ``rows`` rows: ``ceil(rows/tile)``."""
    return -(-rows // tile)


def round_up(n: int, m: int) -> int:
    return tiles_needed(n, m) * m


@dataclass
class Stage:
    name: str
    flops: float
    bytes: float
    bound: str = ""

    def t_math(self, peak_flops=PEAK_BF16_FLOPS) -> float:
        return self.flops / peak_flops

    def t_mem(self, peak_bw=PEAK_HBM_BPS) -> float:
        return self.bytes / peak_bw

    def t_roof(self) -> float:
        return roofline_time(self.t_math(), self.t_mem())


def layer_stages(hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ffn: int,
                 chunk_lens: Sequence[int], chunk_starts: Sequence[int],
                 ctx_lens: Sequence[int], pad: int = 16, chained: bool = False) -> List[Stage]:
    """Algorithmic flops and bytes of every kernel slot of one layer call, in
    the library's launch order and under its slot names.

    Each byte and flop of the layer is given to exactly one kernel: a GEMM's
    main kernel carries the whole projection (weights, activations in, result
    out, residual in); a split-K reduce carries only what its fused epilogue
    adds to the algorithm (the second RMSNorm's output and gain), so a plain
    reduce and the attention key-split merge carry none -- their time is
    overhead of the launch shape, not work of the layer.

    ``chained``: the call with the cross-layer RMSNorm fusion, whose first
    RMSNorm was formed by the previous layer and whose down-projection reduce
    forms the next layer's (the same work, one slot later)."""
    H, nq, nkv, d, F = hidden, n_q_heads, n_kv_heads, head_dim, ffn
    Lp = int(sum(chunk_lens))
    Bd = len(ctx_lens)
    M = Lp + Bd
    Mp = round_up(M, pad)
    nqkv = (nq + 2 * nkv) * d
    kvB = 2 * nkv * d * 2
    st: List[Stage] = []
    norm1 = (3 * M * H, 2 * M * H * 2 + H * 2)
    st.append(Stage("rmsnorm1", *((0.0, 0.0) if chained else norm1)))
    st.append(Stage("gemm_qkv", 2 * Mp * H * nqkv, H * nqkv * 2 + M * H * 2 + M * nqkv * 2))
    # RoPE + KV append (it also sums the QKV split-K partials: not algorithmic)
    st.append(Stage("rope_kv_append", 6 * M * (nq + nkv) * d,
                    M * nqkv * 2 + M * (nq + nkv) * d * 2 + M * kvB))
    pf_flops = 0.0
    pf_bytes = 0.0
    for L, P0 in zip(chunk_lens, chunk_starts):
        pf_flops += 4.0 * d * nq * (L * P0 + L * (L + 1) / 2)
        pf_bytes += (P0 + L) * kvB + 2 * L * nq * d * 2
    keys = sum(int(c) + 1 for c in ctx_lens)
    dc_flops = 4.0 * d * nq * keys
    dc_bytes = keys * kvB + 2 * Bd * nq * d * 2
    # prefill and decode rows run in one launch and overlap: priced together
    st.append(Stage("attention", pf_flops + dc_flops, pf_bytes + dc_bytes))
    st.append(Stage("attention_merge", 0.0, 0.0))
    # O projection + residual: weights, attn in, x in, h out
    st.append(Stage("gemm_o", 2 * Mp * nq * d * H, nq * d * H * 2 + M * nq * d * 2 + 2 * M * H * 2))
    # RMSNorm of h inside the reduce: xn2 out and the gain
    st.append(Stage("gemm_o_reduce_rmsnorm2", 3 * M * H, M * H * 2 + H * 2))
    st.append(Stage("gemm_gate_up", 2 * Mp * H * 2 * F, 2 * F * H * 2 + M * H * 2 + M * F * 2))
    st.append(Stage("gemm_gate_up_reduce", 0.0, 0.0))
    st.append(Stage("gemm_down", 2 * Mp * F * H, F * H * 2 + M * F * 2 + 2 * M * H * 2))
    # chained: the next layer's RMSNorm of out inside the reduce (xn_next out
    # and the gain; out itself is the down projection's)
    st.append(Stage("gemm_down_reduce", *((3 * M * H, M * H * 2 + H * 2) if chained else (0.0, 0.0))))
    for s in st:
        s.bound = "mfma" if s.t_math() > s.t_mem() else "hbm"
    return st


def layer_roofline_time(stages: Sequence[Stage]) -> float:
    return sum(s.t_roof() for s in stages)


def stage_table(stages: Sequence[Stage]) -> Dict[str, Dict[str, float]]:
    return {s.name: {"flops": s.flops, "bytes": s.bytes, "t_roof_us": s.t_roof() * 1e6,
                     "bound": s.bound} for s in stages}

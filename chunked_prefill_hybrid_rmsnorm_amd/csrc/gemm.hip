// bf16 MFMA GEMM for the linear layers of the hybrid batch:
//   C[m, n] = sum_k A[m, k] * W[n, k]      (A = activations, W = [out, in] weights)
// run once on the stacked chunk + decode rows.
//
// Structure (gfx950, wave64):
//  * a workgroup owns a BM x BN output tile and walks its share of K in
//    steps of 64; A and W tiles are copied global -> LDS directly
//    (global_load_lds_dwordx4) into a ring of stages, several k-steps ahead
//    of the step being multiplied;
//  * each wave computes C^T = W A^T on a (BM/WM) x (BN/WN) sub-tile with
//    v_mfma_f32_16x16x32_bf16, so a lane ends up holding four consecutive
//    output columns of one row (one 8-byte store);
//  * at these row counts the weights dominate the traffic, so a tile spans as
//    many rows as registers allow and the workgroups that share one weight
//    tile (different row tiles) are numbered to land on the same XCD
//    (workgroup ids are dealt round-robin over the 8 XCDs) and reuse it from
//    that XCD's L2;
//  * narrow outputs split K over several workgroups (fp32 partial tiles in
//    the workspace, summed in a fixed order by a second kernel, so results
//    are deterministic);
//  * epilogues: plain store (QKV), residual add (O and down projections),
//    SwiGLU (gate and up rows side by side in one tile, combined in
//    registers).
#include "gemm_impl.h"

namespace hl {

// ------------------------------------------------------------ split-K reduce
// The split count is a template parameter: every split's loads are issued
// before the first is waited for (a loop over a runtime count waits for each
// split in turn).  Splits are summed in split order.
template <int EPI, int SPLITS>
__global__ __launch_bounds__(256) void gemm_splitk_reduce(const float* __restrict__ part,
                                                          bf16* __restrict__ C,
                                                          const bf16* __restrict__ R, int M, int Mp,
                                                          int N) {
  const int n4 = N / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int mlim = EPI == EPI_RESIDUAL ? M : Mp;
  if (idx >= mlim * n4) return;
  const int m = idx / n4, n = (idx % n4) * 4;
  const size_t plane = (size_t)Mp * N;
  f32x4 pv[SPLITS];
#pragma unroll
  for (int z = 0; z < SPLITS; ++z)
    pv[z] = *reinterpret_cast<const f32x4*>(part + z * plane + (size_t)m * N + n);
  f32x4 v = pv[0];
#pragma unroll
  for (int z = 1; z < SPLITS; ++z) v += pv[z];
  if (EPI == EPI_RESIDUAL) {
    const u32x2 rr = ld8(R + (size_t)m * N + n);
    v[0] += __uint_as_float(rr[0] << 16);
    v[1] += __uint_as_float(rr[0] & 0xffff0000u);
    v[2] += __uint_as_float(rr[1] << 16);
    v[3] += __uint_as_float(rr[1] & 0xffff0000u);
  }
  u32x2 o;
  o[0] = pack2(v[0], v[1]);
  o[1] = pack2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(C + (size_t)m * N + n) = o;
}

// Split-K reduce of the gate/up GEMM: act = silu(sum gate) * (sum up) over
// the [SPLITS][Mp][2N] partials (gate in columns [0, N), up in [N, 2N)), all
// Mp rows (pad rows come out 0 as in the unsplit epilogue).
template <int SPLITS>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_swiglu(const float* __restrict__ part,
                                                                 bf16* __restrict__ act, int Mp,
                                                                 int N) {
  const int n4 = N / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= Mp * n4) return;
  const int m = idx / n4, n = (idx % n4) * 4;
  const size_t plane = (size_t)Mp * 2 * N;
  const float* p = part + (size_t)m * 2 * N + n;
  f32x4 gv[SPLITS], uv[SPLITS];
#pragma unroll
  for (int z = 0; z < SPLITS; ++z) {
    gv[z] = *reinterpret_cast<const f32x4*>(p + z * plane);
    uv[z] = *reinterpret_cast<const f32x4*>(p + z * plane + N);
  }
  f32x4 g = gv[0], u = uv[0];
#pragma unroll
  for (int z = 1; z < SPLITS; ++z) {
    g += gv[z];
    u += uv[z];
  }
  u32x2 o;
  o[0] = pack2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
  o[1] = pack2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
  *reinterpret_cast<u32x2*>(act + (size_t)m * N + n) = o;
}

// Split-K reduce of a residual GEMM fused with the RMSNorm that follows it:
// one 256-thread workgroup per row sums the partials (8 columns per thread
// per pass), adds the residual, stores h (bf16) and y = h / sqrt(mean(h^2) +
// eps) * g computed from that stored h.  Rows in [M, Mp) get y = 0 (dummy
// tokens).  N = hidden, a multiple of 64, at most 256 * 8 * CH.
template <int CH, int SPLITS>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_norm(
    const float* __restrict__ part, bf16* __restrict__ H_out,
    const bf16* __restrict__ R, const bf16* __restrict__ g, bf16* __restrict__ Y, int M, int Mp,
    int N, float eps) {
  const int tid = threadIdx.x;
  const int m = blockIdx.x;
  bf16* yr = Y + (size_t)m * N;
  if (m >= M) {
    for (int c = tid * 8; c < N; c += 256 * 8) *reinterpret_cast<u32x4*>(yr + c) = u32x4{0, 0, 0, 0};
    return;
  }
  const size_t plane = (size_t)Mp * N;
  u32x4 hv[CH], gvr[CH];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = (i * 256 + tid) * 8;
    if (c >= N) {
      hv[i] = u32x4{0, 0, 0, 0};
      gvr[i] = u32x4{0, 0, 0, 0};
      continue;
    }
    const float* p = part + (size_t)m * N + c;
    f32x4 pa[SPLITS], pb[SPLITS];
#pragma unroll
    for (int z = 0; z < SPLITS; ++z) {
      pa[z] = *reinterpret_cast<const f32x4*>(p + z * plane);
      pb[z] = *reinterpret_cast<const f32x4*>(p + z * plane + 4);
    }
    const u32x4 rr = ld16(R + (size_t)m * N + c);
    gvr[i] = ld16(g + c);  // the gains go out with the partials, not after the row sum
    f32x4 a = pa[0], b = pb[0];
#pragma unroll
    for (int z = 1; z < SPLITS; ++z) {
      a += pa[z];
      b += pb[z];
    }
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hv[i][e] = pack2(v[2 * e] + __uint_as_float(rr[e] << 16),
                       v[2 * e + 1] + __uint_as_float(rr[e] & 0xffff0000u));
      const float h0 = __uint_as_float(hv[i][e] << 16), h1 = __uint_as_float(hv[i][e] & 0xffff0000u);
      ss += h0 * h0 + h1 * h1;
    }
    *reinterpret_cast<u32x4*>(H_out + (size_t)m * N + c) = hv[i];
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = (i * 256 + tid) * 8;
    if (c >= N) continue;
    const u32x4 gv = gvr[i];
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __uint_as_float(hv[i][e] << 16) * inv * __uint_as_float(gv[e] << 16);
      const float b = __uint_as_float(hv[i][e] & 0xffff0000u) * inv * __uint_as_float(gv[e] & 0xffff0000u);
      o[e] = pack2(a, b);
    }
    *reinterpret_cast<u32x4*>(yr + c) = o;
  }
}

// ------------------------------------------------------------ dispatch
// Row tile: 288 rows (one tile spans a whole hybrid batch of up to 288 rows,
// so every weight tile is streamed from HBM once) or 128 rows for small
// batches; 128 weight rows per tile.  K is split so that about one
// workgroup per CU is resident (measured best on MI355X: 8 waves of 144x32,
// two per SIMD, behind a 3-stage copy ring), keeping >= 8 k-steps per split.
struct Choice {
  int big;     // 1: 288-row tile, 0: 128-row tile
  int bn96;    // 1: 96-column tile (288-row tiles of plain / residual GEMMs)
  int bn64;    // 1: 64-column tile (288-row tiles of residual GEMMs)
  int r256;    // 1: 256-row tiles instead of 288 (fewer padded rows)
  int splits;  // K splits (1 = none)
  int wide;    // 1: 256-weight-row tile, two stages (two or more row tiles, long k loops)
  int agpr;    // 1: SwiGLU on the one-wave-per-SIMD kernel (gemm_agpr.hip)
  int agpr_fn; // > 0: plain / residual GEMM on the one-wave-per-SIMD kernel, 32 agpr_fn columns
};

// Split K (powers of two, at most 8, at least 8 k-steps per split) while the
// workgroup count stays within one per CU.  The reduce kernels are
// instantiated for 2, 4 and 8 splits, and the plain reduce and the RoPE step
// (which sums the QKV partials) also for 3, 5, 6 and 7 (small-batch QKV).
static int splits_for(int tiles, int ksteps) {
  int sp = 1;
  while (tiles * sp * 2 <= 256 && ksteps / (sp * 2) >= 8 && sp < 8) sp *= 2;
  return sp;
}

static Choice choose(GemmEpilogue epi, int mp, int n, int k) {
  Choice c;
  c.big = mp > 128 ? 1 : 0;
  c.bn96 = 0;
  c.bn64 = 0;
  // large batches: 256-row tiles whenever they pad fewer rows than 288-row
  // ones (129-256 rows, 512 rows as two of 256, ...)
  c.r256 = mp > 128 && (mp + 255) / 256 * 256 < (mp + 287) / 288 * 288 ? 1 : 0;
  const int bm = c.big ? (c.r256 ? 256 : 288) : 128;
  const int mt = (mp + bm - 1) / bm;
  const int ksteps = k / kGemmBK;
  c.wide = 0;
  c.agpr = 0;
  c.agpr_fn = 0;
  if (c.big && mt >= 2 && epi == EPI_SWIGLU && ksteps >= 16) {
    // one wave per SIMD, 112 outputs per tile, no K split: taken where its
    // rounds of 256 workgroups are at least as full as the default tile's
    // (Llama-2-70B-shaped gate/up: 512 workgroups, exactly two rounds)
    const int wg = mt * ((n + 111) / 112);
    const int dt = mt * ((n + 63) / 64);
    const int dwg = dt * splits_for(dt, ksteps);
    if (wg >= 192 &&
        (long long)wg * ((dwg + 255) / 256) >= (long long)dwg * ((wg + 255) / 256)) {
      c.agpr = 1;
      c.splits = 1;
      return c;
    }
  }
  if (c.big && mt >= 2 && epi != EPI_STORE) {
    // two or more row tiles: the MFMA work per weight byte is high enough
    // that the copies, not the weight stream, bound the k loop; a
    // 256-weight-row tile (two 64-deep stages fit the LDS) copies fewer
    // activation bytes per MFMA.  Long k loops only: with fewer than 64
    // k-steps per split the 128-column tiles were faster (O projection).
    // Fewer, wider tiles can fill the last round of workgroups worse
    // (768 rows: 336 wide tiles are 1.3 rounds of 256): keep the wide tile
    // only where its rounds are at least as full as the default tile's.
    const int outw = epi == EPI_SWIGLU ? 128 : 256;
    const int tiles = mt * ((n + outw - 1) / outw);
    const int sp = splits_for(tiles, ksteps);
    const int dtiles = mt * ((n + outw / 2 - 1) / (outw / 2));
    const int dwg = dtiles * splits_for(dtiles, ksteps), wg = tiles * sp;
    const bool fills = (long long)wg * ((dwg + 255) / 256) >= (long long)dwg * ((wg + 255) / 256);
    if (wg >= 192 && ksteps / sp >= 64 && fills) {
      c.wide = 1;
      c.splits = sp;
      return c;
    }
  }
  if (c.big && mt >= 2 && epi != EPI_SWIGLU && ksteps >= 32) {
    // one wave per SIMD with AGPR accumulators, where the wide tile above
    // does not apply (plain GEMMs; k loops too short for it): the widest
    // tile whose workgroups, K split to fill the CUs, take at least 240 of
    // the 256 CUs in one round.  Llama-2-70B-shaped QKV: 160 columns, 2 x 64
    // tiles x 2 splits, 112.4 -> 84.2 us (+4 us for the RoPE step to sum the
    // partials); O: 128 columns, 75.5 -> 71.4 us.  Residual GEMMs with long
    // k loops keep the other tiles: the Llama-2-70B-shaped down projection
    // (448 k-steps) took 274 us here against 213 on the wide tile, and the
    // 512-row Mistral-shaped one (224 k-steps) 68.1 against 62.6 us.
    for (int fn : {7, 5, 4}) {
      if (epi == EPI_RESIDUAL && (fn == 7 || ksteps > 128)) continue;  // fn 7: epilogue spills
      const int tiles = mt * ((n + 32 * fn - 1) / (32 * fn));
      const int sp = splits_for(tiles, ksteps);
      if (tiles * sp >= 240 && tiles * sp <= 256) {
        c.agpr_fn = fn;
        c.splits = sp;
        return c;
      }
    }
  }
  if (epi == EPI_SWIGLU) {
    // a tile yields 64 outputs (gate and up rows side by side); narrow FFN
    // shares (tensor-parallel shapes) need K splits to fill the CUs
    c.splits = splits_for(mt * ((n + 63) / 64), ksteps);
    return c;
  }
  const int t128 = mt * ((n + 127) / 128);
  c.splits = splits_for(t128, ksteps);
  if (!c.big && epi == EPI_STORE) {
    // plain GEMMs of small batches (the QKV projection of decode-heavy
    // batches, whose partials the RoPE step sums): the most splits, up to 8
    // and not only powers of two, that keep one round of 256 workgroups and
    // >= 8 k-steps per split (48 column tiles: 5 splits, 240 workgroups
    // instead of 4 splits and 192)
    for (int s = c.splits + 1; s <= 8; ++s)
      if (t128 * s <= 256 && ksteps / s >= 8) c.splits = s;
    return c;
  }
  // residual GEMMs with short k loops (the O projection): 64-column tiles
  // need half the K splits, so half the fp32 partials to write and reduce,
  // which outweighs re-reading A for twice as many column tiles (and where
  // the 128-column tile gives few workgroups, doubles them).  They sum K in
  // two k-groups, so very short k loops (< 16 steps) keep the 128-column
  // tile and its per-element summation order, that of the 128-row tile.
  if (c.big && epi == EPI_RESIDUAL && ksteps >= 16 && ksteps <= 64) {
    const int t64 = mt * ((n + 63) / 64);
    const int s64 = splits_for(t64, ksteps);
    if (t64 * s64 <= 256 && t64 * s64 >= t128 * c.splits) {
      c.bn64 = 1;
      c.splits = s64;
      return c;
    }
  }
  if (c.big && ksteps >= 32) {
    // narrower tiles when they fill more CUs (QKV-like widths); they sum K in
    // two k-groups, so short-K shapes keep the 128-column tile and with it the
    // same per-element summation order as the 128-row tile
    const int t96 = mt * ((n + 95) / 96);
    const int s96 = splits_for(t96, ksteps);
    if (t96 * s96 <= 256 && t96 * s96 > t128 * c.splits) {
      c.bn96 = 1;
      c.splits = s96;
    }
  }
  return c;
}

int gemm_splits(GemmEpilogue epi, int mp, int n, int k) { return choose(epi, mp, n, k).splits; }

size_t gemm_workspace_bytes(GemmEpilogue epi, int mp, int n, int k) {
  const Choice c = choose(epi, mp, n, k);
  const size_t width = epi == EPI_SWIGLU ? 2 * (size_t)n : (size_t)n;  // gate and up partials
  return c.splits > 1 ? (size_t)c.splits * mp * width * sizeof(float) : 0;
}

// Row tile BM (288 or 256) of the large-batch GEMMs.
template <int EPI, int BM>
static hipError_t run_big(const Choice& ch, const bf16* a, const bf16* w, const bf16* w2, bf16* c,
                          const bf16* r, float* part, int m, int mp, int n, int k, hipStream_t s) {
  if (ch.wide)
    return run_gemm_dma<BM, 256, 2, 4, EPI, 2, 64, 1>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
  if constexpr (EPI == EPI_RESIDUAL) {
    if (ch.bn64)
      return run_gemm_dma<BM, 64, 2, 2, EPI, 3, 64, 2, true>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
  }
  if constexpr (EPI != EPI_SWIGLU) {
    if (ch.bn96)
      return run_gemm_dma<BM, 96, 2, 2, EPI, 3, 64, 2>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
  }
  // the 128-column tiles run the two waves of a SIMD half a k-step apart
  // (ping-pong); the 96-column tile, whose k loops are short, does not gain
  // from it.
  // long k loops amortise the k-group reduction: 4 waves per group, each
  // with a (BM / 2) x 64 sub-tile (fewer LDS bytes per MFMA)
  if ((k / kGemmBK) / ch.splits >= 48)
    return run_gemm_dma<BM, 128, 2, 2, EPI, 3, 64, 2, true>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
  return run_gemm_dma<BM, 128, 2, 4, EPI, 3, 64, 1, true>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
}

template <int EPI>
static hipError_t run_choice(const Choice& ch, const bf16* a, const bf16* w, const bf16* w2,
                             bf16* c, const bf16* r, float* part, int m, int mp, int n, int k,
                             hipStream_t s) {
  if constexpr (EPI != EPI_SWIGLU) {
    if (ch.agpr_fn)
      return launch_gemm_agpr(static_cast<GemmEpilogue>(EPI), ch.agpr_fn, a, w, c, r, part, m, mp,
                              n, k, ch.splits, ch.r256, s);
  }
  if (ch.big && ch.r256) return run_big<EPI, 256>(ch, a, w, w2, c, r, part, m, mp, n, k, s);
  if (ch.big) return run_big<EPI, 288>(ch, a, w, w2, c, r, part, m, mp, n, k, s);
  // small batches (decode-heavy iterations): the row tile shrinks with the
  // batch, so each k-step copies fewer (clamped, repeated) activation rows
  // beside the same weight rows; the per-element summation order is that of
  // the 128-row tile
  if (mp <= 32)
    return run_gemm_dma<32, 128, 1, 4, EPI, 4>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
  if (mp <= 64)
    return run_gemm_dma<64, 128, 2, 2, EPI, 4>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
  return run_gemm_dma<128, 128, 2, 2, EPI, 4>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
}

hipError_t launch_gemm_partials(const bf16* a, const bf16* w, void* ws, int m, int mp, int n, int k,
                                hipStream_t s) {
  if (mp == 0 || n == 0) return hipSuccess;
  const Choice ch = choose(EPI_STORE, mp, n, k);
  if (ch.splits <= 1 || ws == nullptr) return hipErrorInvalidValue;
  return run_choice<EPI_STORE>(ch, a, w, nullptr, nullptr, nullptr, reinterpret_cast<float*>(ws),
                               m, mp, n, k, s);
}

hipError_t launch_gemm(GemmEpilogue epi, const bf16* a, const bf16* w, const bf16* w2, bf16* c,
                       const bf16* residual, void* ws, int m, int m_padded, int n, int k,
                       hipStream_t s, hipEvent_t mid) {
  if (m_padded == 0 || n == 0) return hipSuccess;
  Choice ch = choose(epi, m_padded, n, k);
  if (ch.splits > 1 && ws == nullptr) ch.splits = 1;
  float* part = reinterpret_cast<float*>(ws);
  hipError_t e;
  if (ch.agpr) {
    if ((e = launch_swiglu_agpr(a, w, w2, c, m_padded, n, k, ch.r256, s)) != hipSuccess) return e;
    return mid ? hipEventRecord(mid, s) : hipSuccess;
  }
  switch (epi) {
    case EPI_STORE:
      e = run_choice<EPI_STORE>(ch, a, w, nullptr, c, nullptr, part, m, m_padded, n, k, s);
      break;
    case EPI_RESIDUAL:
      e = run_choice<EPI_RESIDUAL>(ch, a, w, nullptr, c, residual, part, m, m_padded, n, k, s);
      break;
    default:
      e = run_choice<EPI_SWIGLU>(ch, a, w, w2, c, nullptr, part, m, m_padded, n, k, s);
      break;
  }
  if (e != hipSuccess) return e;
  if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
  if (ch.splits == 1) return hipSuccess;
  if (epi == EPI_SWIGLU) {
    const int threads = m_padded * (n / 4);
    const dim3 grid((threads + 255) / 256), block(256);
    if (ch.splits == 2)
      hipLaunchKernelGGL(gemm_splitk_reduce_swiglu<2>, grid, block, 0, s, part, c, m_padded, n);
    else if (ch.splits == 4)
      hipLaunchKernelGGL(gemm_splitk_reduce_swiglu<4>, grid, block, 0, s, part, c, m_padded, n);
    else
      hipLaunchKernelGGL(gemm_splitk_reduce_swiglu<8>, grid, block, 0, s, part, c, m_padded, n);
    return hipGetLastError();
  }
  const int mlim = epi == EPI_RESIDUAL ? m : m_padded;
  const int threads = mlim * (n / 4);
  if (threads == 0) return hipSuccess;
  const dim3 grid((threads + 255) / 256), block(256);
#define HL_REDUCE(E_, S_) \
  hipLaunchKernelGGL((gemm_splitk_reduce<E_, S_>), grid, block, 0, s, part, c, residual, m, m_padded, n)
  if (epi == EPI_RESIDUAL) {
    if (ch.splits == 2) HL_REDUCE(EPI_RESIDUAL, 2);
    else if (ch.splits == 4) HL_REDUCE(EPI_RESIDUAL, 4);
    else HL_REDUCE(EPI_RESIDUAL, 8);
  } else {
    if (ch.splits == 2) HL_REDUCE(EPI_STORE, 2);
    else if (ch.splits == 3) HL_REDUCE(EPI_STORE, 3);
    else if (ch.splits == 4) HL_REDUCE(EPI_STORE, 4);
    else if (ch.splits == 5) HL_REDUCE(EPI_STORE, 5);
    else if (ch.splits == 6) HL_REDUCE(EPI_STORE, 6);
    else if (ch.splits == 7) HL_REDUCE(EPI_STORE, 7);
    else HL_REDUCE(EPI_STORE, 8);
  }
#undef HL_REDUCE
  return hipGetLastError();
}

template <int CH>
static void launch_rn(const float* part, int splits, bf16* h, const bf16* r, const bf16* g,
                      bf16* y, int m, int mp, int n, float eps, hipStream_t s) {
  if (splits == 2)
    hipLaunchKernelGGL((gemm_splitk_reduce_norm<CH, 2>), dim3(mp), dim3(256), 0, s, part, h, r, g,
                       y, m, mp, n, eps);
  else if (splits == 4)
    hipLaunchKernelGGL((gemm_splitk_reduce_norm<CH, 4>), dim3(mp), dim3(256), 0, s, part, h, r, g,
                       y, m, mp, n, eps);
  else
    hipLaunchKernelGGL((gemm_splitk_reduce_norm<CH, 8>), dim3(mp), dim3(256), 0, s, part, h, r, g,
                       y, m, mp, n, eps);
}

hipError_t launch_gemm_residual_norm(const bf16* a, const bf16* w, bf16* h, const bf16* residual,
                                     const bf16* g, bf16* y, float eps, void* ws, int m,
                                     int m_padded, int n, int k, hipStream_t s, hipEvent_t mid) {
  if (m_padded == 0 || n == 0) return hipSuccess;
  Choice ch = choose(EPI_RESIDUAL, m_padded, n, k);
  const int nch = (n + 2047) / 2048;  // 8-column chunks per thread
  if (ch.splits == 1 || ws == nullptr || nch > 8) {
    hipError_t e = launch_gemm(EPI_RESIDUAL, a, w, nullptr, h, residual, ws, m, m_padded, n, k, s,
                               mid);
    if (e != hipSuccess) return e;
    return launch_rmsnorm(h, g, y, m, m_padded, n, eps, s);
  }
  float* part = reinterpret_cast<float*>(ws);
  hipError_t e = run_choice<EPI_RESIDUAL>(ch, a, w, nullptr, h, residual, part, m, m_padded, n, k, s);
  if (e != hipSuccess) return e;
  if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
  if (nch <= 1) launch_rn<1>(part, ch.splits, h, residual, g, y, m, m_padded, n, eps, s);
  else if (nch <= 2) launch_rn<2>(part, ch.splits, h, residual, g, y, m, m_padded, n, eps, s);
  else if (nch <= 4) launch_rn<4>(part, ch.splits, h, residual, g, y, m, m_padded, n, eps, s);
  else launch_rn<8>(part, ch.splits, h, residual, g, y, m, m_padded, n, eps, s);
  return hipGetLastError();
}

}  // namespace hl

// One-wave-per-SIMD GEMM for the MFMA-bound gate/up projection
// (act = silu(x W_gate^T) * (x W_up^T) on two or more row tiles).
//
// Each workgroup has four waves, one per SIMD, so each wave owns the whole
// register file of its SIMD lane: 256 VGPRs and 256 AGPRs.  That buys a
// large wave tile.  A 288 x 224 tile (288 rows of x; 112 gate and 112 up
// rows of the weights, i.e. 112 outputs) splits into four waves of
// 144 rows x 112 weight rows.  Each wave keeps 9 x 7 MFMA blocks = 252 fp32
// accumulators in AGPRs.  Per 32-wide k sub-step a wave reads 16 KB of
// fragments from LDS for 63 MFMAs, a quarter fewer LDS bytes per MFMA than
// the 144 x 64 wave tiles of gemm_dma_kernel, and the workgroup copies
// (288 + 224) x 128 B per 64-deep k-step, half a byte per 64 flops less.
//
// The loads go global -> LDS directly (global_load_lds_dwordx4), tracked by
// hand with vmcnt waits: x (activation) rows one k-step ahead into two
// 64-deep slots (72 KB), weight rows, which come from HBM, two k-steps ahead
// into three slots (84 KB).  One barrier per k-step.  The fragments of a
// step's second sub-step are read while the first sub-step's MFMAs issue,
// and the copies are spread between the MFMA groups.
//
// Gate and up rows live in different waves (waves 0-1 gate, 2-3 up).  After
// the k loop the up waves hand their accumulators to the gate waves through
// LDS, and the gate waves apply SwiGLU and store.
//
// The MFMAs are written as inline asm with the accumulator tied to one
// AGPR tuple (destination = source C).  Given the builtin, the compiler
// kept these loop-carried accumulators in AGPRs only through two copies per
// MFMA and iteration.  Its hazard tracking does not see into the asm, so the
// code keeps the MFMA results away from other instructions itself: the
// accumulators are read only by later MFMAs of the same shape (back-to-back
// accumulation needs no wait states) and, after the loop, by the epilogue
// behind an explicit s_nop pad.
#include "gemm_impl.h"

namespace hl {

__device__ __forceinline__ void mfma_acc(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

constexpr int kAgprHalf = 112;  // gate (or up) weight rows per tile = outputs per tile

template <int BM>
__global__ __launch_bounds__(256, 1) void gemm_swiglu_agpr_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ Wg, const bf16* __restrict__ Wu,
    bf16* __restrict__ C, int Mp, int N, int K, int n_mtiles, int n_ntiles) {
  constexpr int HALF = kAgprHalf;
  constexpr int BN = 2 * HALF;        // weight rows per tile
  constexpr int WTM = BM / 2;         // rows per wave
  constexpr int FM = WTM / 16;        // MFMA row blocks per wave
  constexpr int FN = HALF / 16;       // MFMA weight-row blocks per wave
  constexpr int A_BLK = BM / 8;       // 1 KB copy blocks of x per stage (8 rows x 128 B)
  constexpr int W_BLK = BN / 8;       // 1 KB blocks of weights per stage
  constexpr int A_PW = A_BLK / 4;     // per wave
  constexpr int W_PW = W_BLK / 4;
  constexpr int A_SLOT = A_BLK * 1024, W_SLOT = W_BLK * 1024;
  constexpr int W_RING = 2 * A_SLOT;  // weight slots follow the two x slots
  static_assert(BM % 32 == 0 && A_BLK % 4 == 0 && W_BLK % 4 == 0, "whole blocks per wave");
  static_assert(W_PW * 2 * 8 == HALF, "each wave copies weight rows of one matrix");
  static_assert(FM * FN * 4 <= 256, "accumulators fit the AGPRs");

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // tiles that share a weight tile (all row tiles of one column tile) are
  // numbered consecutively inside one XCD's share of the grid
  const int total = n_mtiles * n_ntiles;
  const int b = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = b % 8, slot = b / 8;
  const int tile = xcd * per + min(xcd, rem) + slot;
  const int tm = tile % n_mtiles, tn = tile / n_mtiles;
  const int m0 = tm * BM, n0 = tn * HALF;
  const int nk = K / 64;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // wn 0: gate rows, 1: up rows
  const int l16 = lane & 15, q = lane >> 4;
  // 16-byte chunk c of a stage row r sits in slot c ^ (r % 8); copy lanes
  // take row lane / 8 of their block (blocks start at multiples of 8 rows)
  const int chunk = (lane & 7) ^ (lane >> 3);

  // x blocks of this wave: w * A_PW + i (rows clamped to the last padded row)
  uint32_t aoff[A_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) {
    const int row = (wave * A_PW + i) * 8 + (lane >> 3);
    aoff[i] = ((uint32_t)min(m0 + row, Mp - 1) * (uint32_t)K + (uint32_t)chunk * 8u) * 2u;
  }
  // weight blocks of this wave: w * W_PW + j; waves 0-1 copy gate rows,
  // 2-3 up rows, 56 rows each
  const bf16* wmat = wave < 2 ? Wg : Wu;
  uint32_t woff[W_PW];
#pragma unroll
  for (int j = 0; j < W_PW; ++j) {
    const int n = n0 + (wave & 1) * (HALF / 2) + j * 8 + (lane >> 3);
    woff[j] = ((uint32_t)min(n, N - 1) * (uint32_t)K + (uint32_t)chunk * 8u) * 2u;
  }
  auto issue_a = [&](int step) {  // x rows of k-step `step` (clamped) into its slot
    const int kt = min(step, nk - 1);
    char* st = smem + (step & 1) * A_SLOT;
#pragma unroll
    for (int i = 0; i < A_PW; ++i)
      lds_copy16(A + (size_t)kt * 64, aoff[i], st + (wave * A_PW + i) * 1024);
  };
  auto issue_w = [&](int step) {  // weight rows of k-step `step` (clamped) into its slot
    const int kt = min(step, nk - 1);
    char* st = smem + W_RING + (step % 3) * W_SLOT;
#pragma unroll
    for (int j = 0; j < W_PW; ++j)
      lds_copy16(wmat + (size_t)kt * 64, woff[j], st + (wave * W_PW + j) * 1024);
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment rows: x rows wm * WTM + 16 j + l16, weight rows (after the x
  // rows of the stage) wn * HALF + 16 i + l16; both start at multiples of 16
  const int a_base = (wm * WTM + l16) * 128;
  const int w_base = (wn * HALF + l16) * 128;
  auto read_sub = [&](const char* sa, const char* sw, int kk, bf16x8 (&wf)[FN],
                      bf16x8 (&af)[FM]) {
    const int so = (((kk * 4 + q) ^ (l16 & 7)) << 4);
#pragma unroll
    for (int i = 0; i < FN; ++i) wf[i] = as_bf16x8(ld16(sw + w_base + i * 2048 + so));
#pragma unroll
    for (int j = 0; j < FM; ++j) af[j] = as_bf16x8(ld16(sa + a_base + j * 2048 + so));
  };

  if (nk > 0) {
    // per wave, in issue order: ... x(it) w(it+1) | x(it+1) w(it+2) | ...;
    // at the top of step it only the weight copies issued last, w(it+1), may
    // still be in flight
    issue_a(0);
    issue_w(0);
    issue_w(1);
    for (int it = 0; it < nk; ++it) {
      wait_vmcnt<W_PW>();
      asm volatile("" ::: "memory");  // keep LDS reads and copies on their side of the barrier
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const char* sa = smem + (it & 1) * A_SLOT;
      const char* sw = smem + W_RING + (it % 3) * W_SLOT;
      bf16x8 wf0[FN], af0[FM], wf1[FN], af1[FM];
      read_sub(sa, sw, 0, wf0, af0);
      // The copies of the next steps (into the slots of step it-1, which
      // every wave finished reading before this step's barrier) and the
      // second sub-step's fragment reads go between the MFMA groups, one x
      // copy per group of the first sub-step and one weight copy per group
      // of the second, rather than in one burst (a burst after the barrier
      // measured 15 % slower; Llama-2-70B-shaped gate/up 499 -> 435 us).
      const int kta = min(it + 1, nk - 1), ktw = min(it + 2, nk - 1);
      char* da = smem + ((it + 1) & 1) * A_SLOT;
      char* dw = smem + W_RING + ((it + 2) % 3) * W_SLOT;
      const int so1 = (((4 + q) ^ (l16 & 7)) << 4);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
#pragma unroll
        for (int i = 0; i < FN; ++i) mfma_acc(acc[i][j], wf0[i], af0[j]);
        if (j < A_PW) lds_copy16(A + (size_t)kta * 64, aoff[j], da + (wave * A_PW + j) * 1024);
        if (j < FN) wf1[j] = as_bf16x8(ld16(sw + w_base + j * 2048 + so1));
        af1[j] = as_bf16x8(ld16(sa + a_base + j * 2048 + so1));
      }
#pragma unroll
      for (int j = FM; j < A_PW; ++j)
        lds_copy16(A + (size_t)kta * 64, aoff[j], da + (wave * A_PW + j) * 1024);
#pragma unroll
      for (int j = FM; j < FN; ++j) wf1[j] = as_bf16x8(ld16(sw + w_base + j * 2048 + so1));
#pragma unroll
      for (int j = 0; j < FM; ++j) {
#pragma unroll
        for (int i = 0; i < FN; ++i) mfma_acc(acc[i][j], wf1[i], af1[j]);
        if (j < W_PW) lds_copy16(wmat + (size_t)ktw * 64, woff[j], dw + (wave * W_PW + j) * 1024);
      }
    }
  }
  wait_vmcnt<0>();  // the clamped tail copies land before the LDS is reused
  // MFMA results are read below by VALU / LDS instructions the compiler
  // places; pad well past the longest MFMA-write -> read wait
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __syncthreads();
  // up waves hand their accumulators to the gate wave of the same rows
  f32x4* xch = reinterpret_cast<f32x4*>(smem) + (size_t)wm * FN * FM * 64;
  if (wn == 1) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) xch[(i * FM + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  if (wn == 0) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * WTM + j * 16 + l16;
      if (m >= Mp) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + i * 16 + 4 * q;
        if (n >= N) continue;
        const f32x4 g = acc[i][j], u = xch[(i * FM + j) * 64 + lane];
        u32x2 o;
        o[0] = pack2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
        o[1] = pack2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
        *reinterpret_cast<u32x2*>(C + (size_t)m * N + n) = o;
      }
    }
  }
}

// The same schedule for one weight matrix: plain (QKV) and residual (O,
// down) projections.  The tile is BM rows x 2 * 16 FN weight rows; waves
// are (row half) x (column half), each with 9 x FN accumulator blocks of its
// own outputs, so no exchange is needed.  K may be split over workgroups
// (`splits` > 1): the tile then stores its fp32 partial [z][Mp][N] for the
// reduce kernels of gemm.hip; unsplit it stores bf16 (plus the residual R,
// rows < M, for EPI_RESIDUAL).
template <int BM, int FN, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_agpr_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, bf16* __restrict__ C,
    const bf16* __restrict__ R, float* __restrict__ part, int M, int Mp, int N, int K,
    int n_mtiles, int n_ntiles, int splits) {
  constexpr int HALF = 16 * FN;       // weight rows (outputs) per wave
  constexpr int BN = 2 * HALF;        // weight rows per tile
  constexpr int WTM = BM / 2;         // rows per wave
  constexpr int FM = WTM / 16;        // MFMA row blocks per wave
  constexpr int A_BLK = BM / 8;       // 1 KB copy blocks of x per stage (8 rows x 128 B)
  constexpr int W_BLK = BN / 8;       // 1 KB blocks of weights per stage
  constexpr int A_PW = A_BLK / 4;     // per wave
  constexpr int W_PW = W_BLK / 4;
  constexpr int A_SLOT = A_BLK * 1024, W_SLOT = W_BLK * 1024;
  constexpr int W_RING = 2 * A_SLOT;  // weight slots follow the two x slots
  static_assert(BM % 32 == 0 && A_BLK % 4 == 0 && W_BLK % 4 == 0, "whole blocks per wave");
  static_assert(A_PW <= FM && W_PW <= FM, "copies spread over the MFMA groups");
  static_assert(FM * FN * 4 <= 256, "accumulators fit the AGPRs");
  static_assert(EPI == EPI_STORE || EPI == EPI_RESIDUAL, "plain or residual epilogue");

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // the row tiles and K splits that share a weight tile are numbered
  // consecutively inside one XCD's share of the grid
  const int total = n_mtiles * n_ntiles * splits;
  const int b = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = b % 8, slot = b / 8;
  const int tile = xcd * per + min(xcd, rem) + slot;
  const int tm = tile % n_mtiles;
  const int rest = tile / n_mtiles;
  const int z = rest % splits, tn = rest / splits;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = K / 64;
  const int kt_per = (KT + splits - 1) / splits;
  const int kt0 = min(KT, z * kt_per);
  const int nk = min(KT, kt0 + kt_per) - kt0;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, q = lane >> 4;
  const int chunk = (lane & 7) ^ (lane >> 3);

  uint32_t aoff[A_PW];
#pragma unroll
  for (int i = 0; i < A_PW; ++i) {
    const int row = (wave * A_PW + i) * 8 + (lane >> 3);
    aoff[i] = ((uint32_t)min(m0 + row, Mp - 1) * (uint32_t)K + (uint32_t)chunk * 8u) * 2u;
  }
  // weight blocks of this wave: w * W_PW + j of the tile's BN rows
  uint32_t woff[W_PW];
#pragma unroll
  for (int j = 0; j < W_PW; ++j) {
    const int n = n0 + (wave * W_PW + j) * 8 + (lane >> 3);
    woff[j] = ((uint32_t)min(n, N - 1) * (uint32_t)K + (uint32_t)chunk * 8u) * 2u;
  }
  const bf16* Ak = A + (size_t)kt0 * 64;
  const bf16* Wk = W + (size_t)kt0 * 64;
  auto issue_a = [&](int step) {
    const int kt = min(step, nk - 1);
    char* st = smem + (step & 1) * A_SLOT;
#pragma unroll
    for (int i = 0; i < A_PW; ++i)
      lds_copy16(Ak + (size_t)kt * 64, aoff[i], st + (wave * A_PW + i) * 1024);
  };
  auto issue_w = [&](int step) {
    const int kt = min(step, nk - 1);
    char* st = smem + W_RING + (step % 3) * W_SLOT;
#pragma unroll
    for (int j = 0; j < W_PW; ++j)
      lds_copy16(Wk + (size_t)kt * 64, woff[j], st + (wave * W_PW + j) * 1024);
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int a_base = (wm * WTM + l16) * 128;
  const int w_base = (wn * HALF + l16) * 128;
  auto read_sub = [&](const char* sa, const char* sw, int kk, bf16x8 (&wf)[FN],
                      bf16x8 (&af)[FM]) {
    const int so = (((kk * 4 + q) ^ (l16 & 7)) << 4);
#pragma unroll
    for (int i = 0; i < FN; ++i) wf[i] = as_bf16x8(ld16(sw + w_base + i * 2048 + so));
#pragma unroll
    for (int j = 0; j < FM; ++j) af[j] = as_bf16x8(ld16(sa + a_base + j * 2048 + so));
  };

  if (nk > 0) {
    issue_a(0);
    issue_w(0);
    issue_w(1);
    for (int it = 0; it < nk; ++it) {
      wait_vmcnt<W_PW>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const char* sa = smem + (it & 1) * A_SLOT;
      const char* sw = smem + W_RING + (it % 3) * W_SLOT;
      bf16x8 wf0[FN], af0[FM], wf1[FN], af1[FM];
      read_sub(sa, sw, 0, wf0, af0);
      const int kta = min(it + 1, nk - 1), ktw = min(it + 2, nk - 1);
      char* da = smem + ((it + 1) & 1) * A_SLOT;
      char* dw = smem + W_RING + ((it + 2) % 3) * W_SLOT;
      const int so1 = (((4 + q) ^ (l16 & 7)) << 4);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
#pragma unroll
        for (int i = 0; i < FN; ++i) mfma_acc(acc[i][j], wf0[i], af0[j]);
        if (j < A_PW) lds_copy16(Ak + (size_t)kta * 64, aoff[j], da + (wave * A_PW + j) * 1024);
        if (j < FN) wf1[j] = as_bf16x8(ld16(sw + w_base + j * 2048 + so1));
        af1[j] = as_bf16x8(ld16(sa + a_base + j * 2048 + so1));
      }
#pragma unroll
      for (int j = FM; j < FN; ++j) wf1[j] = as_bf16x8(ld16(sw + w_base + j * 2048 + so1));
#pragma unroll
      for (int j = 0; j < FM; ++j) {
#pragma unroll
        for (int i = 0; i < FN; ++i) mfma_acc(acc[i][j], wf1[i], af1[j]);
        if (j < W_PW) lds_copy16(Wk + (size_t)ktw * 64, woff[j], dw + (wave * W_PW + j) * 1024);
      }
    }
  }
  wait_vmcnt<0>();  // the clamped tail copies land before the workgroup ends
  // MFMA results are read below by instructions the compiler places; pad
  // well past the longest MFMA-write -> read wait
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = m0 + wm * WTM + j * 16 + l16;
    if (splits > 1) {
      if (m >= Mp) continue;
      float* pp = part + ((size_t)z * Mp + m) * N;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * HALF + i * 16 + 4 * q;
        if (n < N) *reinterpret_cast<f32x4*>(pp + n) = acc[i][j];
      }
      continue;
    }
    if (m >= (EPI == EPI_RESIDUAL ? M : Mp)) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = n0 + wn * HALF + i * 16 + 4 * q;
      if (n >= N) continue;
      f32x4 v = acc[i][j];
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
  }
}

template <int BM>
static hipError_t run_agpr(const bf16* a, const bf16* wg, const bf16* wu, bf16* c, int mp, int n,
                           int k, hipStream_t s) {
  constexpr size_t ring = (size_t)(2 * (BM / 8) + 3 * (2 * kAgprHalf / 8)) * 1024;
  constexpr size_t xch = (size_t)2 * (BM / 32) * (kAgprHalf / 16) * 1024;
  constexpr size_t lds = ring > xch ? ring : xch;
  static_assert(lds <= 160 * 1024, "LDS budget");
  if ((size_t)mp * k * sizeof(bf16) > UINT32_MAX || (size_t)n * k * sizeof(bf16) > UINT32_MAX)
    return hipErrorInvalidValue;
  const int mt = (mp + BM - 1) / BM, nt = (n + kAgprHalf - 1) / kAgprHalf;
  auto kern = gemm_swiglu_agpr_kernel<BM>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(mt * nt), dim3(256), lds, s, a, wg, wu, c, mp, n, k, mt, nt);
  return hipGetLastError();
}

hipError_t launch_swiglu_agpr(const bf16* a, const bf16* wg, const bf16* wu, bf16* act, int mp,
                              int f, int k, bool rows256, hipStream_t s) {
  return rows256 ? run_agpr<256>(a, wg, wu, act, mp, f, k, s)
                 : run_agpr<288>(a, wg, wu, act, mp, f, k, s);
}

template <int BM, int FN, int EPI>
static hipError_t run_agpr_plain(const bf16* a, const bf16* w, bf16* c, const bf16* r,
                                 float* part, int m, int mp, int n, int k, int splits,
                                 hipStream_t s) {
  constexpr int BN = 32 * FN;
  constexpr size_t lds = (size_t)(2 * (BM / 8) + 3 * (BN / 8)) * 1024;
  static_assert(lds <= 160 * 1024, "LDS budget");
  if ((size_t)mp * k * sizeof(bf16) > UINT32_MAX || (size_t)n * k * sizeof(bf16) > UINT32_MAX)
    return hipErrorInvalidValue;
  const int mt = (mp + BM - 1) / BM, nt = (n + BN - 1) / BN;
  auto kern = gemm_agpr_kernel<BM, FN, EPI>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(mt * nt * splits), dim3(256), lds, s, a, w, c, r, part, m, mp, n,
                     k, mt, nt, splits);
  return hipGetLastError();
}

hipError_t launch_gemm_agpr(GemmEpilogue epi, int fn, const bf16* a, const bf16* w, bf16* c,
                            const bf16* r, float* part, int m, int mp, int n, int k, int splits,
                            bool rows256, hipStream_t s) {
#define HL_AGPR(BM_, FN_)                                                                      \
  return epi == EPI_RESIDUAL                                                                   \
             ? run_agpr_plain<BM_, FN_, EPI_RESIDUAL>(a, w, c, r, part, m, mp, n, k, splits, s) \
             : run_agpr_plain<BM_, FN_, EPI_STORE>(a, w, c, r, part, m, mp, n, k, splits, s)
#define HL_AGPR_STORE(BM_, FN_) \
  return run_agpr_plain<BM_, FN_, EPI_STORE>(a, w, c, r, part, m, mp, n, k, splits, s)
  // fn 7 is plain only: with the residual epilogue its registers spill
  if (epi == EPI_SWIGLU || (fn == 7 && epi == EPI_RESIDUAL)) return hipErrorInvalidValue;
  if (rows256) {
    if (fn == 4) HL_AGPR(256, 4);
    if (fn == 5) HL_AGPR(256, 5);
    if (fn == 7) HL_AGPR_STORE(256, 7);
  } else {
    if (fn == 4) HL_AGPR(288, 4);
    if (fn == 5) HL_AGPR(288, 5);
    if (fn == 7) HL_AGPR_STORE(288, 7);
  }
#undef HL_AGPR_STORE
#undef HL_AGPR
  return hipErrorInvalidValue;
}

}  // namespace hl

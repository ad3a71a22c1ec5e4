// bf16 MFMA GEMM for the linear layers of the hybrid batch:
//   C[m, n] = sum_k A[m, k] * W[n, k]      (A = activations, W = [out, in] weights)
// run once on the stacked chunk + decode rows.
//
// Structure (gfx950, wave64):
//  * a workgroup owns a BM x BN output tile and walks K in steps of 64;
//    A and W tiles are staged through LDS, double-buffered, with the next
//    tile's global loads in flight while the current one is multiplied;
//  * each wave computes C^T = W A^T on its sub-tile with
//    v_mfma_f32_16x16x32_bf16, so a lane ends up holding four consecutive
//    output columns of one row and stores them as one 8-byte write;
//  * workgroups are numbered so that the ones sharing a weight tile land on
//    the same XCD (workgroup ids are dealt round-robin over the 8 XCDs) and
//    reuse it from that XCD's L2;
//  * epilogues: plain store (QKV), residual add (O and down projections),
//    SwiGLU (gate and up tiles side by side in one workgroup, combined in
//    registers).
#include "kernels.h"

namespace hl {

constexpr int kBK = 64;
constexpr int kLdsPad = 8;  // bf16 elements of padding per LDS row
constexpr int kLdsRow = kBK + kLdsPad;

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W2,
    bf16* __restrict__ C, const bf16* __restrict__ R, int M, int Mp, int N, int K, int n_mtiles,
    int n_ntiles) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM;  // rows of a wave tile
  constexpr int WTN = BN / WN;  // LDS W rows of a wave tile
  constexpr int FM = WTM / 16;
  constexpr int FN = WTN / 16;
  constexpr int OUT_N = EPI == EPI_SWIGLU ? BN / 2 : BN;  // output columns per tile
  constexpr int A_CHUNKS = BM * (kBK / 8) / NT;
  constexpr int W_CHUNKS = BN * (kBK / 8) / NT;
  static_assert(BM * (kBK / 8) % NT == 0 && BN * (kBK / 8) % NT == 0, "tile/thread mismatch");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "swiglu needs paired fragments");

  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16 Ws[2][BN * kLdsRow];

  // XCD-aware tile order: XCD x runs a contiguous range of tiles, n-major,
  // so the m-tiles of one weight tile run together on one XCD.
  const int total = n_mtiles * n_ntiles;
  const int b = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int x = b % 8, s = b / 8;
  const int tile = x * per + min(x, rem) + s;
  const int tn = tile / n_mtiles, tm = tile % n_mtiles;
  const int m0 = tm * BM, n0 = tn * OUT_N;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, q = lane >> 4;

  u32x4 ra[A_CHUNKS], rw[W_CHUNKS];

  auto load_global = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + i * NT;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      const int m = m0 + row;
      ra[i] = m < Mp ? ld16(A + (size_t)m * K + k0 + kc) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int c = tid + i * NT;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      const bf16* src;
      int n;
      if (EPI == EPI_SWIGLU) {
        const bool up = row >= BN / 2;
        n = n0 + (up ? row - BN / 2 : row);
        src = up ? W2 : W;
      } else {
        n = n0 + row;
        src = W;
      }
      rw[i] = n < N ? ld16(src + (size_t)n * K + k0 + kc) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_lds = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + i * NT;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      *reinterpret_cast<u32x4*>(&As[st][row * kLdsRow + kc]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int c = tid + i * NT;
      const int row = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ws[st][row * kLdsRow + kc]) = rw[i];
    }
  };
  // LDS row of the wave's fn-th 16-row W fragment
  auto w_row = [&](int fn) {
    if (EPI == EPI_SWIGLU) {
      constexpr int HALF = FN / 2;
      return fn < HALF ? wn * (WTN / 2) + fn * 16 : BN / 2 + wn * (WTN / 2) + (fn - HALF) * 16;
    }
    return wn * WTN + fn * 16;
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = K / kBK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8 af[FN], bfr[FM];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        af[fn] = as_bf16x8(ld16(&Ws[st][(w_row(fn) + l16) * kLdsRow + ks * 32 + q * 8]));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        bfr[fm] = as_bf16x8(ld16(&As[st][(wm * WTM + fm * 16 + l16) * kLdsRow + ks * 32 + q * 8]));
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma16x16x32(af[fn], bfr[fm], acc[fn][fm]);
    }
    if (kt + 1 < KT) store_lds(st ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[m][n .. n+3] for m = .. + l16, n = .. + 4q
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + wm * WTM + fm * 16 + l16;
    if (EPI == EPI_SWIGLU) {
      if (m >= Mp) continue;
#pragma unroll
      for (int fn = 0; fn < FN / 2; ++fn) {
        const int n = n0 + wn * (WTN / 2) + fn * 16 + 4 * q;
        if (n >= N) continue;
        const f32x4 g = acc[fn][fm], u = acc[fn + FN / 2][fm];
        u32x2 o;
        o[0] = pack2(silu_f(g[0]) * u[0], silu_f(g[1]) * u[1]);
        o[1] = pack2(silu_f(g[2]) * u[2], silu_f(g[3]) * u[3]);
        *reinterpret_cast<u32x2*>(C + (size_t)m * N + n) = o;
      }
    } else {
      const int mlim = EPI == EPI_RESIDUAL ? M : Mp;
      if (m >= mlim) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + wn * WTN + fn * 16 + 4 * q;
        if (n >= N) continue;
        f32x4 v = acc[fn][fm];
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
}

template <int BM, int BN, int WM, int WN, int EPI>
static hipError_t run_gemm(const bf16* a, const bf16* w, const bf16* w2, bf16* c, const bf16* r,
                           int m, int mp, int n, int k, hipStream_t s) {
  constexpr int OUT_N = EPI == EPI_SWIGLU ? BN / 2 : BN;
  const int mt = (mp + BM - 1) / BM, nt = (n + OUT_N - 1) / OUT_N;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI>), dim3(mt * nt), dim3(64 * WM * WN), 0, s,
                     a, w, w2, c, r, m, mp, n, k, mt, nt);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmEpilogue epi, const bf16* a, const bf16* w, const bf16* w2, bf16* c,
                       const bf16* residual, int m, int m_padded, int n, int k, hipStream_t s) {
  if (m_padded == 0 || n == 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE:
      return run_gemm<64, 64, 2, 2, EPI_STORE>(a, w, nullptr, c, nullptr, m, m_padded, n, k, s);
    case EPI_RESIDUAL:
      return run_gemm<64, 64, 2, 2, EPI_RESIDUAL>(a, w, nullptr, c, residual, m, m_padded, n, k, s);
    case EPI_SWIGLU:
      return run_gemm<64, 128, 2, 2, EPI_SWIGLU>(a, w, w2, c, nullptr, m, m_padded, n, k, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hl

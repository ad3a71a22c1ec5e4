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
template <int EPI>
__global__ __launch_bounds__(256) void gemm_splitk_reduce(const float* __restrict__ part, int splits,
                                                          bf16* __restrict__ C,
                                                          const bf16* __restrict__ R, int M, int Mp,
                                                          int N) {
  const int n4 = N / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int mlim = EPI == EPI_RESIDUAL ? M : Mp;
  if (idx >= mlim * n4) return;
  const int m = idx / n4, n = (idx % n4) * 4;
  const size_t plane = (size_t)Mp * N;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)m * N + n);
  for (int z = 1; z < splits; ++z) v += *reinterpret_cast<const f32x4*>(part + z * plane + (size_t)m * N + n);
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

// ------------------------------------------------------------ dispatch
// Row tile: 288 rows (one tile spans a whole hybrid batch of up to 288 rows,
// so every weight tile is streamed from HBM once) or 128 rows for small
// batches; 128 weight rows per tile.  K is split so that about one
// workgroup per CU is resident (measured best on MI355X: 4 waves, 1 per SIMD,
// with the copy pipeline hiding HBM latency), keeping >= 8 k-steps per split.
struct Choice {
  int big;     // 1: 288-row tile, 0: 128-row tile
  int splits;  // K splits (1 = none)
};

static Choice choose(GemmEpilogue epi, int mp, int n, int k) {
  Choice c;
  c.big = mp > 128 ? 1 : 0;
  const int bm = c.big ? 288 : 128;
  const int out_n = epi == EPI_SWIGLU ? 64 : 128;
  const int tiles = ((mp + bm - 1) / bm) * ((n + out_n - 1) / out_n);
  const int ksteps = k / kGemmBK;
  c.splits = 1;
  if (epi != EPI_SWIGLU)
    while (tiles * c.splits * 2 <= 256 && ksteps / (c.splits * 2) >= 8 && c.splits < 8) c.splits *= 2;
  return c;
}

size_t gemm_workspace_bytes(GemmEpilogue epi, int mp, int n, int k) {
  const Choice c = choose(epi, mp, n, k);
  return c.splits > 1 ? (size_t)c.splits * mp * n * sizeof(float) : 0;
}

template <int EPI>
static hipError_t run_choice(const Choice& ch, const bf16* a, const bf16* w, const bf16* w2,
                             bf16* c, const bf16* r, float* part, int m, int mp, int n, int k,
                             hipStream_t s) {
  if (ch.big) return run_gemm_dma<288, 128, 2, 2, EPI, 3>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
  return run_gemm_dma<128, 128, 2, 2, EPI, 4>(a, w, w2, c, r, part, m, mp, n, k, ch.splits, s);
}

hipError_t launch_gemm(GemmEpilogue epi, const bf16* a, const bf16* w, const bf16* w2, bf16* c,
                       const bf16* residual, void* ws, int m, int m_padded, int n, int k,
                       hipStream_t s) {
  if (m_padded == 0 || n == 0) return hipSuccess;
  Choice ch = choose(epi, m_padded, n, k);
  if (ch.splits > 1 && ws == nullptr) ch.splits = 1;
  float* part = reinterpret_cast<float*>(ws);
  hipError_t e;
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
  if (e != hipSuccess || ch.splits == 1) return e;
  const int mlim = epi == EPI_RESIDUAL ? m : m_padded;
  const int threads = mlim * (n / 4);
  if (threads == 0) return hipSuccess;
  if (epi == EPI_RESIDUAL)
    hipLaunchKernelGGL(gemm_splitk_reduce<EPI_RESIDUAL>, dim3((threads + 255) / 256), dim3(256), 0,
                       s, part, ch.splits, c, residual, m, m_padded, n);
  else
    hipLaunchKernelGGL(gemm_splitk_reduce<EPI_STORE>, dim3((threads + 255) / 256), dim3(256), 0,
                       s, part, ch.splits, c, residual, m, m_padded, n);
  return hipGetLastError();
}

}  // namespace hl

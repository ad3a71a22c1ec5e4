// Tile template of the bf16 MFMA GEMM (see gemm.hip for the design notes).
#pragma once
#include "kernels.h"

namespace hl {

constexpr int kGemmBK = 64;

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Global -> LDS copies (global_load_lds_dwordx4, no
// register staging) into a ring of STAGES buffers, so STAGES-1 k-steps of
// loads are in flight while one is multiplied.  A stage holds BK (64 or 32)
// values of K per row, i.e. 8 or 4 chunks of 16 B; one copy instruction fills
// 1 KB = 8 or 16 rows.  Chunk c of row r sits in slot c ^ (r % 8) (BK 64) or
// c ^ ((r / 4) % 4) (BK 32), which keeps the 16-row fragment reads free of
// bank conflicts.  Wave w issues blocks w, w + NW, ...  Rows past the end of
// A or W are clamped to the last valid row: their products only reach
// outputs that are never stored.
// 16-byte global -> LDS copy per lane (global_load_lds_dwordx4), written as
// inline asm.  The compiler models its own form of this copy as an LDS access
// that may complete out of order with LDS reads, and then makes every LDS read
// in the loop wait for all reads before it; hidden from it, the reads get
// exact counts.  Completion of the copies is tracked by hand with vmcnt waits
// and the workgroup barrier.  `lds` is wave-uniform; M0 carries it.
__device__ __forceinline__ void lds_copy16(const bf16* src, char* lds) {
  const uint32_t dst = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(dst)
               : "memory");
}

// Instruction schedule of one stage's fragment reads and MFMAs: kLead LDS
// reads, then after each group of FN MFMAs (one A fragment times the W
// fragments) one more read while any remain.  An A fragment is thus read
// kReadAhead groups before its MFMAs issue, so LDS latency hides behind them.
constexpr int kReadAhead = 3;
template <int GROUP, int NGROUPS, int EXTRA, int g = 0>
__device__ __forceinline__ void sched_stream() {
  if constexpr (g < NGROUPS) {
    __builtin_amdgcn_sched_group_barrier(0x008, GROUP, 0);  // MFMA
    if constexpr (g < EXTRA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    sched_stream<GROUP, NGROUPS, EXTRA, g + 1>();
  }
}

template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  return BK == 64 ? (chunk ^ (row & 7)) : (chunk ^ ((row >> 2) & 3));
}

// KG > 1 splits each k-step between KG groups of WM x WN waves (group g
// multiplies the g-th 32-wide slice of every stage): every wave keeps a large
// sub-tile, so fewer LDS bytes are read per MFMA, while the workgroup still
// holds two waves per SIMD.  The groups' partial tiles are summed through LDS
// at the end, each group finishing half of the row fragments.
template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int BK = 64, int KG = 1>
__global__ __launch_bounds__(64 * WM * WN * KG) void gemm_dma_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* __restrict__ W2,
    bf16* __restrict__ C, const bf16* __restrict__ R, float* __restrict__ part, int M, int Mp,
    int N, int K, int n_mtiles, int n_ntiles, int splits) {
  static_assert(BK == 64 || BK == 32, "stage depth");
  constexpr int ROWB = BK * 2;            // bytes of one tile row in a stage
  constexpr int BLK_ROWS = 1024 / ROWB;   // rows per 1 KB copy block
  constexpr int NCH = BK / 8;             // 16-byte chunks per row
  constexpr int NWG = WM * WN;  // waves per k-group
  constexpr int NW = NWG * KG;  // waves in the workgroup
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int OUT_N = EPI == EPI_SWIGLU ? BN / 2 : BN;
  constexpr int A_BLK = BM / BLK_ROWS, W_BLK = BN / BLK_ROWS;  // 1 KB blocks per stage
  constexpr int NBLK = A_BLK + W_BLK;
  // copy instructions per wave per stage: the first NBLK % NW waves take one more
  constexpr int PER_WAVE = (NBLK + NW - 1) / NW;
  constexpr int PER_WAVE_LO = NBLK / NW;
  constexpr int STAGE_BYTES = NBLK * 1024;
  static_assert(BM % BLK_ROWS == 0 && BN % BLK_ROWS == 0, "tiles are whole copy blocks");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole MFMA blocks");
  static_assert(EPI != EPI_SWIGLU || (FN % 2 == 0 && (BN / 2) % BLK_ROWS == 0), "swiglu pairing");
  static_assert(STAGES >= 3, "need at least three stages");
  static_assert(PER_WAVE * (STAGES - 2) < 64, "vmcnt range");
  static_assert(KG == 1 || KG == BK / 32, "a k-group takes one 32-wide slice of a stage");
  static_assert(KG == 1 || NWG * FM * FN * 1024 <= STAGES * STAGE_BYTES, "reduction fits the ring");

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int total = n_mtiles * n_ntiles * splits;
  const int b = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = b % 8, slot = b / 8;
  const int tile = xcd * per + min(xcd, rem) + slot;
  const int tm = tile % n_mtiles;
  const int rest = tile / n_mtiles;
  const int z = rest % splits;
  const int tn = rest / splits;
  const int m0 = tm * BM, n0 = tn * OUT_N;

  const int KT = K / BK;
  const int kt_per = (KT + splits - 1) / splits;
  const int kt0 = min(KT, z * kt_per);
  const int kt1 = min(KT, kt0 + kt_per);
  const int nk = kt1 - kt0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int kg = wave / NWG, wl = wave % NWG;
  const int wm = wl / WN, wn = wl % WN;
  const int l16 = lane & 15, q = lane >> 4;

  // per-lane source row pointers of this wave's copy blocks (k offset added per stage)
  const bf16* src[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int blk = min(wave + i * NW, NBLK - 1);
    const int row = blk * BLK_ROWS + lane / NCH;
    const int chunk = swz<BK>(row, lane % NCH);
    const bf16* p;
    if (blk < A_BLK) {
      const int m = min(m0 + row, Mp - 1);
      p = A + (size_t)m * K;
    } else {
      const int wr = row - BM;
      const bf16* base = W;
      int n;
      if (EPI == EPI_SWIGLU) {
        const bool up = wr >= BN / 2;
        base = up ? W2 : W;
        n = n0 + (up ? wr - BN / 2 : wr);
      } else {
        n = n0 + wr;
      }
      p = base + (size_t)min(n, N - 1) * K;
    }
    src[i] = p + chunk * 8;
  }
  auto issue = [&](int step) {  // copy k-step `step` (clamped) into its ring slot
    const int kt = kt0 + min(step, max(nk - 1, 0));
    char* st = smem + (step % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      if (wave + i * NW < NBLK) lds_copy16(src[i] + kt * BK, st + (wave + i * NW) * 1024);
  };
  const bool more = (NBLK % NW) != 0 && wave < NBLK % NW;  // this wave copies PER_WAVE blocks

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment byte offsets inside a stage (row-dependent swizzle)
  int a_off[FM], w_off[FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int row = wm * WTM + fm * 16 + l16;
    a_off[fm] = row * ROWB;
  }
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    int row;
    if (EPI == EPI_SWIGLU) {
      constexpr int HALF = FN / 2;
      row = fn < HALF ? wn * (WTN / 2) + fn * 16 : BN / 2 + wn * (WTN / 2) + (fn - HALF) * 16;
    } else {
      row = wn * WTN + fn * 16;
    }
    row += l16;
    w_off[fn] = (BM + row) * ROWB;
  }
  // fragment rows start at multiples of 16, so the swizzle depends on l16 only

  constexpr int NSUB = BK / 32 / KG;  // 32-wide sub-steps per wave per stage
  constexpr int kLead = NSUB * FN + kReadAhead < NSUB * (FN + FM) ? NSUB * FN + kReadAhead
                                                                  : NSUB * (FN + FM);
  // Kernel arguments read only after the loop arrive by scalar loads; such
  // loads may complete out of order with LDS reads, so while one is pending
  // every LDS wait in the loop would have to drain all reads.  Consume them
  // here so the loop's waits count LDS reads alone.
  asm volatile("" ::"s"(C), "s"(R), "s"(part), "s"(M), "s"(N));
  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s);
    for (int it = 0; it < nk; ++it) {
      if (PER_WAVE == PER_WAVE_LO || more)
        wait_vmcnt<PER_WAVE * (STAGES - 2)>();
      else
        wait_vmcnt<PER_WAVE_LO * (STAGES - 2)>();
      asm volatile("" ::: "memory");  // keep LDS reads and copies on their side of the barrier
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(it + STAGES - 1);
      const char* st = smem + (it % STAGES) * STAGE_BYTES;
      // W fragments of every sub-step first, then the A fragments in the
      // order the MFMA groups consume them; the schedule below keeps
      // kReadAhead A reads in flight ahead of the group that needs them
      bf16x8 af[NSUB][FN], bfr[NSUB][FM];
#pragma unroll
      for (int kk = 0; kk < NSUB; ++kk) {
        const int so = swz<BK>(l16, (kk * KG + kg) * 4 + q) << 4;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) af[kk][fn] = as_bf16x8(ld16(st + w_off[fn] + so));
      }
#pragma unroll
      for (int kk = 0; kk < NSUB; ++kk) {
        const int so = swz<BK>(l16, (kk * KG + kg) * 4 + q) << 4;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) bfr[kk][fm] = as_bf16x8(ld16(st + a_off[fm] + so));
      }
#pragma unroll
      for (int kk = 0; kk < NSUB; ++kk)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fn][fm] = mfma16x16x32(af[kk][fn], bfr[kk][fm], acc[fn][fm]);
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);  // LDS reads
      sched_stream<FN, NSUB * FM, NSUB * (FN + FM) - kLead>();
    }
  }
  wait_vmcnt<0>();  // drain the clamped tail copies before the workgroup ends
  // k-groups: group 0 finishes row fragments [0, FSPLIT), group 1 the rest;
  // each hands the other group's share to its partner wave through LDS
  constexpr int FSPLIT = (FM + 1) / 2;
  if (KG > 1) {
    __syncthreads();  // every wave is done with the ring and every copy has landed
    f32x4* red = reinterpret_cast<f32x4*>(smem) + (size_t)wl * FM * FN * 64;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if ((fm < FSPLIT) == (kg == 0)) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) red[(fm * FN + fn) * 64 + lane] = acc[fn][fm];
    }
    __syncthreads();
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if ((fm < FSPLIT) != (kg == 0)) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const f32x4 o = red[(fm * FN + fn) * 64 + lane];
        acc[fn][fm] += o;
      }
    }
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if (KG > 1 && (fm < FSPLIT) != (kg == 0)) continue;
    const int m = m0 + wm * WTM + fm * 16 + l16;
    if (splits > 1 && EPI == EPI_SWIGLU) {
      // split-K SwiGLU: gate and up partial sums side by side, [splits][Mp][2N]
      if (m >= Mp) continue;
      float* pp = part + ((size_t)z * Mp + m) * 2 * N;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const bool up = fn >= FN / 2;
        const int n = n0 + wn * (WTN / 2) + (up ? fn - FN / 2 : fn) * 16 + 4 * q;
        if (n < N) *reinterpret_cast<f32x4*>(pp + (up ? N : 0) + n) = acc[fn][fm];
      }
      continue;
    }
    if (splits > 1) {
      if (m >= Mp) continue;
      float* pp = part + (size_t)z * Mp * N + (size_t)m * N;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + wn * WTN + fn * 16 + 4 * q;
        if (n < N) *reinterpret_cast<f32x4*>(pp + n) = acc[fn][fm];
      }
      continue;
    }
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

template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int BK = 64, int KG = 1>
hipError_t run_gemm_dma(const bf16* a, const bf16* w, const bf16* w2, bf16* c, const bf16* r,
                        float* part, int m, int mp, int n, int k, int splits, hipStream_t s) {
  constexpr int OUT_N = EPI == EPI_SWIGLU ? BN / 2 : BN;
  constexpr size_t lds = (size_t)STAGES * (BM + BN) * BK * 2;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const int mt = (mp + BM - 1) / BM, nt = (n + OUT_N - 1) / OUT_N;
  auto kern = gemm_dma_kernel<BM, BN, WM, WN, EPI, STAGES, BK, KG>;
  // raise the dynamic LDS limit once per instantiation (thread-safe static init)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(mt * nt * splits), dim3(64 * WM * WN * KG), lds, s, a, w, w2, c, r, part,
                     m, mp, n, k, mt, nt, splits);
  return hipGetLastError();
}

}  // namespace hl

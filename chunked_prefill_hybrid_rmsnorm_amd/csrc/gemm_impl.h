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
// bank conflicts.  Copying wave w issues blocks w, w + NCW, ...  Rows past
// the end of A or W are clamped to the last valid row: their products only
// reach outputs that are never stored.
// 16-byte global -> LDS copy per lane, written as inline asm.  The compiler
// models its own form of this copy as an LDS access that may complete out of
// order with LDS reads, and then makes every LDS read in the loop wait for
// all reads before it; hidden from it, the reads get exact counts.
// Completion of the copies is tracked by hand with vmcnt waits and the
// workgroup barrier.  The address is a scalar base plus a per-lane 32-bit
// byte offset (the instruction's saddr form: one VGPR per copy instead of
// two).  `lds` is wave-uniform; M0 carries it.
__device__ __forceinline__ void lds_copy16(const bf16* base, uint32_t voff, char* lds) {
  const uint32_t dst = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(base), "s"(dst)
               : "memory", "m0");
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
//
// PP (ping-pong): the two waves that share a SIMD (wave w and w + NW/2) work
// half a k-step apart, so one reads fragments from LDS while the other keeps
// the SIMD's matrix pipe busy.  Each k-step has two workgroup barriers:
//   slot 1: first half copies stage it+2 and reads stage it; second half
//           multiplies stage it-1
//   slot 2: first half multiplies stage it and waits for its copies of stage
//           it+1; second half reads stage it
// Only the first half issues copies, so its own vmcnt waits plus the barrier
// cover every copy.  Every wave passes the same barriers (1 + 2 per k-step).
template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int BK = 64, int KG = 1,
          bool PP = false>
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
  constexpr int NCW = PP ? NW / 2 : NW;  // waves that issue copies
  // copy instructions per copying wave per stage: the first NBLK % NCW take one more
  constexpr int PER_WAVE = (NBLK + NCW - 1) / NCW;
  constexpr int PER_WAVE_LO = NBLK / NCW;
  constexpr int STAGE_BYTES = NBLK * 1024;
  static_assert(BM % BLK_ROWS == 0 && BN % BLK_ROWS == 0, "tiles are whole copy blocks");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole MFMA blocks");
  static_assert(EPI != EPI_SWIGLU || (FN % 2 == 0 && (BN / 2) % BLK_ROWS == 0), "swiglu pairing");
  // two stages: the copies of step it+1 go into the slot every wave finished
  // reading before the barrier of step it
  static_assert(STAGES >= 2, "need at least two stages");
  static_assert(PER_WAVE * (STAGES - 2) < 64, "vmcnt range");
  static_assert(!PP || (STAGES == 3 && NW % 2 == 0 && NBLK % NCW == 0),
                "ping-pong: three stages, equal copy shares");
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

  // Per-lane byte offsets of this wave's copy blocks from their matrix's base
  // (A, W or W2, uniform per block since a block never straddles two); the
  // k offset is added to the scalar base per stage.  32-bit offsets keep one
  // VGPR per block (matrices here are far below 4 GiB; the host checks).
  uint32_t voff[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int blk = min(wave + i * NCW, NBLK - 1);
    const int row = blk * BLK_ROWS + lane / NCH;
    const int chunk = swz<BK>(row, lane % NCH);
    size_t r;
    if (blk < A_BLK) {
      r = (size_t)min(m0 + row, Mp - 1);
    } else {
      const int wr = row - BM;
      const int n = EPI == EPI_SWIGLU && wr >= BN / 2 ? n0 + wr - BN / 2 : n0 + wr;
      r = (size_t)min(n, N - 1);
    }
    voff[i] = (uint32_t)((r * K + chunk * 8) * sizeof(bf16));
  }
  auto block_base = [&](int blk) -> const bf16* {  // wave-uniform
    if (blk < A_BLK) return A;
    if (EPI == EPI_SWIGLU && (blk - A_BLK) * BLK_ROWS >= BN / 2) return W2;
    return W;
  };
  auto issue = [&](int step) {  // copy k-step `step` (clamped) into its ring slot
    const int kt = kt0 + min(step, max(nk - 1, 0));
    char* st = smem + (step % STAGES) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int blk = wave + i * NCW;
      if (blk < NBLK) lds_copy16(block_base(blk) + (size_t)kt * BK, voff[i], st + blk * 1024);
    }
  };
  const bool more = (NBLK % NCW) != 0 && wave < NBLK % NCW;  // this wave copies PER_WAVE blocks

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
  if constexpr (PP) {
    // fragments live across the slot boundary (second half: across the k-step)
    bf16x8 af[NSUB][FN], bfr[NSUB][FM];
    const bool first = wave < NCW;
    auto read_frags = [&](const char* st) {
#pragma unroll
      for (int kk = 0; kk < NSUB; ++kk) {
        const int so = swz<BK>(l16, (kk * KG + kg) * 4 + q) << 4;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) af[kk][fn] = as_bf16x8(ld16(st + w_off[fn] + so));
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) bfr[kk][fm] = as_bf16x8(ld16(st + a_off[fm] + so));
      }
      // the reads must have landed before the barrier: the stage is
      // overwritten by copies issued after a later one
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    };
    auto multiply = [&]() {
#pragma unroll
      for (int kk = 0; kk < NSUB; ++kk)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fn][fm] = mfma16x16x32(af[kk][fn], bfr[kk][fm], acc[fn][fm]);
    };
    auto barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // the two halves run separate loops (clear register lifetimes), with the
    // same barrier count: 1 + 2 nk
    if (nk > 0 && first) {
      issue(0);
      issue(1);
      wait_vmcnt<PER_WAVE>();  // stage 0 landed
      barrier();
      for (int it = 0; it < nk; ++it) {
        issue(it + 2);  // into the slot of stage it-1, read by everyone before the last barrier
        read_frags(smem + (it % STAGES) * STAGE_BYTES);
        barrier();
        multiply();  // stage it
        __builtin_amdgcn_sched_barrier(0);  // every MFMA issues before the wait
        wait_vmcnt<PER_WAVE>();  // stage it+1 landed; stage it+2 may be in flight
        barrier();
      }
    } else if (nk > 0) {
      barrier();
      barrier();
      read_frags(smem);  // stage 0
      barrier();
      for (int it = 1; it < nk; ++it) {
        multiply();  // stage it-1
        barrier();
        read_frags(smem + (it % STAGES) * STAGE_BYTES);
        barrier();
      }
      multiply();  // stage nk-1
    }
  } else if (nk > 0) {
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

template <int BM, int BN, int WM, int WN, int EPI, int STAGES, int BK = 64, int KG = 1,
          bool PP = false>
hipError_t run_gemm_dma(const bf16* a, const bf16* w, const bf16* w2, bf16* c, const bf16* r,
                        float* part, int m, int mp, int n, int k, int splits, hipStream_t s) {
  constexpr int OUT_N = EPI == EPI_SWIGLU ? BN / 2 : BN;
  constexpr size_t lds = (size_t)STAGES * (BM + BN) * BK * 2;
  static_assert(lds <= 160 * 1024, "LDS budget");
  // the copies address A and W by 32-bit byte offsets
  if ((size_t)mp * k * sizeof(bf16) > UINT32_MAX || (size_t)n * k * sizeof(bf16) > UINT32_MAX)
    return hipErrorInvalidValue;
  const int mt = (mp + BM - 1) / BM, nt = (n + OUT_N - 1) / OUT_N;
  auto kern = gemm_dma_kernel<BM, BN, WM, WN, EPI, STAGES, BK, KG, PP>;
  // raise the dynamic LDS limit once per instantiation (thread-safe static init)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(mt * nt * splits), dim3(64 * WM * WN * KG), lds, s, a, w, w2, c, r, part,
                     m, mp, n, k, mt, nt, splits);
  return hipGetLastError();
}

}  // namespace hl

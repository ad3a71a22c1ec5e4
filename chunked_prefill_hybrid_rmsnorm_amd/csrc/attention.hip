// Attention of the hybrid batch: chunk-prefill rows and decode rows in one
// launch.  The pages' design runs FlashAttention on the prefill part and
// PagedAttention on the decode part as two kernels on two streams joined by
// an event; here one heterogeneous grid carries both, so the MFMA-heavy
// prefill workgroups and the HBM-bound decode workgroups share the GPU at the
// same time, and one merge kernel finishes the rows whose keys were split.
//
// Prefill: row i of a chunk (position start_pos + i) attends keys 0 ..
// start_pos + i of its request -- the KV earlier chunks left in the pages plus
// the chunk's own keys, causally -- through the chunk's block table.  Every
// chunk re-reads the KV of all earlier chunks, so a prompt prefilled in N
// chunks reads chunk KV N(N-1)/2 extra times; that cost stays visible.  GQA
// packing: the 16 rows of a wave are (token, q head) pairs of one kv head
// (row = token * G + head), so one K/V fragment serves all G heads; the 4
// waves of a workgroup cover 64 consecutive rows and walk the same keys.  With
// few row groups the key range is split into segments (more workgroups).
//
// Decode: the G query heads of kv head g are the tile rows, and every K and V
// byte of a context is read once.  The 32-key steps of all decodes, laid end
// to end in decode order, are cut into P equal slices per kv head, one wave
// each, so every decode wave carries the same number of bytes whatever the
// mix of context lengths (fixed per-decode partitions leave most waves of
// short contexts idle and load some compute units twice as much as others).
// A decode that falls inside one slice is finished by its wave; otherwise
// each slice leaves a partial result for the merge.
#include <atomic>
#include <type_traits>
#include <string.h>

#include "attn_common.h"

namespace hl {

// Waves per workgroup, a template parameter of the kernel: 8 (a prefill
// workgroup is two groups of four waves on the same rows) or 4 (one group).
constexpr int kPfHalfWaves = 4;  // waves of one prefill group
constexpr int kPfRowsPerWave = 32;                         // two 16-row MFMA blocks
constexpr int kPrefillRows = kPfRowsPerWave * kPfHalfWaves;  // rows per prefill workgroup
// LDS ring of prefill K/V: kPfStages slots, copies issued kPfAhead steps
// ahead of the step being opened.  A copy then lands in the slot of step t - 2,
// whose fragments every wave has used (not only read) before the barrier
// that opens step t, so the barrier needs no wait for outstanding LDS reads.
constexpr int kPfStages = 4;
constexpr int kPfAhead = 2;
constexpr bool kPfPipelined = true;  // prefill waves score the next step during this step's softmax
constexpr int kDecMinSliceSteps = 4;   // fewest 32-key steps in a decode slice
constexpr int kDecSlotsPerWave = 4;    // wave slots of the free workgroups per decode wave
constexpr int kDecMaxWaves = 4096;     // decode waves of one launch, all kv heads

struct AttnArgs {
  const bf16* qkv;
  bf16* attn;
  KvDev kv;
  int nq, nkv;
  // prefill
  ChunkList chunks;
  int pf_gx;   // row groups of the longest chunk
  int pf_ns;   // key segments (1: no split)
  int pf_seg;  // keys per segment
  int pf_wgs;  // prefill workgroups = pf_gx * pf_ns * nkv * chunks.n
  float* pf_o;
  float* pf_ml;
  // decode
  DecDev dec;
  int dc_row0;   // first decode row
  int dc_slices;  // slices per kv head the grid provides (upper bound of P)
  int dc_pn;      // partial slots per q head = dc_slices + n
  int dc_wgs;     // decode workgroups: min(free workgroups, dc_slices * nkv), >= units / NW
  float* dc_o;
  float* dc_ml;
  int merge_row0;  // first row the merge grid covers (chunk rows only when keys were split)
};

template <int D>
__device__ __forceinline__ void init_acc(AttnAcc<D>& a) {
  a.m = -INFINITY;
  a.l = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) a.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// K/V of one 32-key step staged in LDS for all waves of a prefill workgroup:
// [K page 0 | K page 1 | V page 0 | V page 1], each 16 x D bf16.  Within a K
// row the 16-byte chunks are permuted (chunk c at slot c ^ k_swz(row)) and
// within a V row of 16 keys the two 8-key halves are swapped when
// v_swz(dim) is set, so that every group of 8 lanes of a fragment read
// touches 8 different 16-byte bank groups.
template <int D>
struct PfStage {
  static constexpr int PAGE = 16 * D * 2;     // bytes of one page of one kv head
  static constexpr int BYTES = 4 * PAGE;      // K and V of two pages
  static constexpr int COPIES = BYTES / 1024;  // 1 KB copy instructions per step
  static constexpr int PER_WAVE = COPIES / kPfHalfWaves;  // copies per wave of one group
};

__device__ __forceinline__ int k_swz(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int v_swz(int dim) { return (dim >> 2) & 1; }

template <int D>
__device__ __forceinline__ void prefill_copy(char* stage, const KvDev& kv, int g, int p0, int p1,
                                             int wave, int lane) {
  constexpr int PAGE = PfStage<D>::PAGE;
#pragma unroll
  for (int i = 0; i < PfStage<D>::PER_WAVE; ++i) {
    const int ci = wave * PfStage<D>::PER_WAVE + i;  // 1 KB block of the stage
    const int off = ci * 1024;                        // byte offset in the stage
    const int region = off / PAGE;                    // 0, 1: K pages; 2, 3: V pages
    const int page = (region & 1) ? p1 : p0;
    const int in = off % PAGE + lane * 16;            // byte offset inside the page
    const bf16* src;
    if (region < 2) {
      const int row = in / (D * 2), slot = (in % (D * 2)) / 16;
      src = kv.k_page(page, g) + row * D + (slot ^ k_swz(row)) * 8;
    } else {
      const int dim = in / 32, half = (in % 32) / 16;
      src = kv.v_page(page, g) + dim * 16 + (half ^ v_swz(dim)) * 8;
    }
    lds_dma16(src, stage + off);  // lane i fills bytes [16 i, 16 i + 16) of the block
  }
}

template <int D>
__device__ __forceinline__ void prefill_frags_k(KvFrag<D>& f, const char* stage, int l16, int q) {
  constexpr int PAGE = PfStage<D>::PAGE;
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    const int key = step_key(hp, l16);
    const int row = key & 15;
    const char* kr = stage + (key >> 4) * PAGE + row * D * 2;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) f.k[hp][ks] = ld16(kr + (((ks * 4 + q) ^ k_swz(row)) * 16));
  }
}

template <int D>
__device__ __forceinline__ void prefill_frags_v(KvFrag<D>& f, const char* stage, int l16, int q) {
  constexpr int PAGE = PfStage<D>::PAGE;
  const char* vb = stage + (2 + (q >> 1)) * PAGE;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int dim = db * 16 + l16;
    f.v[db] = ld16(vb + dim * 32 + (((q & 1) ^ v_swz(dim)) * 16));
  }
}

template <int D>
__device__ __forceinline__ void prefill_frags(KvFrag<D>& f, const char* stage, int l16, int q) {
  prefill_frags_k<D>(f, stage, l16, q);
  prefill_frags_v<D>(f, stage, l16, q);
}

// Merge the (m, l, o) of the same rows over another key range into `a`
// (base-2 scaled maxima; a part with m = -inf has seen no key).
template <int D>
__device__ __forceinline__ void merge_acc(AttnAcc<D>& a, float m1, float l1, const f32x4* o1) {
  const float m = fmaxf(a.m, m1);
  if (m == -INFINITY) return;  // neither part has a key for this row
  const float f0 = a.m == -INFINITY ? 0.f : fast_exp2(a.m - m);
  const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - m);
  a.m = m;
  a.l = a.l * f0 + l1 * f1;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) a.o[i] = a.o[i] * f0 + o1[i] * f1;
}

// A prefill workgroup: 128 GQA rows (row = token * G + head) of one chunk and
// one kv head, 32 per wave as two 16-row MFMA blocks, over one key segment.
// With eight waves (NW = 8) they form two groups of four on the same rows:
// group 0 takes the first half of the segment's 32-key steps, group 1 the
// rest, so every SIMD holds two waves of the workgroup.  Each group copies
// its steps' K/V pages into its own LDS ring (global -> LDS, kPfStages deep)
// and reads them from there, so a K/V byte crosses the L2 -> CU path once per
// 128 rows.  At the end group 1 hands its (m, l, o) to group 0 through LDS,
// which merges and stores the rows.
template <int D, int NW>
__device__ __forceinline__ void prefill_block(const AttnArgs& A, int b, int wave_id, int lane,
                                              char* ring_all) {
  static_assert(NW == kPfHalfWaves || NW == 2 * kPfHalfWaves, "one or two wave groups");
  constexpr int NGROUPS = NW / kPfHalfWaves;
  const int l16 = lane & 15, q = lane >> 4;
  const int half = NGROUPS == 1 ? 0 : wave_id / kPfHalfWaves;  // the wave's group
  const int wave = wave_id % kPfHalfWaves;
  char* ring = ring_all + half * kPfStages * PfStage<D>::BYTES;
  const int per_chunk = A.pf_gx * A.pf_ns * A.nkv;
  const int c = b / per_chunk;
  const int rem = b % per_chunk;
  const int g = rem / (A.pf_gx * A.pf_ns);
  const int x = rem % (A.pf_gx * A.pf_ns);
  const int rg = x / A.pf_ns, sp = x % A.pf_ns;
  const ChunkDev ch = A.chunks.c[c];
  const int G = A.nq / A.nkv;
  const int rows_total = ch.len * G;
  const int wg_row0 = rg * kPrefillRows;
  if (wg_row0 >= rows_total) return;  // whole workgroup idle (uniform)
  const int kv_len = ch.start_pos + ch.len;
  const int wg_last = min(wg_row0 + kPrefillRows, rows_total) - 1;
  const int k_stop = ch.start_pos + wg_last / G + 1;
  const int k0 = sp * A.pf_seg;
  const int k1 = min(k_stop, k0 + A.pf_seg);
  if (k0 >= k1) return;  // no row of the workgroup reaches this segment (uniform)
  const int ld = (A.nq + 2 * A.nkv) * D;

  // this wave's two row blocks
  const int rbase = wg_row0 + wave * kPfRowsPerWave;
  bf16x8 qf[2][D / 32];
  int row_limit[2];
  bool valid[2];
  int tok[2], hh[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = rbase + rb * 16 + l16;
    valid[rb] = row < rows_total;
    tok[rb] = valid[rb] ? row / G : 0;
    hh[rb] = row % G;
    row_limit[rb] = valid[rb] ? ch.start_pos + tok[rb] : -1;
    const bf16* qp = A.qkv + (size_t)(ch.row0 + tok[rb]) * ld + (size_t)(g * G + hh[rb]) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[rb][ks] = valid[rb] ? as_bf16x8(ld16(qp + ks * 32 + q * 8))
                             : as_bf16x8(u32x4{0, 0, 0, 0});
  }
  const bool busy = rbase < rows_total;  // wave has rows (still copies and syncs if not)
  const int lim_min[2] = {wave_min(row_limit[0]), wave_min(row_limit[1])};

  const int blk_end = (k1 + 15) >> 4;
  const int nsteps = (k1 - k0 + 31) / 32;
  // the group's steps: [s0, s0 + my_n); group 0 takes the larger half, and
  // both groups run n_iter iterations (one barrier each)
  const int n_iter = (nsteps + NGROUPS - 1) / NGROUPS;
  const int s0 = half ? n_iter : 0;
  const int my_n = half ? nsteps - n_iter : n_iter;
  const int kg0 = k0 + s0 * 32;  // first key of the group
  PageWindow win;
  win.fill(ch.block_table, ch.n_blocks, kg0 >> 4, blk_end, A.kv.num_pages, lane);
  // keys from block blk_end on are read from a stand-in page: zero their V
  const int v_end = min(kv_len, blk_end * 16);
  // copies of the group's step i (pages past the table read page 0, whose
  // keys are masked); every wave of the group issues its share of the same
  // copies, and none past the group's last step
  auto issue = [&](int i) {
    const int t = kg0 + i * 32;
    int p0 = win.at(t, ch.block_table, ch.n_blocks, blk_end, A.kv.num_pages, lane);
    int p1 = win.at(t + 16, ch.block_table, ch.n_blocks, blk_end, A.kv.num_pages, lane);
    prefill_copy<D>(ring + (i % kPfStages) * PfStage<D>::BYTES, A.kv, g, max(p0, 0), max(p1, 0),
                    wave, lane);
  };

  AttnAcc<D> a[2];
  init_acc<D>(a[0]);
  init_acc<D>(a[1]);
  const float scale = kAttnLog2e * rsqrtf((float)D);
  static_assert(kPfAhead >= 1 && kPfAhead <= 3 && kPfStages >= kPfAhead + 1,
                "the waits below allow 0 .. 2 later steps in flight");
  for (int s = 0; s < kPfAhead; ++s)
    if (s < my_n) issue(s);
  if constexpr (kPfPipelined) {
    // Each wave runs one step ahead of its softmax: while step i's softmax
    // (VALU) and V product run, step i+1's K fragments are read and its
    // scores multiplied, so a wave keeps the matrix pipe and the vector ALU
    // busy together instead of in turn.  Stage t is waited for, and its
    // copies made visible by the barrier, before any of its fragments are
    // read; the copies issued after that barrier refill the slot of stage
    // t - 2, whose V fragments every wave consumed in the previous iteration
    // (with a ring one slot shorter it would be stage t - 1, whose V reads
    // may still be in flight, and the barrier would first wait for them).
    // Every wave passes my_n barriers, then one per step the other group has
    // beyond them.
    auto open_stage = [&](int t) {
      const int after = min(kPfAhead - 1, my_n - 1 - t);  // later stages that may be in flight
      if (after >= 2)
        wait_vmcnt<2 * PfStage<D>::PER_WAVE>();
      else if (after == 1)
        wait_vmcnt<PfStage<D>::PER_WAVE>();
      else
        wait_vmcnt<0>();
      if constexpr (kPfStages < kPfAhead + 2) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + kPfAhead < my_n) issue(t + kPfAhead);
    };
    KvFrag<D> fk, fv;  // K of the step being scored; V of the step being summed
    f32x4 sc[2][2];    // scores of the step whose softmax is next
    bf16x8 pf[2];
    if (my_n > 0) {
      open_stage(0);
      if (busy) {
        prefill_frags_k<D>(fk, ring, l16, q);
        prefill_frags_v<D>(fv, ring, l16, q);
        step_scores<D, 2>(sc, fk, qf);
      }
    }
    for (int i = 0; i + 1 < my_n; ++i) {
      open_stage(i + 1);
      if (!busy) continue;
      const char* st = ring + ((i + 1) % kPfStages) * PfStage<D>::BYTES;
      prefill_frags_k<D>(fk, st, l16, q);
      // step i's max and rescale while step i+1's K reads are in flight;
      // every step but the group's last ends below k1 <= v_end
      float m_use[2];
      step_softmax_head<D, 2, false>(a, sc, fv, m_use, kg0 + i * 32, row_limit, lim_min, k1,
                                     v_end, scale, q);
      // step i+1's scores (MFMA) interleaved with step i's exponentials
      // (VALU): one MFMA, then three vector instructions
      f32x4 sn[2][2];
      step_scores<D, 2>(sn, fk, qf);
      step_softmax_tail<D, 2>(a, sc, m_use, pf, scale);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      }
      step_pv<D, 2>(a, fv, pf);
      prefill_frags_v<D>(fv, st, l16, q);  // step i+1
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) sc[rb][hp] = sn[rb][hp];
    }
    if (my_n > 0 && busy) {  // the group's last step, V tail masked
      step_softmax<D, 2, true>(a, sc, fv, pf, kg0 + (my_n - 1) * 32, row_limit, lim_min, k1,
                               v_end, scale, q);
      step_pv<D, 2>(a, fv, pf);
    }
    for (int i = my_n; i < n_iter; ++i) __builtin_amdgcn_s_barrier();
  } else {
    // the group's own steps (the same loop shape as a single group, so that
    // `busy`, invariant, can take the whole loop apart), then a barrier for
    // each step the other group has beyond them (at most one).  Every step but
    // the group's last ends below k1 <= v_end, so only the last one (peeled
    // off the loop: one copy of the step code in the loop keeps the register
    // budget) may have V to mask.
    auto step = [&](int i, auto last) {
      // this step's copies have landed; those of up to kPfAhead - 1 later
      // steps may still be in flight
      const int ahead = min(kPfAhead - 1, my_n - 1 - i);
      if (ahead >= 2)
        wait_vmcnt<2 * PfStage<D>::PER_WAVE>();
      else if (ahead == 1)
        wait_vmcnt<PfStage<D>::PER_WAVE>();
      else
        wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // into the slot of step i + kPfAhead - kPfStages, which every wave
      // finished reading before this barrier
      if (i + kPfAhead < my_n) issue(i + kPfAhead);
      if (!busy) return;
      KvFrag<D> f;
      prefill_frags<D>(f, ring + (i % kPfStages) * PfStage<D>::BYTES, l16, q);
      const int t0 = kg0 + i * 32;
      compute_step<D, 2, decltype(last)::value>(a, f, qf, t0, row_limit, lim_min, k1, v_end, scale,
                                                q);
    };
    int i = 0;
    for (; i + 1 < my_n; ++i) step(i, std::false_type{});
    if (my_n > 0) step(i++, std::true_type{});
    for (; i < n_iter; ++i) __builtin_amdgcn_s_barrier();
  }
  // group 1 hands its rows' (m, l, o) to group 0 through the rings' LDS:
  // per wave and row block, D/4 + 2 floats per lane, lane-minor
  constexpr int XF = D / 4 + 2;
  static_assert(NGROUPS == 1 || kPfHalfWaves * 2 * XF * 64 * 4 <= 2 * kPfStages * PfStage<D>::BYTES,
                "exchange fits the rings");
  float* xbuf = reinterpret_cast<float*>(ring_all) + (size_t)wave * 2 * XF * 64;
  if (NGROUPS == 2) __syncthreads();  // every wave is done with both rings
  if (NGROUPS == 2 && half == 1 && busy) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float* xr = xbuf + rb * XF * 64;
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) xr[(i * 4 + r) * 64 + lane] = a[rb].o[i][r];
      xr[(D / 4) * 64 + lane] = a[rb].m;
      xr[(D / 4 + 1) * 64 + lane] = a[rb].l;
    }
  }
  if (NGROUPS == 2) __syncthreads();
  if (half == 1 || !busy) return;
#pragma unroll
  for (int rb = 0; rb < 2 && NGROUPS == 2; ++rb) {
    const float* xr = xbuf + rb * XF * 64;
    f32x4 o1[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) o1[i][r] = xr[(i * 4 + r) * 64 + lane];
    merge_acc<D>(a[rb], xr[(D / 4) * 64 + lane], xr[(D / 4 + 1) * 64 + lane], o1);
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l_tot = row_total(a[rb].l);
    if (!valid[rb]) continue;
    const int h = g * G + hh[rb];
    const int n_parts = min(A.pf_ns, (row_limit[rb] + A.pf_seg) / A.pf_seg);
    if (sp >= n_parts) continue;  // this row has no key in the segment
    const int grow = ch.row0 + tok[rb];
    if (n_parts == 1) {
      store_row<D>(a[rb], l_tot, A.attn + (size_t)grow * A.nq * D + (size_t)h * D, q);
      continue;
    }
    const size_t pidx = ((size_t)grow * A.nq + h) * A.pf_ns + sp;
    store_partial<D>(a[rb], l_tot, A.pf_o + pidx * D, A.pf_ml + pidx * 2, q);
  }
}

// Split of the decode steps.  Slice s of P covers concatenated steps
// [floor(s S / P), floor((s + 1) S / P)); with P <= S no slice is empty.
struct DecodeSplit {
  int S;  // 32-key steps of all decodes
  int P;  // slices in use
};
__device__ __forceinline__ int decode_steps(int ctx) { return (ctx + 32) >> 5; }  // ceil((ctx+1)/32)
__device__ __forceinline__ int slice_begin(int s, const DecodeSplit& d) {
  return (int)((long long)s * d.S / d.P);
}
// the slice holding step t: the last s with slice_begin(s) <= t
__device__ __forceinline__ int slice_of(int t, const DecodeSplit& d) {
  return (int)(((long long)(t + 1) * d.P - 1) / d.S);
}
// P = min(max_slices, S / kDecMinSliceSteps) for S steps in all
__device__ __forceinline__ DecodeSplit split_of(int S, int max_slices) {
  DecodeSplit d;
  d.S = S;
  d.P = max(1, min(max_slices, S / kDecMinSliceSteps));
  return d;
}
// S from the context lengths (one wave); the attention waves and the merge
// compute it alike
__device__ __forceinline__ DecodeSplit decode_split(const DecDev& dec, int max_slices, int lane) {
  int S = 0;
  for (int c0 = 0; c0 < dec.n; c0 += 64) {
    const int j = c0 + lane;
    const int st = j < dec.n ? decode_steps(dec.ctx_lens[j]) : 0;
    S += __builtin_amdgcn_readlane(wave_incl_scan(st, lane), 63);
  }
  return split_of(S, max_slices);
}

// Steps [t0, t1) of decode j (first step cj, nj steps) for kv head g; the
// result goes to the output row when slice s holds the whole decode, else to
// partial slot s + j (consecutive pieces of a kv head raise s, j or both, so
// the slot is distinct for every piece).
template <int D>
__device__ __forceinline__ void decode_piece(const AttnArgs& A, const DecodeSplit& sp, int s,
                                             int j, int g, int ctx, int cj, int nj, int t0, int t1,
                                             int l16, int q) {
  const int G = A.nq / A.nkv;
  const int row = A.dc_row0 + j;
  const int ld = (A.nq + 2 * A.nkv) * D;
  const bf16* qrow = A.qkv + (size_t)row * ld + (size_t)(g * G) * D;
  bf16x8 qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = l16 < G ? as_bf16x8(ld16(qrow + l16 * D + ks * 32 + q * 8))
                     : as_bf16x8(u32x4{0, 0, 0, 0});
  AttnAcc<D> a;
  init_acc<D>(a);
  const int k0 = (t0 - cj) * 32, k1 = min((t1 - cj) * 32, ctx + 1);
  const int32_t* bt = A.dec.block_tables + (size_t)j * A.dec.max_blocks;
  // one block-table window (64 blocks) per call
  for (int kk = k0; kk < k1; kk += 64 * 16)
    attend_segment<D>(a, qf, ctx, kk, min(k1, kk + 64 * 16), ctx + 1, bt, A.dec.max_blocks, A.kv,
                      g, l16, q);
  const float l_tot = row_total(a.l);
  if (l16 < G) {
    const int h = g * G + l16;
    if (slice_of(cj, sp) == slice_of(cj + nj - 1, sp)) {
      store_row<D>(a, l_tot, A.attn + (size_t)row * A.nq * D + (size_t)h * D, q);
    } else {
      const size_t pidx = (size_t)h * A.dc_pn + s + j;
      store_partial<D>(a, l_tot, A.dc_o + pidx * D, A.dc_ml + pidx * 2, q);
    }
  }
}

// Work unit u = s * nkv + g (slice s, kv head g).  A workgroup's waves take
// consecutive units, so they share slices (the same pages).  When the context
// lengths give fewer slices than the grid has decode waves, every workgroup
// takes fewer units, so the busy waves spread over all decode workgroups (and
// compute units) instead of filling the first ones.
template <int D, int NW>
__device__ __forceinline__ void decode_wave(const AttnArgs& A, int wg, int wave, int lane,
                                            int l16, int q) {
  const DecodeSplit sp = decode_split(A.dec, A.dc_slices, lane);
  const int units = sp.P * A.nkv;
  const int per_wg = min(NW, (units + A.dc_wgs - 1) / A.dc_wgs);
  if (wave >= per_wg) return;
  const int unit = wg * per_wg + wave;
  if (unit >= units) return;
  const int g = unit % A.nkv;
  const int s = unit / A.nkv;
  const int b0 = slice_begin(s, sp), b1 = slice_begin(s + 1, sp);
  int base = 0;  // steps of the decodes before this group of 64
  for (int c0 = 0; c0 < A.dec.n && base < b1; c0 += 64) {
    const int j = c0 + lane;
    const int ctx = j < A.dec.n ? A.dec.ctx_lens[j] : 0;
    const int st = j < A.dec.n ? decode_steps(ctx) : 0;
    const int incl = base + wave_incl_scan(st, lane);
    const int excl = incl - st;
    uint64_t m = __ballot(st > 0 && incl > b0 && excl < b1);  // decodes overlapping the slice
    while (m) {
      const int i = __builtin_ctzll(m);
      m &= m - 1;
      const int cj = __builtin_amdgcn_readlane(excl, i);
      const int nj = __builtin_amdgcn_readlane(st, i);
      decode_piece<D>(A, sp, s, c0 + i, g, __builtin_amdgcn_readlane(ctx, i), cj, nj,
                      max(cj, b0), min(cj + nj, b1), l16, q);
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
}

// Register budget: two waves per SIMD in either shape (the four-wave
// workgroups ask for two resident workgroups per CU), so that a SIMD can
// interleave a second wave's MFMAs, softmax or loads with the first's
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attention_kernel(AttnArgs A) {
  __shared__ __attribute__((aligned(1024)))
  char ring[NW / kPfHalfWaves * kPfStages * PfStage<D>::BYTES];
  // the wave index is uniform across the wave: keep it (and everything derived
  // from it: work unit, key range, loop bounds) in scalar registers, so that
  // the loops branch on scalars instead of masking lanes
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int b = blockIdx.x;
  if (b < A.pf_wgs) {
    // Workgroup ids are dealt round-robin over the 8 XCDs, each with its own
    // L2.  Prefill units are numbered kv head by kv head; XCD x takes a
    // contiguous run of them, so with 8 kv heads all row groups of one head
    // share one L2, which then fetches that head's keys once instead of
    // every XCD fetching every head's keys.
    const int per = A.pf_wgs / 8, rem = A.pf_wgs % 8, xcd = b % 8;
    prefill_block<D, NW>(A, xcd * per + min(xcd, rem) + b / 8, wave, lane, ring);
  } else
    decode_wave<D, NW>(A, b - A.pf_wgs, wave, lane, l16, q);
}

// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over the parts of one
// (row, head), stored consecutively from `base`; lane i takes dims D/64 i ...
// Up to 32 parts: lane p loads the (m, l) of part p while every lane loads its
// dims of all parts, in one round, and each part's weight is computed once,
// by its lane, and read from there.  More parts are loaded 8 at a time
// (indices clamped to the last part) in two passes.  Either way the parts are
// summed in part order with the same weights.
template <int D>
__device__ __forceinline__ void merge_unit(const float* __restrict__ o_part,
                                           const float* __restrict__ ml_part, size_t base,
                                           int n_parts, bf16* __restrict__ orow) {
  constexpr int PER = D / 64;
  // n_parts is uniform over the block, so the guards are scalar branches
  constexpr int ONE = 32;
  const int lane = threadIdx.x;
  if (n_parts <= ONE) {
    float mv = -INFINITY, lv = 0.f, ov[ONE][PER];
    if (lane < n_parts) {
      mv = ml_part[(base + lane) * 2];
      lv = ml_part[(base + lane) * 2 + 1];
    }
#pragma unroll
    for (int u = 0; u < ONE; ++u) {
      if (u < n_parts) {
#pragma unroll
        for (int i = 0; i < PER; ++i) ov[u][i] = o_part[(base + u) * D + lane * PER + i];
      }
    }
    const float mmax = wave_max(mv);
    const float wl = mv == -INFINITY ? 0.f : exp2f(mv - mmax);
    float o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < ONE; ++u) {
      if (u >= n_parts) continue;
      // no visible key in this part
      if (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), u)) == -INFINITY) continue;
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
      lsum += w * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), u));
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] += w * ov[u][i];
    }
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < PER; ++i) orow[lane * PER + i] = f2bf(o[i] * inv);
    return;
  }
  constexpr int U = 8;
  float mmax = -INFINITY;
  for (int p0 = 0; p0 < n_parts; p0 += U) {
    float mv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) mv[u] = ml_part[(base + min(p0 + u, n_parts - 1)) * 2];
#pragma unroll
    for (int u = 0; u < U; ++u) mmax = fmaxf(mmax, mv[u]);
  }
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  float lsum = 0.f;
  for (int p0 = 0; p0 < n_parts; p0 += U) {
    float mv[U], lv[U], ov[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t pi = base + min(p0 + u, n_parts - 1);
      mv[u] = ml_part[pi * 2];
      lv[u] = ml_part[pi * 2 + 1];
#pragma unroll
      for (int i = 0; i < PER; ++i) ov[u][i] = o_part[pi * D + threadIdx.x * PER + i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // past the last part, or no visible key in this part
      if (p0 + u >= n_parts || mv[u] == -INFINITY) continue;
      const float w = exp2f(mv[u] - mmax);
      lsum += w * lv[u];
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] += w * ov[u][i];
    }
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[threadIdx.x * PER + i] = f2bf(o[i] * inv);
}

// One 64-thread block per (row, q head), rows being the chunk rows and then
// the decodes: many small independent blocks, so that their load latencies
// overlap.  Rows whose keys were not split were written by the attention
// kernel.
template <int D>
__global__ __launch_bounds__(64) void attention_merge_kernel(AttnArgs A) {
  const int h = blockIdx.x, r = A.merge_row0 + blockIdx.y;
  bf16* orow = A.attn;
  if (r < A.chunks.n_rows) {
    if (A.pf_ns <= 1) return;
    int c = 0;
    while (c + 1 < A.chunks.n && r >= A.chunks.c[c + 1].row0) ++c;
    const int pos = A.chunks.c[c].start_pos + (r - A.chunks.c[c].row0);
    const int n_parts = min(A.pf_ns, (pos + A.pf_seg) / A.pf_seg);
    if (n_parts <= 1) return;
    orow += (size_t)r * A.nq * D + (size_t)h * D;
    merge_unit<D>(A.pf_o, A.pf_ml, ((size_t)r * A.nq + h) * A.pf_ns, n_parts, orow);
  } else {
    const int j = r - A.chunks.n_rows;
    if (j >= A.dec.n) return;
    const int lane = threadIdx.x;
    // one pass over the context lengths: the steps of all decodes (the
    // split), of the decodes before j (cj) and of decode j (nj)
    int S = 0, cj = 0, nj = 0;
    for (int c0 = 0; c0 < A.dec.n; c0 += 64) {
      const int i = c0 + lane;
      const int st = i < A.dec.n ? decode_steps(A.dec.ctx_lens[i]) : 0;
      const int incl = wave_incl_scan(st, lane);
      if (j >= c0 && j < c0 + 64) {
        cj = S + __builtin_amdgcn_readlane(incl - st, j - c0);
        nj = __builtin_amdgcn_readlane(st, j - c0);
      }
      S += __builtin_amdgcn_readlane(incl, 63);
    }
    const DecodeSplit sp = split_of(S, A.dc_slices);
    const int s_lo = slice_of(cj, sp);
    const int s_hi = slice_of(cj + nj - 1, sp);
    if (s_lo == s_hi) return;
    orow += (size_t)(A.dc_row0 + j) * A.nq * D + (size_t)h * D;
    merge_unit<D>(A.dc_o, A.dc_ml, (size_t)h * A.dc_pn + s_lo + j, s_hi - s_lo + 1, orow);
  }
}

// ---------------------------------------------------------------- host side
// Prefill key split over workgroups: only when the chunk rows give few
// workgroups, into segments of >= 256 keys (multiples of 32).  Prefill alone
// aims at ~256 workgroups, one per CU (split below 128), each splitting its
// segment once more between its two wave groups.  Beside decodes it aims at
// 64 (split below 64): there the decode waves set the kernel time, every
// prefill workgroup takes a slot a decode wave group could use, and every
// split adds partials for the merge to read.
constexpr int kPfAimAlone = 256, kPfAimHybrid = 64;
// 128-row groups (over all kv heads) from which a chunk beside decodes runs
// in four-wave workgroups
constexpr int kPfFourWaveFrom = 256;
// segment length of a chunk of few row groups over a long cached prefix
constexpr int kPfFewSeg = 512;

// prefill workgroups before any key split (128-row groups over all kv heads)
// and the longest key range of the chunks
static void chunk_extent(const ChunkList& chunks, int nq, int nkv, int* base, int* max_keys) {
  const int G = nq / nkv;
  *base = 0;
  *max_keys = 0;
  for (int i = 0; i < chunks.n; ++i) {
    *base += (chunks.c[i].len * G + kPrefillRows - 1) / kPrefillRows * nkv;
    *max_keys = max(*max_keys, chunks.c[i].start_pos + chunks.c[i].len);
  }
}

// Beside decodes, a chunk of few row groups over a long cached prefix (a
// tensor-parallel share: one or two kv heads) runs in four-wave workgroups
// and walks its keys in segments of at most kPfFewSeg, up to ~256
// workgroups, so that each CU holds one prefill and one decode workgroup:
// Mistral-7B-shaped T=4 share 125.6 -> 120.6 us per layer; Llama-2-70B-shaped
// T=8 share: attention 30.4 -> 28.8 us, its merge 7.8 -> 8.6 us (before:
// eight-wave workgroups in 1024-key segments, themselves 60.3 -> 37.6 us over
// no split).  Short key ranges keep the eight-wave layout, which runs a chunk
// the same way beside decodes as alone.
static bool few_groups_long_keys(int base, int max_keys, bool with_decodes) {
  return with_decodes && base > 0 && base < kPfAimAlone / 4 && max_keys > kPfFewSeg;
}

void prefill_split(const ChunkList& chunks, int nq, int nkv, bool with_decodes, int* nsplit,
                   int* seg) {
  int base, max_keys;
  chunk_extent(chunks, nq, nkv, &base, &max_keys);
  int ns = 1;
  const int aim = with_decodes ? kPfAimHybrid : kPfAimAlone;
  const int below = with_decodes ? kPfAimHybrid : kPfAimAlone / 2;
  if (base > 0 && base < below) ns = min((aim + base - 1) / base, max(1, max_keys / 256));
  if (few_groups_long_keys(base, max_keys, with_decodes))
    ns = max(ns, min((max_keys + kPfFewSeg - 1) / kPfFewSeg, (kPfAimAlone + base - 1) / base));
  ns = max(ns, 1);
  int sg = (max_keys + ns - 1) / ns;
  sg = (sg + 31) / 32 * 32;
  if (sg <= 0) sg = 32;
  *seg = sg;
  *nsplit = max(1, (max_keys + sg - 1) / sg);
}

// Upper bound of the prefill partials over every chunk layout with at most
// `rows` chunk rows (any start positions), with or without decodes: the split
// count is at most ceil(kPfAimAlone / base) with base >= ceil(r G /
// kPrefillRows) nkv workgroups for r rows.
size_t prefill_workspace_bound(int rows, int nq, int nkv, int d) {
  const int G = nq / nkv;
  size_t worst = 0;
  for (int r = 1; r <= rows; ++r) {
    const int base = (r * G + kPrefillRows - 1) / kPrefillRows * nkv;
    if (base >= kPfAimAlone / 2) continue;
    const size_t ns = (kPfAimAlone + base - 1) / base;
    worst = max(worst, ns * (size_t)r);
  }
  return worst ? worst * nq * (d + 2) * sizeof(float) + 256 : 0;
}

size_t prefill_workspace_bytes(const ChunkList& chunks, int nq, int nkv, int d) {
  int ns, sg;
  prefill_split(chunks, nq, nkv, false, &ns, &sg);
  if (ns <= 1) return 0;
  return (size_t)ns * chunks.n_rows * nq * (d + 2) * sizeof(float) + 256;
}

// Most decode slices per kv head a launch can use: bounded by the wave budget
// and by the steps n decodes of at most max_ctx + 1 keys can have.
static int decode_slice_cap(int n, int nkv, int max_ctx) {
  const long long steps = (long long)n * ((max_ctx + 32) / 32);
  return (int)max(1LL, min((long long)(kDecMaxWaves / nkv), steps / kDecMinSliceSteps));
}

size_t decode_workspace_bytes(int n_decodes, int nq, int nkv, int d, int max_ctx) {
  const size_t pn = (size_t)decode_slice_cap(n_decodes, nkv, max_ctx) + n_decodes;
  return (size_t)nq * pn * (d + 2) * sizeof(float) + 256;
}

// Workgroups of attention_kernel<D, NW> the device holds at once, cached per
// device.  Host threads may race to fill an entry; each computes the same
// value, and the atomic makes the store and the loads well defined.
template <int D, int NW>
static int attention_slots() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::atomic<int>& slot = cache[dev];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    const hipError_t e =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attention_kernel<D, NW>, 64 * NW, 0);
    if (e != hipSuccess || per_cu <= 0) per_cu = 1;
    c = max(1, cus * per_cu);
    slot.store(c, std::memory_order_relaxed);
  }
  return c;
}

// One launch of attention_kernel<D, NW> and, when keys were split, the merge.
template <int D, int NW>
static hipError_t run_attention(AttnArgs& A, void* pf_ws, void* dc_ws, hipStream_t s,
                                hipEvent_t mid) {
  const ChunkList& chunks = A.chunks;
  const DecDev& dec = A.dec;
  const int nq = A.nq, nkv = A.nkv;
  if (chunks.n > 0 && chunks.n_rows > 0) {
    const int G = nq / nkv;
    int max_len = 0;
    for (int i = 0; i < chunks.n; ++i) max_len = max(max_len, chunks.c[i].len);
    A.pf_gx = (max_len * G + kPrefillRows - 1) / kPrefillRows;
    A.pf_ns = 1;
    A.pf_seg = 1 << 30;
    if (pf_ws) {
      prefill_split(chunks, nq, nkv, dec.n > 0, &A.pf_ns, &A.pf_seg);
      if (A.pf_ns <= 1) {
        A.pf_ns = 1;
        A.pf_seg = 1 << 30;
      }
    }
    A.pf_wgs = A.pf_gx * A.pf_ns * nkv * chunks.n;
    A.pf_o = reinterpret_cast<float*>(pf_ws);
    A.pf_ml = A.pf_ns > 1 ? A.pf_o + (size_t)A.pf_ns * chunks.n_rows * nq * D : nullptr;
  }
  if (dec.n > 0) {
    // decode workgroups take the slots the prefill part leaves free (at least
    // a quarter of them), so that both kinds run side by side, with one busy
    // decode wave per kDecSlotsPerWave wave slots: fewer, longer slices than
    // one per slot keep HBM as busy with fewer loads queued in each CU's
    // memory path (where the prefill copies wait behind them) and fewer
    // partials to merge.  The busy waves spread evenly over the workgroups.
    const int slots = attention_slots<D, NW>();
    const int free_wgs = max(slots - A.pf_wgs, slots / 4);
    A.dc_slices = max(1, min(free_wgs * NW / (kDecSlotsPerWave * nkv),
                             decode_slice_cap(dec.n, nkv, dec.max_ctx)));
    A.dc_pn = A.dc_slices + dec.n;
    // at most NW units per workgroup, however many kv heads a single slice
    // per head gives (the second term only binds past ~free_wgs * NW heads)
    A.dc_wgs = max(min(free_wgs, A.dc_slices * nkv), (A.dc_slices * nkv + NW - 1) / NW);
    A.dc_o = reinterpret_cast<float*>(dc_ws);
    A.dc_ml = A.dc_o + (size_t)nq * A.dc_pn * D;
  }
  const int wgs = A.pf_wgs + A.dc_wgs;
  if (wgs == 0) return mid ? hipEventRecord(mid, s) : hipSuccess;
  // chunk rows need the merge only when their keys were split; decode rows
  // whenever there is more than one slice
  A.merge_row0 = A.pf_ns > 1 ? 0 : chunks.n_rows;
  const int merge_rows = chunks.n_rows + dec.n - A.merge_row0;
  const bool merge = (A.pf_ns > 1 || A.dc_slices > 1) && merge_rows > 0;
  hipLaunchKernelGGL((attention_kernel<D, NW>), dim3(wgs), dim3(64 * NW), 0, s, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
  if (!merge) return hipSuccess;
  hipLaunchKernelGGL(attention_merge_kernel<D>, dim3(nq, merge_rows), dim3(64), 0, s, A);
  return hipGetLastError();
}

hipError_t launch_attention(const bf16* qkv, int nq, int nkv, int d, const ChunkList& chunks,
                            const DecDev& dec, int dec_row0, const KvDev& kv, bf16* attn,
                            void* pf_ws, void* dc_ws, hipStream_t s, hipEvent_t mid) {
  AttnArgs A;
  memset(&A, 0, sizeof(A));
  A.qkv = qkv;
  A.attn = attn;
  A.kv = kv;
  A.nq = nq;
  A.nkv = nkv;
  A.chunks = chunks;
  A.dec = dec;
  A.dc_row0 = dec_row0;
  // Eight-wave workgroups split each chunk row group's keys between two wave
  // groups.  Beside decodes, a chunk whose row groups alone fill half of the
  // four-wave workgroup slots keeps four-wave workgroups instead: every CU
  // then holds a prefill and a decode workgroup (MFMA-bound and HBM-bound
  // waves side by side), where eight-wave prefill workgroups would take
  // every slot and leave the decodes waiting.  So does a chunk of few row
  // groups over a long cached prefix, whose keys are then split into about
  // one segment per CU.
  int base, max_keys;
  chunk_extent(chunks, nq, nkv, &base, &max_keys);
  const bool four = (dec.n > 0 && base >= kPfFourWaveFrom) ||
                    few_groups_long_keys(base, max_keys, dec.n > 0);
  if (d == 128)
    return four ? run_attention<128, 4>(A, pf_ws, dc_ws, s, mid)
                : run_attention<128, 8>(A, pf_ws, dc_ws, s, mid);
  return four ? run_attention<64, 4>(A, pf_ws, dc_ws, s, mid)
              : run_attention<64, 8>(A, pf_ws, dc_ws, s, mid);
}

hipError_t launch_prefill_attention(const bf16* qkv, int nq, int nkv, int d,
                                    const ChunkList& chunks, const KvDev& kv, bf16* attn,
                                    void* ws, hipStream_t s) {
  DecDev none{};
  return launch_attention(qkv, nq, nkv, d, chunks, none, 0, kv, attn, ws, nullptr, s);
}

hipError_t launch_decode_attention(const bf16* qkv, int row0, int nq, int nkv, int d,
                                   const DecDev& dec, const KvDev& kv, bf16* attn, void* ws,
                                   hipStream_t s) {
  ChunkList none;
  memset(&none, 0, sizeof(none));
  return launch_attention(qkv, nq, nkv, d, none, dec, row0, kv, attn, nullptr, ws, s);
}

}  // namespace hl

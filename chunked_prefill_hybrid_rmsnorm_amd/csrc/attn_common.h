// One wave's walk over a segment of a request's paged KV, shared by the
// chunk-prefill and the decode attention kernels.
//
// The wave owns 16 query rows (the columns of the MFMA tile): for decode the
// G query heads of one token, for prefill (token, head) pairs of one kv head.
//   S^T[key][row] = K[key][:] . q[row][:]          A = K rows (token-major page)
//   O^T[dim][row] += V^T[dim][key] P^T[key][row]   A = V^T (dim-major page)
// Lane l holds row l % 16 of every tile, so the probabilities it computes
// are exactly the B operand it feeds to the second product.  Softmax is
// online in base 2.  Keys are visited 32 at a time (two pages); page ids come
// from a register window of the block table and the next step's K/V
// fragments are loaded while the current step is multiplied.
//
// Key order inside a 32-key step: S^T is computed as two 16-row blocks hp,
// and row r of block hp holds key kappa(hp, r) = 8 (r / 4) + 4 hp + r % 4.  Lane
// (l16, q) then receives keys 8q .. 8q + 7 (four from each block), which are
// 8 consecutive keys of one page: its P values are the B operand of the second
// product in key order, and its V^T operand is one 16-byte piece of the page.
#pragma once
#include "kernels.h"

namespace hl {

constexpr float kAttnLog2e = 1.4426950408889634f;

// key (0..31 inside the step) held by S^T row r of block hp
__device__ __forceinline__ int step_key(int hp, int r) { return 8 * (r >> 2) + 4 * hp + (r & 3); }

// max / sum over the four lanes l16, l16 + 16, l16 + 32, l16 + 48 (one row)
//
// The max of two swapped halves is one v_max_f32 written out: through
// fmaxf the compiler cannot tell that bits coming back from a permlane are a
// canonical float and first passes each operand through another max with
// itself (two extra vector instructions per swap, four per row block and
// step).  A plain VALU instruction with register operands; no memory access.
__device__ __forceinline__ float max_bits(uint32_t a, uint32_t b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float quad_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_bits(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_bits(b[0], b[1]);
}
__device__ __forceinline__ float quad_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x with the hardware instruction (results below 2^-126 flush to 0, which
// only drops probabilities that cannot change an fp32 sum)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct AttnAcc {
  f32x4 o[D / 16];  // O^T[16 db + 4q + r][row], unnormalised
  float m, l;       // running max (base-2 scaled score) and partial sum of this lane
};

template <int D>
struct KvFrag {
  u32x4 k[2][D / 32];  // K rows of keys kappa(hp, l16), 16 B per lane per k-step
  u32x4 v[D / 16];     // V^T of keys 8q .. 8q + 7 for dims 16 db + l16
};

// Step fragments straight from the pages (decode).  A missing page (-1, past
// the block table or the segment) reads page 0 instead: its keys are past
// the segment end, so their scores are masked, and their V is zeroed through
// v_end (see attend_segment).  Nothing here looks at the loaded values, so
// the loads stay in flight while the previous step is multiplied.
template <int D>
__device__ __forceinline__ void load_step(KvFrag<D>& f, const KvDev& kv, int g, int p0, int p1,
                                          int l16, int q) {
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    const int key = step_key(hp, l16);
    const int pg = key < 16 ? p0 : p1;
    const bf16* kp = kv.k_page(max(pg, 0), g) + (key & 15) * D + q * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) f.k[hp][ks] = ld16(kp + ks * 32);
  }
  // V: every instruction reads whole lines (512 contiguous bytes per page)
  // that nothing reads again, so the loads are non-temporal.  K stays
  // ordinary: each of its lines is read in two halves by consecutive loads.
  const int pv = q < 2 ? p0 : p1;
  const bf16* vp = kv.v_page(max(pv, 0), g) + (q & 1) * 8 + l16 * 16;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    f.v[db] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + db * 256));
}

// Largest growth of the running max (base-2 units) that is not folded into
// the accumulators at once: while a new max stays within kRescaleSlack of the
// one in use, probabilities are taken against the old max (they stay below
// 2^kRescaleSlack, exact in fp32 and bf16 range) and the O / l rescale is
// skipped.  The final o / l does not depend on which max was used.
constexpr float kRescaleSlack = 8.f;

// Multiply one 32-key step starting at t0 for NRB 16-row blocks sharing the
// step's K/V fragments.  Key t counts for a lane's row iff t <= row_limit
// (causal / context bound) and t < k_end (segment end); keys >= v_end have no
// valid V (past the request, or a stand-in page) and are zeroed before the
// product.  `lim_min[rb]` is the smallest row_limit over the wave's rows of
// block rb: a step below it and below v_end needs no masking at all.
//
// The step runs in three phases, which the ping-pong prefill loop places in
// different halves of its schedule: the scores (MFMA), the online softmax
// (VALU), and the probability-weighted V sum (MFMA).
//
// VMASK = false: the caller knows every key of the step is below v_end (all
// steps but a segment's last), so no V mask is formed.  The mask is a
// compile-time choice because the compiler turns a runtime test of it into
// selects on every V register of every step.
template <int D, int NRB>
__device__ __forceinline__ void step_scores(f32x4 (&s)[NRB][2], const KvFrag<D>& f,
                                            const bf16x8 (&qf)[NRB][D / 32]) {
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      s[rb][hp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        s[rb][hp] = mfma16x16x32(as_bf16x8(f.k[hp][ks]), qf[rb][ks], s[rb][hp]);
    }
}

// Zero V of the step's keys at or past v_end (a request's last page read
// past its end, or a stand-in page), whose probabilities are 0 but whose
// bytes are arbitrary.  Wave-uniform test.
template <int D>
__device__ __forceinline__ void mask_v_tail(KvFrag<D>& f, int t0, int v_end, int q) {
  if (t0 + 31 < v_end) return;
#pragma unroll
  for (int w = 0; w < 4; ++w) {  // keep-masks of this lane's V keys t0 + 8q + 2w, + 1
    const int t = t0 + 8 * q + 2 * w;
    const uint32_t vm = (t < v_end ? 0x0000ffffu : 0u) | (t + 1 < v_end ? 0xffff0000u : 0u);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) f.v[db][w] &= vm;
  }
}

// Online softmax of one step, in two parts.  The head masks the scores of
// keys a row may not see and moves the running max (rescaling o and l); it
// returns the shift each row's exponents use.  The tail (straight-line
// code, which a caller can interleave with independent MFMAs) forms the
// step's probabilities, adds them to l and packs them as the B operand of
// the V product.  With VMASK, V of keys at or past v_end is zeroed in place.
template <int D, int NRB, bool VMASK>
__device__ __forceinline__ void step_softmax_head(AttnAcc<D> (&a)[NRB], f32x4 (&s)[NRB][2],
                                                  KvFrag<D>& f, float (&m_use)[NRB], int t0,
                                                  const int (&row_limit)[NRB],
                                                  const int (&lim_min)[NRB], int k_end,
                                                  int v_end, float scale, int q) {
  if (VMASK) mask_v_tail<D>(f, t0, v_end, q);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    AttnAcc<D>& acc = a[rb];
    const bool full = t0 + 31 <= min(lim_min[rb], k_end - 1);  // wave-uniform
    // the scale (> 0) is applied once to the row maximum and inside the
    // exponent's fma below, not to every score
    float smax = -INFINITY;
    if (full) {
#pragma unroll
      for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int r = 0; r < 4; ++r) smax = fmaxf(smax, s[rb][hp][r]);
    } else {
      const int lim = min(row_limit[rb], k_end - 1);
#pragma unroll
      for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 8 * q + 4 * hp + r;
          s[rb][hp][r] = t <= lim ? s[rb][hp][r] : -INFINITY;
          smax = fmaxf(smax, s[rb][hp][r]);
        }
    }
    smax = quad_max(smax) * scale;
    // move the max in use only when the new one is well above it; a row with
    // no visible key so far keeps m = -inf and uses 0 as its shift, so that
    // no -inf - -inf appears (its probabilities are exactly 0)
    const bool grow = smax > acc.m + kRescaleSlack;
    if (__any(grow)) {
      const float m_next = grow ? smax : acc.m;
      const float alpha = grow ? fast_exp2(acc.m - m_next) : 1.f;  // 2^-inf = 0 on the first key
      acc.m = m_next;
      acc.l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) acc.o[db] *= alpha;
    }
    m_use[rb] = acc.m == -INFINITY ? 0.f : acc.m;
  }
}

template <int D, int NRB>
__device__ __forceinline__ void step_softmax_tail(AttnAcc<D> (&a)[NRB], const f32x4 (&s)[NRB][2],
                                                  const float (&m_use)[NRB], bf16x8 (&pf)[NRB],
                                                  float scale) {
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(__builtin_fmaf(s[rb][hp][r], scale, -m_use[rb]));
        psum += p[r];
      }
      pk[hp * 2 + 0] = pack2(p[0], p[1]);
      pk[hp * 2 + 1] = pack2(p[2], p[3]);
    }
    a[rb].l += psum;
    pf[rb] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
  }
}

template <int D, int NRB, bool VMASK>
__device__ __forceinline__ void step_softmax(AttnAcc<D> (&a)[NRB], f32x4 (&s)[NRB][2],
                                             KvFrag<D>& f, bf16x8 (&pf)[NRB], int t0,
                                             const int (&row_limit)[NRB],
                                             const int (&lim_min)[NRB], int k_end, int v_end,
                                             float scale, int q) {
  float m_use[NRB];
  step_softmax_head<D, NRB, VMASK>(a, s, f, m_use, t0, row_limit, lim_min, k_end, v_end, scale, q);
  step_softmax_tail<D, NRB>(a, s, m_use, pf, scale);
}

template <int D, int NRB>
__device__ __forceinline__ void step_pv(AttnAcc<D> (&a)[NRB], const KvFrag<D>& f,
                                        const bf16x8 (&pf)[NRB]) {
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      a[rb].o[db] = mfma16x16x32(as_bf16x8(f.v[db]), pf[rb], a[rb].o[db]);
}

template <int D, int NRB, bool VMASK = true>
__device__ __forceinline__ void compute_step(AttnAcc<D> (&a)[NRB], const KvFrag<D>& fin,
                                             const bf16x8 (&qf)[NRB][D / 32], int t0,
                                             const int (&row_limit)[NRB],
                                             const int (&lim_min)[NRB], int k_end, int v_end,
                                             float scale, int q) {
  KvFrag<D> f = fin;
  f32x4 s[NRB][2];
  bf16x8 pf[NRB];
  step_scores<D, NRB>(s, f, qf);
  step_softmax<D, NRB, VMASK>(a, s, f, pf, t0, row_limit, lim_min, k_end, v_end, scale, q);
  step_pv<D, NRB>(a, f, pf);
}

// Smallest value of v over the wave.
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// A wave's window of 64 consecutive block-table entries (lane i holds the page
// of block base + i, or -1 past the table, the segment or the pool), so that
// a step's page ids are a register read instead of a dependent global load.
struct PageWindow {
  int base = -(1 << 30);
  int page = -1;
  __device__ __forceinline__ void fill(const int32_t* bt, int n_blocks, int blk0, int blk_end,
                                       int num_pages, int lane) {
    base = blk0;
    const int b = blk0 + lane;
    int pg = -1;
    if (b < n_blocks && b < blk_end) pg = bt[b];
    page = (pg >= 0 && pg < num_pages) ? pg : -1;
  }
  // page of key t (uniform across the wave), refilling the window when needed
  __device__ __forceinline__ int at(int t, const int32_t* bt, int n_blocks, int blk_end,
                                    int num_pages, int lane) {
    const int b = t >> 4;
    if (b >= blk_end) return -1;
    if (b - base >= 64 || b < base) fill(bt, n_blocks, b, blk_end, num_pages, lane);
    return __builtin_amdgcn_readlane(page, b - base);
  }
};

// Keys [k0, k1) of one decode (k0 a multiple of 32, at most 64 blocks, so one
// block-table window covers them) through its block table.  Every step loads
// its fragments one step ahead.  The loop body always issues exactly two
// steps' loads and the last one or two steps are peeled off, so the count of
// loads in flight is the same on every path: the wait before a multiply
// covers only the loads of that step, and no load goes past the last step.
template <int D>
__device__ __forceinline__ void attend_segment(AttnAcc<D>& a, const bf16x8 (&qf)[D / 32],
                                               int row_limit, int k0, int k1, int kv_len,
                                               const int32_t* bt, int n_blocks, const KvDev& kv,
                                               int g, int l16, int q) {
  const float scale = kAttnLog2e * rsqrtf((float)D);
  if (k0 >= k1) return;
  const int lane = l16 + 16 * q;
  const int blk0 = k0 >> 4, blk_end = (k1 + 15) >> 4;
  PageWindow win;
  win.fill(bt, n_blocks, blk0, blk_end, kv.num_pages, lane);
  const int nst = (k1 - k0 + 31) / 32;
  auto load = [&](KvFrag<D>& f, int st) {
    const int b = blk0 + 2 * st;
    const int p0 = b < blk_end ? __builtin_amdgcn_readlane(win.page, b - blk0) : -1;
    const int p1 = b + 1 < blk_end ? __builtin_amdgcn_readlane(win.page, b + 1 - blk0) : -1;
    load_step<D>(f, kv, g, p0, p1, l16, q);
  };
  AttnAcc<D> ab[1] = {a};
  bf16x8 qb[1][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qb[0][ks] = qf[ks];
  const int rl[1] = {row_limit};
  const int lm[1] = {wave_min(row_limit)};
  // keys from block blk_end on come from a stand-in page: zero their V
  const int v_end = min(kv_len, blk_end * 16);
  // every step but the last ends below k1 <= v_end: only the last masks V
  KvFrag<D> fa, fb;
  load(fa, 0);
  int i = 0;
  for (; i + 2 < nst; i += 2) {
    load(fb, i + 1);
    compute_step<D, 1, false>(ab, fa, qb, k0 + 32 * i, rl, lm, k1, v_end, scale, q);
    load(fa, i + 2);
    compute_step<D, 1, false>(ab, fb, qb, k0 + 32 * (i + 1), rl, lm, k1, v_end, scale, q);
  }
  if (i + 1 < nst) {  // two steps left, the first already loaded
    load(fb, i + 1);
    compute_step<D, 1, false>(ab, fa, qb, k0 + 32 * i, rl, lm, k1, v_end, scale, q);
    compute_step<D, 1>(ab, fb, qb, k0 + 32 * (i + 1), rl, lm, k1, v_end, scale, q);
  } else {
    compute_step<D, 1>(ab, fa, qb, k0 + 32 * i, rl, lm, k1, v_end, scale, q);
  }
  a = ab[0];
}

// Sum of l over the four lanes holding one row.
__device__ __forceinline__ float row_total(float l) { return quad_sum(l); }

// Final bf16 output of one row: lane writes dims 16 db + 4q .. + 4.
template <int D>
__device__ __forceinline__ void store_row(const AttnAcc<D>& a, float l_tot, bf16* orow, int q) {
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    u32x2 o;
    o[0] = pack2(a.o[db][0] * inv, a.o[db][1] * inv);
    o[1] = pack2(a.o[db][2] * inv, a.o[db][3] * inv);
    *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * q) = o;
  }
}

// Partial result of one row for a later merge: o (unnormalised), m, l.
template <int D>
__device__ __forceinline__ void store_partial(const AttnAcc<D>& a, float l_tot, float* op,
                                              float* mlp, int q) {
#pragma unroll
  for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(op + db * 16 + 4 * q) = a.o[db];
  if (q == 0) {
    mlp[0] = a.m;
    mlp[1] = l_tot;
  }
}

}  // namespace hl

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
#pragma once
#include "kernels.h"

namespace hl {

constexpr float kAttnLog2e = 1.4426950408889634f;

template <int D>
struct AttnAcc {
  f32x4 o[D / 16];  // O^T[16 db + 4q + r][row], unnormalised
  float m, l;       // running max (base-2 scaled score) and partial sum of this lane
};

template <int D>
struct KvFrag {
  u32x4 k[2][D / 32];  // two pages, K rows (16 B per lane per k-step)
  u32x2 v[2][D / 16];  // two pages, V^T pieces (8 B per lane per dim block)
};

template <int D>
__device__ __forceinline__ void load_step(KvFrag<D>& f, const KvDev& kv, int g, int p0, int p1,
                                          int l16, int q) {
  const int pg[2] = {p0, p1};
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    const bf16* kp = pg[hp] >= 0 ? kv.k_page(pg[hp], g) : nullptr;
    const bf16* vp = pg[hp] >= 0 ? kv.v_page(pg[hp], g) : nullptr;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      f.k[hp][ks] = kp ? ld16(kp + l16 * D + ks * 32 + q * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      f.v[hp][db] = vp ? ld8(vp + (db * 16 + l16) * 16 + 4 * q) : u32x2{0, 0};
  }
}

// Multiply one 32-key step starting at t0.  Key t counts for this lane's row
// iff t <= row_limit (causal / context bound) and t < k_end (segment end);
// keys >= kv_len hold no token, so their V is zeroed before the product.
template <int D>
__device__ __forceinline__ void compute_step(AttnAcc<D>& a, const KvFrag<D>& f,
                                             const bf16x8 (&qf)[D / 32], int t0, int row_limit,
                                             int k_end, int kv_len, float scale, int q) {
  const int lim = min(row_limit, k_end - 1);
  f32x4 s[2];
  float smax = -INFINITY;
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    s[hp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) s[hp] = mfma16x16x32(as_bf16x8(f.k[hp][ks]), qf[ks], s[hp]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + hp * 16 + 4 * q + r;
      s[hp][r] = t <= lim ? s[hp][r] * scale : -INFINITY;
      smax = fmaxf(smax, s[hp][r]);
    }
  }
  smax = fmaxf(smax, __shfl_xor(smax, 16));
  smax = fmaxf(smax, __shfl_xor(smax, 32));
  const float m_new = fmaxf(a.m, smax);
  // a row with no visible key so far keeps m = -inf: use 0 as the shift so
  // that no -inf - -inf appears; its probabilities are exactly 0
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2f(a.m - m_use);
  a.m = m_new;
  float psum = 0.f;
  uint32_t pk[4];
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = exp2f(s[hp][r] - m_use);
      psum += p[r];
    }
    pk[hp * 2 + 0] = pack2(p[0], p[1]);
    pk[hp * 2 + 1] = pack2(p[2], p[3]);
  }
  a.l = a.l * alpha + psum;
  const bf16x8 pf = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
  uint32_t vm[2][2];
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    const int t = t0 + hp * 16 + 4 * q;
    vm[hp][0] = (t + 0 < kv_len ? 0x0000ffffu : 0u) | (t + 1 < kv_len ? 0xffff0000u : 0u);
    vm[hp][1] = (t + 2 < kv_len ? 0x0000ffffu : 0u) | (t + 3 < kv_len ? 0xffff0000u : 0u);
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    a.o[db] *= alpha;
    const u32x4 va = {f.v[0][db][0] & vm[0][0], f.v[0][db][1] & vm[0][1],
                      f.v[1][db][0] & vm[1][0], f.v[1][db][1] & vm[1][1]};
    a.o[db] = mfma16x16x32(as_bf16x8(va), pf, a.o[db]);
  }
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

// Keys [k0, k1) (k0 a multiple of 32) of one request through its block table.
template <int D>
__device__ __forceinline__ void attend_segment(AttnAcc<D>& a, const bf16x8 (&qf)[D / 32],
                                               int row_limit, int k0, int k1, int kv_len,
                                               const int32_t* bt, int n_blocks, const KvDev& kv,
                                               int g, int l16, int q) {
  const float scale = kAttnLog2e * rsqrtf((float)D);
  if (k0 >= k1) return;
  const int lane = l16 + 16 * q;
  const int blk_end = (k1 + 15) >> 4;
  PageWindow win;
  win.fill(bt, n_blocks, k0 >> 4, blk_end, kv.num_pages, lane);
  auto pages = [&](int t, int& p0, int& p1) {
    p0 = win.at(t, bt, n_blocks, blk_end, kv.num_pages, lane);
    p1 = win.at(t + 16, bt, n_blocks, blk_end, kv.num_pages, lane);
  };
  KvFrag<D> fa, fb;
  int p0, p1;
  pages(k0, p0, p1);
  load_step<D>(fa, kv, g, p0, p1, l16, q);
  int t0 = k0;
  while (true) {
    // fa holds step t0; fetch t0 + 32 into fb, then multiply fa
    const int t1 = t0 + 32;
    if (t1 < k1) {
      pages(t1, p0, p1);
      load_step<D>(fb, kv, g, p0, p1, l16, q);
    }
    compute_step<D>(a, fa, qf, t0, row_limit, k1, kv_len, scale, q);
    if (t1 >= k1) break;
    const int t2 = t1 + 32;
    if (t2 < k1) {
      pages(t2, p0, p1);
      load_step<D>(fa, kv, g, p0, p1, l16, q);
    }
    compute_step<D>(a, fb, qf, t1, row_limit, k1, kv_len, scale, q);
    if (t2 >= k1) break;
    t0 = t2;
  }
}

// Sum of l over the four lanes holding one row.
__device__ __forceinline__ float row_total(float l) {
  l += __shfl_xor(l, 16);
  return l + __shfl_xor(l, 32);
}

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

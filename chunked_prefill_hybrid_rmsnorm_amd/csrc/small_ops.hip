// Row metadata, RMSNorm and RoPE + KV append: the HBM-bound small steps of
// the hybrid-batch layer.
#include <string.h>

#include <cmath>

#include "kernels.h"

namespace hl {

// ----------------------------------------------------------------- slots
// Row r < n_rows of the chunks: position start_pos + (r - row0) of its chunk;
// decode row j: position ctx_lens[j].  Slot = page * page_size + offset with
// page = block_table[pos / page_size] (PagedAttention addressing); -1 when the
// table or the page id is out of range.
__device__ __forceinline__ void row_pos_slot(const ChunkList& chunks, const DecDev& dec,
                                             int page_size, int num_pages, int r, int* pos_out,
                                             int* slot_out) {
  int pos, blk, page = -1;
  if (r < chunks.n_rows) {
    int c = 0;
    while (c + 1 < chunks.n && r >= chunks.c[c + 1].row0) ++c;
    pos = chunks.c[c].start_pos + (r - chunks.c[c].row0);
    blk = pos / page_size;
    if (blk < chunks.c[c].n_blocks) page = chunks.c[c].block_table[blk];
  } else {
    const int j = r - chunks.n_rows;
    pos = dec.ctx_lens[j];
    blk = pos / page_size;
    if (blk >= 0 && blk < dec.max_blocks) page = dec.block_tables[(size_t)j * dec.max_blocks + blk];
  }
  *pos_out = pos;
  *slot_out = (page >= 0 && page < num_pages) ? page * page_size + pos % page_size : -1;
}

__global__ void slot_map_kernel(ChunkList chunks, DecDev dec, int page_size, int num_pages,
                                int32_t* __restrict__ pos_out, int32_t* __restrict__ slot_out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= chunks.n_rows + dec.n) return;
  int pos, slot;
  row_pos_slot(chunks, dec, page_size, num_pages, r, &pos, &slot);
  pos_out[r] = pos;
  slot_out[r] = slot;
}

hipError_t launch_slot_map(const ChunkList& chunks, const DecDev& dec, int page_size,
                           int num_pages, int32_t* pos, int32_t* slot, hipStream_t s) {
  const int total = chunks.n_rows + dec.n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_map_kernel, dim3((total + 255) / 256), dim3(256), 0, s, chunks, dec,
                     page_size, num_pages, pos, slot);
  return hipGetLastError();
}

// ----------------------------------------------------------------- RMSNorm
// One wave per row, four rows per workgroup; the row stays in registers
// between the sum of squares and the scaling (one global read).  hidden is a
// multiple of 64 and at most 64 * 8 * kNormMaxChunks.
constexpr int kNormRowsPerBlock = 4;
constexpr int kNormMaxChunks = 32;  // 16-byte chunks per lane: hidden <= 16384

// One row per wave, in two halves so that a caller can put other work
// between issuing the loads and using them: the row and the gain vector are
// loaded together (one memory round trip), then reduced, scaled and stored.
template <int CH>
struct NormRow {
  u32x4 v[CH], g[CH];
};

template <int CH>
__device__ __forceinline__ void rmsnorm_load(NormRow<CH>& n, const bf16* __restrict__ xr,
                                             const bf16* __restrict__ g, int hidden, int lane) {
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = (i * 64 + lane) * 8;
    n.v[i] = c < hidden ? ld16(xr + c) : u32x4{0, 0, 0, 0};
    n.g[i] = c < hidden ? ld16(g + c) : u32x4{0, 0, 0, 0};
  }
}

template <int CH>
__device__ __forceinline__ void rmsnorm_finish(const NormRow<CH>& n, bf16* __restrict__ yr,
                                               int hidden, float eps, int lane) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __uint_as_float(n.v[i][e] << 16), b = __uint_as_float(n.v[i][e] & 0xffff0000u);
      ss += a * a + b * b;
    }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)hidden + eps);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = (i * 64 + lane) * 8;
    if (c >= hidden) continue;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __uint_as_float(n.v[i][e] << 16) * inv * __uint_as_float(n.g[i][e] << 16);
      const float b = __uint_as_float(n.v[i][e] & 0xffff0000u) * inv *
                      __uint_as_float(n.g[i][e] & 0xffff0000u);
      o[e] = pack2(a, b);
    }
    *reinterpret_cast<u32x4*>(yr + c) = o;
  }
}

template <int CH>
__device__ __forceinline__ void rmsnorm_row(const bf16* __restrict__ xr, const bf16* __restrict__ g,
                                            bf16* __restrict__ yr, int hidden, float eps, int lane) {
  NormRow<CH> n;
  rmsnorm_load<CH>(n, xr, g, hidden, lane);
  rmsnorm_finish<CH>(n, yr, hidden, eps, lane);
}

template <int CH>
__global__ __launch_bounds__(64 * kNormRowsPerBlock) void rmsnorm_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ g, bf16* __restrict__ y, int rows,
    int rows_padded, int hidden, float eps) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kNormRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= rows_padded) return;
  bf16* yr = y + (size_t)r * hidden;
  if (r >= rows) {  // padding row: zero dummy token
    for (int c = lane * 8; c < hidden; c += 64 * 8) *reinterpret_cast<u32x4*>(yr + c) = u32x4{0, 0, 0, 0};
    return;
  }
  rmsnorm_row<CH>(x + (size_t)r * hidden, g, yr, hidden, eps, lane);
}

template <int CH>
static void launch_norm(const bf16* x, const bf16* g, bf16* y, int rows, int rows_padded,
                        int hidden, float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel<CH>,
                     dim3((rows_padded + kNormRowsPerBlock - 1) / kNormRowsPerBlock),
                     dim3(64 * kNormRowsPerBlock), 0, s, x, g, y, rows, rows_padded, hidden, eps);
}

hipError_t launch_rmsnorm(const bf16* x, const bf16* g, bf16* y, int rows, int rows_padded,
                          int hidden, float eps, hipStream_t s) {
  if (rows_padded == 0) return hipSuccess;
  const int ch = (hidden + 511) / 512;  // 16-byte chunks per lane
  if (ch <= 1) launch_norm<1>(x, g, y, rows, rows_padded, hidden, eps, s);
  else if (ch <= 2) launch_norm<2>(x, g, y, rows, rows_padded, hidden, eps, s);
  else if (ch <= 4) launch_norm<4>(x, g, y, rows, rows_padded, hidden, eps, s);
  else if (ch <= 8) launch_norm<8>(x, g, y, rows, rows_padded, hidden, eps, s);
  else if (ch <= 16) launch_norm<16>(x, g, y, rows, rows_padded, hidden, eps, s);
  else if (ch <= kNormMaxChunks) launch_norm<kNormMaxChunks>(x, g, y, rows, rows_padded, hidden, eps, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ----------------------------------------------------------------- RoPE + append
// One workgroup per row.  Pair i turns by pos * theta^(-2i/d): the row's d/2
// angles are formed and reduced modulo 2*pi in fp64 (positions up to millions
// keep full precision), their cos/sin taken once in fp32 and shared by every
// head through LDS.  A thread then takes 8 consecutive pairs of one head:
// 16-byte loads of u[i .. i+8) and u[i+d/2 .. i+d/2+8).
// Rotated q and k go back into qkv; K and V go to the row's KV slot (V
// dimension-major inside the page).
//
// cos / sin of pos * inv_freq: the angle is formed and reduced to [0, 2 pi)
// in fp64, the functions are taken in fp32
__device__ __forceinline__ void rope_cos_sin(int pos, double inv_freq, float* c, float* sn) {
  const double two_pi = 6.283185307179586476925, inv_two_pi = 0.15915494309189533576888;
  double ang = (double)pos * inv_freq;
  ang -= two_pi * floor(ang * inv_two_pi);
  sincosf((float)ang, sn, c);
}

// theta^(-2 i / d) for the d / 2 rotation pairs, in fp64 (host side)
static RopeFreq rope_freq(int d, float theta) {
  RopeFreq f;
  for (int i = 0; i < kRopeMaxPairs; ++i)
    f.inv[i] = i < d / 2 ? std::exp2(-2.0 * i / d * std::log2((double)theta)) : 0.0;
  return f;
}

__global__ __launch_bounds__(256) void rope_kv_append_kernel(
    bf16* __restrict__ qkv, const int32_t* __restrict__ pos_in, const int32_t* __restrict__ slot_in,
    ChunkList chunks, DecDev dec, int nq, int nkv, int d, RopeFreq freq, KvDev kv) {
  const int r = blockIdx.x;
  const int half = d >> 1;
  const int groups = half / 8;  // 8-pair groups per head
  const int ld = (nq + 2 * nkv) * d;
  bf16* row = qkv + (size_t)r * ld;
  int pos, slot;
  if (pos_in) {
    pos = pos_in[r];
    slot = slot_in[r];
  } else {
    row_pos_slot(chunks, dec, kv.page_size, kv.num_pages, r, &pos, &slot);
  }
  // a slot outside the pool (negative, or a page id >= num_pages) writes no KV
  const bool in_pool = slot >= 0 && slot / kv.page_size < kv.num_pages;
  const int page = in_pool ? slot / kv.page_size : -1;
  const int off = in_pool ? slot % kv.page_size : 0;
  __shared__ float cs_tab[64], sn_tab[64];  // d/2 <= 64
  if (threadIdx.x < half)
    rope_cos_sin(pos, freq.inv[threadIdx.x], &cs_tab[threadIdx.x], &sn_tab[threadIdx.x]);
  __syncthreads();
  for (int t = threadIdx.x; t < (nq + nkv) * groups; t += blockDim.x) {
    const int h = t / groups, i0 = (t % groups) * 8;
    bf16* u = row + h * d;
    const u32x4 av = ld16(u + i0), bv = ld16(u + i0 + half);
    float a[8], b[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] = __uint_as_float(av[e] << 16);
      a[2 * e + 1] = __uint_as_float(av[e] & 0xffff0000u);
      b[2 * e] = __uint_as_float(bv[e] << 16);
      b[2 * e + 1] = __uint_as_float(bv[e] & 0xffff0000u);
    }
    float ra[8], rb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float cs = cs_tab[i0 + e], sn = sn_tab[i0 + e];
      ra[e] = a[e] * cs - b[e] * sn;
      rb[e] = a[e] * sn + b[e] * cs;
    }
    u32x4 oa, ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      oa[e] = pack2(ra[2 * e], ra[2 * e + 1]);
      ob[e] = pack2(rb[2 * e], rb[2 * e + 1]);
    }
    *reinterpret_cast<u32x4*>(u + i0) = oa;
    *reinterpret_cast<u32x4*>(u + i0 + half) = ob;
    if (h >= nq && page >= 0) {
      bf16* kp = kv.k_page(page, h - nq) + (size_t)off * d;
      *reinterpret_cast<u32x4*>(kp + i0) = oa;
      *reinterpret_cast<u32x4*>(kp + i0 + half) = ob;
    }
  }
  if (page >= 0) {
    const bf16* v = row + (nq + nkv) * d;
    for (int e = threadIdx.x; e < nkv * d; e += blockDim.x) {
      const int g = e / d, dd = e % d;
      kv.v_page(page, g)[(size_t)dd * kv.page_size + off] = v[e];
    }
  }
}

hipError_t launch_rope_kv_append(bf16* qkv, const int32_t* pos, const int32_t* slot, int rows,
                                 int nq, int nkv, int d, float theta, const KvDev& kv,
                                 hipStream_t s) {
  if (rows == 0) return hipSuccess;
  ChunkList none_c;
  memset(&none_c, 0, sizeof(none_c));
  DecDev none_d{};
  if (d / 2 > kRopeMaxPairs) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_kv_append_kernel, dim3(rows), dim3(256), 0, s, qkv, pos, slot, none_c,
                     none_d, nq, nkv, d, rope_freq(d, theta), kv);
  return hipGetLastError();
}

// ---------------------------------------------------- layer path: table + wide append
// The first RMSNorm kernel also resolves every row's position and KV slot and
// tabulates its RoPE cos / sin, so the append kernel that follows the QKV
// projection is pure element-wise work spread over (row, 4 heads) groups.
template <int CH>
__global__ __launch_bounds__(64 * kNormRowsPerBlock) void rmsnorm_rope_table_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ g, bf16* __restrict__ y, int rows,
    int rows_padded, int hidden, float eps, ChunkList chunks, DecDev dec, int page_size,
    int num_pages, int d, RopeFreq freq, RopeTab tab) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kNormRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= rows_padded) return;
  bf16* yr = y + (size_t)r * hidden;
  if (r >= rows) {  // padding row: zero dummy token
    for (int c = lane * 8; c < hidden; c += 64 * 8) *reinterpret_cast<u32x4*>(yr + c) = u32x4{0, 0, 0, 0};
    return;
  }
  // the row's loads go out first; the table is worked out while they are in flight
  NormRow<CH> n;
  rmsnorm_load<CH>(n, x + (size_t)r * hidden, g, hidden, lane);
  int pos, slot;
  row_pos_slot(chunks, dec, page_size, num_pages, r, &pos, &slot);
  if (lane == 0) {
    tab.pos[r] = pos;
    tab.slot[r] = slot;
  }
  const int half = d >> 1;
  if (lane < half)
    rope_cos_sin(pos, freq.inv[lane], tab.cs + (size_t)r * half + lane,
                 tab.sn + (size_t)r * half + lane);
  rmsnorm_finish<CH>(n, yr, hidden, eps, lane);
}

hipError_t launch_rmsnorm_rope_table(const bf16* x, const bf16* g, bf16* y, int rows,
                                     int rows_padded, int hidden, float eps,
                                     const ChunkList& chunks, const DecDev& dec, const KvDev& kv,
                                     int d, float theta, const RopeTab& tab, hipStream_t s) {
  if (rows_padded == 0) return hipSuccess;
  if (d / 2 > kRopeMaxPairs) return hipErrorInvalidValue;
  const RopeFreq freq = rope_freq(d, theta);
  const dim3 grid((rows_padded + kNormRowsPerBlock - 1) / kNormRowsPerBlock);
  const dim3 block(64 * kNormRowsPerBlock);
#define HL_LAUNCH_TAB(CH_)                                                                    \
  hipLaunchKernelGGL(rmsnorm_rope_table_kernel<CH_>, grid, block, 0, s, x, g, y, rows,        \
                     rows_padded, hidden, eps, chunks, dec, kv.page_size, kv.num_pages, d,   \
                     freq, tab)
  const int ch = (hidden + 511) / 512;  // 16-byte chunks per lane
  if (ch <= 1) HL_LAUNCH_TAB(1);
  else if (ch <= 2) HL_LAUNCH_TAB(2);
  else if (ch <= 4) HL_LAUNCH_TAB(4);
  else if (ch <= 8) HL_LAUNCH_TAB(8);
  else if (ch <= 16) HL_LAUNCH_TAB(16);
  else if (ch <= kNormMaxChunks) HL_LAUNCH_TAB(kNormMaxChunks);
  else return hipErrorInvalidValue;
#undef HL_LAUNCH_TAB
  return hipGetLastError();
}

// 8 consecutive values of a row starting at column c, as bf16: from the bf16
// row (SPLITS = 0), or summed over SPLITS split-K partials in split order and
// rounded exactly as the separate reduce does (all loads issued first)
template <int SPLITS>
__device__ __forceinline__ u32x4 row8(const bf16* row, const float* part, size_t plane, int c) {
  if constexpr (SPLITS == 0) {
    return ld16(row + c);
  } else {
    f32x4 plo[SPLITS], phi[SPLITS];
#pragma unroll
    for (int z = 0; z < SPLITS; ++z) {
      plo[z] = *reinterpret_cast<const f32x4*>(part + z * plane + c);
      phi[z] = *reinterpret_cast<const f32x4*>(part + z * plane + c + 4);
    }
    f32x4 lo = plo[0], hi = phi[0];
#pragma unroll
    for (int z = 1; z < SPLITS; ++z) {
      lo += plo[z];
      hi += phi[z];
    }
    return u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
  }
}

constexpr int kRopeHeads = 4;  // heads per workgroup of the wide append kernel

// Workgroup (row r, heads 4 y .. 4 y + 3) of the q, k, v heads.  q / k heads:
// a thread takes 8 consecutive pairs, rotates them with the row's table and
// writes them back (k also to the row's KV slot).  v heads: a thread takes 8
// values and writes them to the slot (dimension-major in the page).  With
// partials (SPLITS > 0 of them) the row is formed from them and written back
// whole, and rows in [rows, Mp) are zero rows.
template <int SPLITS>
__global__ __launch_bounds__(64) void rope_append_wide_kernel(
    bf16* __restrict__ qkv, const float* __restrict__ part, int rows, int Mp, int nq, int nkv,
    int d, KvDev kv, RopeTab tab) {
  const int r = blockIdx.x;
  const int h0 = blockIdx.y * kRopeHeads;
  const int nh = nq + 2 * nkv;
  const int ld = nh * d;
  const int half = d >> 1;
  bf16* row = qkv + (size_t)r * ld;
  const int hend = min(h0 + kRopeHeads, nh);
  if (r >= rows) {
    for (int c = h0 * d + threadIdx.x * 8; c < hend * d; c += 64 * 8)
      *reinterpret_cast<u32x4*>(row + c) = u32x4{0, 0, 0, 0};
    return;
  }
  const float* pr = part ? part + (size_t)r * ld : nullptr;
  const size_t plane = (size_t)Mp * ld;
  const int slot = tab.slot[r];
  const int page = slot >= 0 ? slot / kv.page_size : -1;
  const int off = slot >= 0 ? slot % kv.page_size : 0;
  const float* cs = tab.cs + (size_t)r * half;
  const float* sn = tab.sn + (size_t)r * half;
  const int qk_groups = half / 8;  // 8-pair groups per q / k head
  const int v_groups = d / 8;      // 8-value groups per v head
  // items: (head, group) over the workgroup's heads, in head order
  int items = 0;
  for (int h = h0; h < hend; ++h) items += h >= nq + nkv ? v_groups : qk_groups;
  for (int it = threadIdx.x; it < items; it += 64) {
    int h = h0, t = it;
    while (true) {  // at most 4 heads
      const int per = h >= nq + nkv ? v_groups : qk_groups;
      if (t < per) break;
      t -= per;
      ++h;
    }
    bf16* u = row + h * d;
    if (h < nq + nkv) {
      const int i0 = t * 8;
      const u32x4 av = row8<SPLITS>(row, pr, plane, h * d + i0);
      const u32x4 bv = row8<SPLITS>(row, pr, plane, h * d + i0 + half);
      u32x4 oa, ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = __uint_as_float(av[e] << 16), a1 = __uint_as_float(av[e] & 0xffff0000u);
        const float b0 = __uint_as_float(bv[e] << 16), b1 = __uint_as_float(bv[e] & 0xffff0000u);
        const float c0 = cs[i0 + 2 * e], c1 = cs[i0 + 2 * e + 1];
        const float s0 = sn[i0 + 2 * e], s1 = sn[i0 + 2 * e + 1];
        oa[e] = pack2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
        ob[e] = pack2(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
      }
      *reinterpret_cast<u32x4*>(u + i0) = oa;
      *reinterpret_cast<u32x4*>(u + i0 + half) = ob;
      if (h >= nq && page >= 0) {
        bf16* kp = kv.k_page(page, h - nq) + (size_t)off * d;
        *reinterpret_cast<u32x4*>(kp + i0) = oa;
        *reinterpret_cast<u32x4*>(kp + i0 + half) = ob;
      }
    } else {
      const int gv = h - nq - nkv, dd = t * 8;
      const u32x4 vv = row8<SPLITS>(row, pr, plane, h * d + dd);
      if (pr) *reinterpret_cast<u32x4*>(u + dd) = vv;
      if (page < 0) continue;
      bf16* vp = kv.v_page(page, gv) + (size_t)dd * kv.page_size + off;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vp[(2 * j) * kv.page_size] = (bf16)(vv[j] & 0xffffu);
        vp[(2 * j + 1) * kv.page_size] = (bf16)(vv[j] >> 16);
      }
    }
  }
}

hipError_t launch_rope_append_wide(bf16* qkv, const float* part, int splits, int rows, int Mp,
                                   int nq, int nkv, int d, const KvDev& kv, const RopeTab& tab,
                                   hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nh = nq + 2 * nkv;
  const dim3 grid(part ? Mp : rows, (nh + kRopeHeads - 1) / kRopeHeads);
#define HL_ROPE(S_)                                                                          \
  hipLaunchKernelGGL(rope_append_wide_kernel<S_>, grid, dim3(64), 0, s, qkv, part, rows, Mp, nq, \
                     nkv, d, kv, tab)
  if (!part) HL_ROPE(0);
  else if (splits == 2) HL_ROPE(2);
  else if (splits == 4) HL_ROPE(4);
  else if (splits == 8) HL_ROPE(8);
  else return hipErrorInvalidValue;
#undef HL_ROPE
  return hipGetLastError();
}

}  // namespace hl

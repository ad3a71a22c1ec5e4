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
// One 256-thread workgroup per row: each thread loads its CH 16-byte chunks
// of the row and of the gain together (one memory round trip), the sum of
// squares is reduced over the workgroup, and the scaled row is stored from
// registers.  One row per workgroup keeps hundreds of workgroups in flight
// even for a few hundred rows.  hidden is a multiple of 8 and at most
// 256 * 8 * kNormMaxChunks.
constexpr int kNormThreads = 256;
constexpr int kNormMaxChunks = 8;  // 16-byte chunks per thread: hidden <= 16384

template <int CH>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ g, bf16* __restrict__ y, int rows,
    int hidden, float eps) {
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  bf16* yr = y + (size_t)r * hidden;
  if (r >= rows) {  // padding row: zero dummy token
    for (int c = tid * 8; c < hidden; c += kNormThreads * 8)
      *reinterpret_cast<u32x4*>(yr + c) = u32x4{0, 0, 0, 0};
    return;
  }
  const bf16* xr = x + (size_t)r * hidden;
  u32x4 v[CH], gv[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = (i * kNormThreads + tid) * 8;
    v[i] = c < hidden ? ld16(xr + c) : u32x4{0, 0, 0, 0};
    gv[i] = c < hidden ? ld16(g + c) : u32x4{0, 0, 0, 0};
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __uint_as_float(v[i][e] << 16), b = __uint_as_float(v[i][e] & 0xffff0000u);
      ss += a * a + b * b;
    }
  __shared__ float red[kNormThreads / 64];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)hidden + eps);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = (i * kNormThreads + tid) * 8;
    if (c >= hidden) continue;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __uint_as_float(v[i][e] << 16) * inv * __uint_as_float(gv[i][e] << 16);
      const float b = __uint_as_float(v[i][e] & 0xffff0000u) * inv *
                      __uint_as_float(gv[i][e] & 0xffff0000u);
      o[e] = pack2(a, b);
    }
    *reinterpret_cast<u32x4*>(yr + c) = o;
  }
}

hipError_t launch_rmsnorm(const bf16* x, const bf16* g, bf16* y, int rows, int rows_padded,
                          int hidden, float eps, hipStream_t s) {
  if (rows_padded == 0) return hipSuccess;
  if (hidden % 8) return hipErrorInvalidValue;
  const int ch = (hidden + kNormThreads * 8 - 1) / (kNormThreads * 8);  // chunks per thread
  const dim3 grid(rows_padded), block(kNormThreads);
#define HL_NORM(CH_) \
  hipLaunchKernelGGL(rmsnorm_kernel<CH_>, grid, block, 0, s, x, g, y, rows, hidden, eps)
  if (ch <= 1) HL_NORM(1);
  else if (ch <= 2) HL_NORM(2);
  else if (ch <= 4) HL_NORM(4);
  else if (ch <= kNormMaxChunks) HL_NORM(kNormMaxChunks);
  else return hipErrorInvalidValue;
#undef HL_NORM
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

// ---------------------------------------------------- layer path: wide append
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

constexpr int kRopeHeads = 16;     // heads per workgroup of the wide append kernel
constexpr int kRopeThreads = 256;

// Workgroup (row r, heads 16 y .. 16 y + 15) of the q, k, v heads, one 8-wide
// item per thread: a q / k item is 8 consecutive rotation pairs of one head
// (rotated and written back, k also to the row's KV slot), a v item 8 values
// of one head (written to the slot, dimension-major in the page).  The row's
// position and slot are resolved in the workgroup and its cos / sin are
// formed while the row's loads are in flight (one pair per thread of the
// first d/2).  With partials (SPLITS > 0 of them) the row is formed from them
// and written back whole, and rows in [rows, Mp) are zero rows.
template <int SPLITS>
__global__ __launch_bounds__(kRopeThreads) void rope_append_wide_kernel(
    bf16* __restrict__ qkv, const float* __restrict__ part, int rows, int Mp, int nq, int nkv,
    int d, ChunkList chunks, DecDev dec, RopeFreq freq, KvDev kv) {
  // Rows go to the XCDs in contiguous runs (workgroup ids are dealt
  // round-robin over the 8 XCDs, and the grid's x extent is a multiple of 8
  // when it is Mp): the tokens of one KV page, whose V values share the
  // page's dimension rows (dimension-major V), are then written through one
  // L2, which merges them, instead of each XCD's L2 writing back its own
  // part of every line.
  const int nrows = gridDim.x;
  const int per = nrows / 8, rem = nrows % 8, xcd = blockIdx.x % 8;
  const int r = xcd * per + min(xcd, rem) + blockIdx.x / 8;
  const int tid = threadIdx.x;
  const int h0 = blockIdx.y * kRopeHeads;
  const int nh = nq + 2 * nkv;
  const int ld = nh * d;
  const int half = d >> 1;
  bf16* row = qkv + (size_t)r * ld;
  const int hend = min(h0 + kRopeHeads, nh);
  if (r >= rows) {
    for (int c = h0 * d + tid * 8; c < hend * d; c += kRopeThreads * 8)
      *reinterpret_cast<u32x4*>(row + c) = u32x4{0, 0, 0, 0};
    return;
  }
  const float* pr = part ? part + (size_t)r * ld : nullptr;
  const size_t plane = (size_t)Mp * ld;
  const int qk_groups = half / 8;  // 8-pair items per q / k head
  const int v_groups = d / 8;      // 8-value items per v head
  // the workgroup's q / k heads come first, then its v heads
  const int qk_end = min(hend, nq + nkv);
  const int n_qk = max(qk_end - h0, 0) * qk_groups;
  const int v_begin = max(h0, nq + nkv);
  const int items = n_qk + max(hend - v_begin, 0) * v_groups;
  // one item per thread (d <= 128: at most 16 heads x 16 items)
  const int it = tid;
  const bool has = it < items;
  const bool is_qk = it < n_qk;
  const int h = is_qk ? h0 + it / qk_groups : v_begin + (it - n_qk) / v_groups;
  const int t = is_qk ? it % qk_groups : (it - n_qk) % v_groups;
  u32x4 av{0, 0, 0, 0}, bv{0, 0, 0, 0};
  if (has) {
    if (is_qk) {
      av = row8<SPLITS>(row, pr, plane, h * d + t * 8);
      bv = row8<SPLITS>(row, pr, plane, h * d + t * 8 + half);
    } else {
      av = row8<SPLITS>(row, pr, plane, h * d + t * 8);
    }
  }
  int pos, slot;
  row_pos_slot(chunks, dec, kv.page_size, kv.num_pages, r, &pos, &slot);
  const int page = slot >= 0 ? slot / kv.page_size : -1;
  const int off = slot >= 0 ? slot % kv.page_size : 0;
  __shared__ float cs_tab[kRopeMaxPairs], sn_tab[kRopeMaxPairs];
  if (n_qk > 0) {  // uniform
    if (tid < half) rope_cos_sin(pos, freq.inv[tid], &cs_tab[tid], &sn_tab[tid]);
    __syncthreads();
  }
  if (!has) return;
  bf16* u = row + h * d;
  if (is_qk) {
    const int i0 = t * 8;
    u32x4 oa, ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = __uint_as_float(av[e] << 16), a1 = __uint_as_float(av[e] & 0xffff0000u);
      const float b0 = __uint_as_float(bv[e] << 16), b1 = __uint_as_float(bv[e] & 0xffff0000u);
      const float c0 = cs_tab[i0 + 2 * e], c1 = cs_tab[i0 + 2 * e + 1];
      const float s0 = sn_tab[i0 + 2 * e], s1 = sn_tab[i0 + 2 * e + 1];
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
    if (pr) *reinterpret_cast<u32x4*>(u + dd) = av;
    if (page < 0) return;
    bf16* vp = kv.v_page(page, gv) + (size_t)dd * kv.page_size + off;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vp[(2 * j) * kv.page_size] = (bf16)(av[j] & 0xffffu);
      vp[(2 * j + 1) * kv.page_size] = (bf16)(av[j] >> 16);
    }
  }
}

hipError_t launch_rope_append_wide(bf16* qkv, const float* part, int splits, int rows, int Mp,
                                   int nq, int nkv, int d, float theta, const ChunkList& chunks,
                                   const DecDev& dec, const KvDev& kv, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (d / 2 > kRopeMaxPairs || kRopeHeads * (d / 8) > kRopeThreads) return hipErrorInvalidValue;
  const RopeFreq freq = rope_freq(d, theta);
  const int nh = nq + 2 * nkv;
  const dim3 grid(part ? Mp : rows, (nh + kRopeHeads - 1) / kRopeHeads);
#define HL_ROPE(S_)                                                                           \
  hipLaunchKernelGGL(rope_append_wide_kernel<S_>, grid, dim3(kRopeThreads), 0, s, qkv, part, rows, \
                     Mp, nq, nkv, d, chunks, dec, freq, kv)
  if (!part) HL_ROPE(0);
  else if (splits == 2) HL_ROPE(2);
  else if (splits == 3) HL_ROPE(3);
  else if (splits == 4) HL_ROPE(4);
  else if (splits == 5) HL_ROPE(5);
  else if (splits == 6) HL_ROPE(6);
  else if (splits == 7) HL_ROPE(7);
  else if (splits == 8) HL_ROPE(8);
  else return hipErrorInvalidValue;
#undef HL_ROPE
  return hipGetLastError();
}

}  // namespace hl

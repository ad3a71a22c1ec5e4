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
// Decode: one wave per (decode j, kv head g, 256-key partition); the G query
// heads of kv head g are the tile rows.  Every K and V byte of the context is
// read once.  A decode whose context fits one partition writes its output
// directly.
#include <string.h>

#include "attn_common.h"

namespace hl {

constexpr int kAttnWaves = 4;
constexpr int kPrefillRows = 16 * kAttnWaves;  // rows per prefill workgroup

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
  int dc_parts;  // partitions of the longest context
  int dc_wgs;    // decode workgroups = ceil(n * parts * nkv / 4)
  float* dc_o;
  float* dc_ml;
};

template <int D>
__device__ __forceinline__ void init_acc(AttnAcc<D>& a) {
  a.m = -INFINITY;
  a.l = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) a.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D>
__device__ __forceinline__ void prefill_wave(const AttnArgs& A, int b, int wave, int l16, int q) {
  const int per_chunk = A.pf_gx * A.pf_ns * A.nkv;
  const int c = b / per_chunk;
  const int rem = b % per_chunk;
  const int g = rem / (A.pf_gx * A.pf_ns);
  const int x = rem % (A.pf_gx * A.pf_ns);
  const int rg = x / A.pf_ns, sp = x % A.pf_ns;
  const ChunkDev ch = A.chunks.c[c];
  const int G = A.nq / A.nkv;
  const int rows_total = ch.len * G;
  const int rbase = (rg * kAttnWaves + wave) * 16;
  if (rbase >= rows_total) return;
  const int kv_len = ch.start_pos + ch.len;
  const int ld = (A.nq + 2 * A.nkv) * D;

  const int row = rbase + l16;
  const bool valid = row < rows_total;
  const int tok = valid ? row / G : 0;
  const int hh = row % G;
  const int row_limit = valid ? ch.start_pos + tok : -1;
  bf16x8 qf[D / 32];
  const bf16* qp = A.qkv + (size_t)(ch.row0 + tok) * ld + (size_t)(g * G + hh) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = valid ? as_bf16x8(ld16(qp + ks * 32 + q * 8)) : as_bf16x8(u32x4{0, 0, 0, 0});

  const int last_row = min(rbase + 16, rows_total) - 1;
  const int k_stop = ch.start_pos + last_row / G + 1;
  const int k0 = sp * A.pf_seg;
  const int k1 = min(k_stop, k0 + A.pf_seg);
  if (k0 >= k1) return;  // none of this wave's rows reaches this segment

  AttnAcc<D> a;
  init_acc<D>(a);
  attend_segment<D>(a, qf, row_limit, k0, k1, kv_len, ch.block_table, ch.n_blocks, A.kv, g, l16, q);
  const float l_tot = row_total(a.l);
  if (!valid) return;
  const int h = g * G + hh;
  const int n_parts = min(A.pf_ns, (row_limit + A.pf_seg) / A.pf_seg);
  if (sp >= n_parts) return;  // this row has no key in the segment
  const int grow = ch.row0 + tok;
  if (n_parts == 1) {
    store_row<D>(a, l_tot, A.attn + (size_t)grow * A.nq * D + (size_t)h * D, q);
    return;
  }
  const size_t pidx = ((size_t)grow * A.nq + h) * A.pf_ns + sp;
  store_partial<D>(a, l_tot, A.pf_o + pidx * D, A.pf_ml + pidx * 2, q);
}

template <int D>
__device__ __forceinline__ void decode_wave(const AttnArgs& A, int unit, int l16, int q) {
  // unit = ((j * parts + part) * nkv + g): a workgroup's waves share (j, part)
  const int g = unit % A.nkv;
  const int jp = unit / A.nkv;
  const int part = jp % A.dc_parts, j = jp / A.dc_parts;
  if (j >= A.dec.n) return;
  const int G = A.nq / A.nkv;
  const int ctx = A.dec.ctx_lens[j];
  const int n_keys = ctx + 1;
  const int k0 = part * kDecodePart;
  if (k0 >= n_keys) return;
  const int k1 = min(n_keys, k0 + kDecodePart);
  const int n_parts = (n_keys + kDecodePart - 1) / kDecodePart;
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
  attend_segment<D>(a, qf, ctx, k0, k1, n_keys,
                    A.dec.block_tables + (size_t)j * A.dec.max_blocks, A.dec.max_blocks, A.kv, g,
                    l16, q);
  const float l_tot = row_total(a.l);
  if (l16 >= G) return;
  const int h = g * G + l16;
  if (n_parts == 1) {
    store_row<D>(a, l_tot, A.attn + (size_t)row * A.nq * D + (size_t)h * D, q);
    return;
  }
  const size_t pidx = ((size_t)j * A.nq + h) * A.dc_parts + part;
  store_partial<D>(a, l_tot, A.dc_o + pidx * D, A.dc_ml + pidx * 2, q);
}

template <int D>
__global__ __launch_bounds__(64 * kAttnWaves) void attention_kernel(AttnArgs A) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int b = blockIdx.x;
  if (b < A.pf_wgs)
    prefill_wave<D>(A, b, wave, l16, q);
  else
    decode_wave<D>(A, (b - A.pf_wgs) * kAttnWaves + wave, l16, q);
}

// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over the parts a unit
// (row, head) used; a unit with one part was written directly.
template <int D>
__device__ __forceinline__ void merge_unit(const float* __restrict__ o_part,
                                           const float* __restrict__ ml_part, size_t base,
                                           int n_parts, bf16* __restrict__ orow) {
  float mmax = -INFINITY;
  for (int p = 0; p < n_parts; ++p) mmax = fmaxf(mmax, ml_part[(base + p) * 2]);
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  float lsum = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float mp = ml_part[(base + p) * 2];
    if (mp == -INFINITY) continue;  // no visible key in this part
    const float w = exp2f(mp - mmax);
    lsum += w * ml_part[(base + p) * 2 + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += w * o_part[(base + p) * D + threadIdx.x * PER + i];
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[threadIdx.x * PER + i] = f2bf(o[i] * inv);
}

// one 64-thread block per (row, q head); grid.y spans chunk rows then decodes
template <int D>
__global__ __launch_bounds__(64) void attention_merge_kernel(AttnArgs A) {
  const int h = blockIdx.x, r = blockIdx.y;
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
    const int n_parts = min(A.dc_parts, (A.dec.ctx_lens[j] + kDecodePart) / kDecodePart);
    if (n_parts <= 1) return;
    orow += (size_t)(A.dc_row0 + j) * A.nq * D + (size_t)h * D;
    merge_unit<D>(A.dc_o, A.dc_ml, ((size_t)j * A.nq + h) * A.dc_parts, n_parts, orow);
  }
}

// ---------------------------------------------------------------- host side
// Prefill key split: only when the chunk rows give fewer than 256 workgroups,
// into segments of >= 256 keys (multiples of 32), aiming at ~512 workgroups.
void prefill_split(const ChunkList& chunks, int nq, int nkv, int* nsplit, int* seg) {
  const int G = nq / nkv;
  int base = 0, max_keys = 0;
  for (int i = 0; i < chunks.n; ++i) {
    base += (chunks.c[i].len * G + kPrefillRows - 1) / kPrefillRows * nkv;
    max_keys = max(max_keys, chunks.c[i].start_pos + chunks.c[i].len);
  }
  int ns = 1;
  if (base > 0 && base < 256) ns = min((512 + base - 1) / base, max(1, max_keys / 256));
  ns = max(ns, 1);
  int sg = (max_keys + ns - 1) / ns;
  sg = (sg + 31) / 32 * 32;
  if (sg <= 0) sg = 32;
  *seg = sg;
  *nsplit = max(1, (max_keys + sg - 1) / sg);
}

// Upper bound of prefill_workspace_bytes over every chunk layout with at most
// `rows` chunk rows (any start positions): the split count is at most
// ceil(512 / base) with base >= ceil(r G / 64) nkv workgroups for r rows.
size_t prefill_workspace_bound(int rows, int nq, int nkv, int d) {
  const int G = nq / nkv;
  size_t worst = 0;
  for (int r = 1; r <= rows; ++r) {
    const int base = (r * G + kPrefillRows - 1) / kPrefillRows * nkv;
    if (base >= 256) continue;
    const size_t ns = (512 + base - 1) / base;
    worst = max(worst, ns * (size_t)r);
  }
  return worst ? worst * nq * (d + 2) * sizeof(float) + 256 : 0;
}

size_t prefill_workspace_bytes(const ChunkList& chunks, int nq, int nkv, int d) {
  int ns, sg;
  prefill_split(chunks, nq, nkv, &ns, &sg);
  if (ns <= 1) return 0;
  return (size_t)ns * chunks.n_rows * nq * (d + 2) * sizeof(float) + 256;
}

static int parts_for(int max_ctx) { return (max_ctx + 1 + kDecodePart - 1) / kDecodePart; }

size_t decode_workspace_bytes(int n_decodes, int nq, int d, int max_ctx) {
  const size_t parts = (size_t)parts_for(max_ctx);
  return (size_t)n_decodes * nq * parts * (d + 2) * sizeof(float) + 256;
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
  const int G = nq / nkv;
  if (chunks.n > 0 && chunks.n_rows > 0) {
    int max_len = 0;
    for (int i = 0; i < chunks.n; ++i) max_len = max(max_len, chunks.c[i].len);
    A.pf_gx = (max_len * G + kPrefillRows - 1) / kPrefillRows;
    A.pf_ns = 1;
    A.pf_seg = 1 << 30;
    if (pf_ws) {
      prefill_split(chunks, nq, nkv, &A.pf_ns, &A.pf_seg);
      if (A.pf_ns <= 1) {
        A.pf_ns = 1;
        A.pf_seg = 1 << 30;
      }
    }
    A.pf_wgs = A.pf_gx * A.pf_ns * nkv * chunks.n;
    A.pf_o = reinterpret_cast<float*>(pf_ws);
    A.pf_ml = A.pf_ns > 1 ? A.pf_o + (size_t)A.pf_ns * chunks.n_rows * nq * d : nullptr;
  }
  A.dec = dec;
  A.dc_row0 = dec_row0;
  if (dec.n > 0) {
    A.dc_parts = parts_for(dec.max_ctx);
    A.dc_wgs = (dec.n * A.dc_parts * nkv + kAttnWaves - 1) / kAttnWaves;
    A.dc_o = reinterpret_cast<float*>(dc_ws);
    A.dc_ml = A.dc_o + (size_t)dec.n * nq * A.dc_parts * d;
  }
  const int wgs = A.pf_wgs + A.dc_wgs;
  if (wgs == 0) return mid ? hipEventRecord(mid, s) : hipSuccess;
  const int merge_rows = chunks.n_rows + dec.n;
  const bool merge = A.pf_ns > 1 || A.dc_parts > 1;
  if (d == 128)
    hipLaunchKernelGGL(attention_kernel<128>, dim3(wgs), dim3(64 * kAttnWaves), 0, s, A);
  else
    hipLaunchKernelGGL(attention_kernel<64>, dim3(wgs), dim3(64 * kAttnWaves), 0, s, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mid && (e = hipEventRecord(mid, s)) != hipSuccess) return e;
  if (!merge) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL(attention_merge_kernel<128>, dim3(nq, merge_rows), dim3(64), 0, s, A);
  else
    hipLaunchKernelGGL(attention_merge_kernel<64>, dim3(nq, merge_rows), dim3(64), 0, s, A);
  return hipGetLastError();
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

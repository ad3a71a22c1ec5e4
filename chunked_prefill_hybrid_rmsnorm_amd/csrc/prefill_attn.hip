// Chunk-prefill attention: row i of a chunk (position start_pos + i) attends
// keys 0 .. start_pos + i of its request -- the KV that earlier chunks left in
// the pages plus the chunk's own keys, causally -- read through the chunk's
// block table.  Because every chunk re-reads the KV of all earlier chunks,
// prefilling a prompt in N chunks reads chunk KV N(N-1)/2 extra times; the
// kernel reads each needed page once per workgroup and kv head and leaves
// that cost visible.
//
// GQA packing: the 16 rows of a wave are (token, q head) pairs of one kv head,
// row = token * G + head, so one K/V fragment serves all G heads.  A
// workgroup is 4 waves over 64 consecutive rows; the waves walk the same keys
// (their K/V fragments hit in L1).  When the chunk has few row groups the key
// range is also split into segments handled by separate workgroups (more
// waves in flight), and a merge combines the segments; a row whose keys fit in
// the first segment writes its output directly.
#include "attn_common.h"

namespace hl {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillRows = 16 * kPrefillWaves;  // rows per workgroup

template <int D>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_attn_kernel(
    const bf16* __restrict__ qkv, int nq, int nkv, ChunkList chunks, KvDev kv,
    bf16* __restrict__ attn, float* __restrict__ o_part, float* __restrict__ ml_part, int nsplit,
    int seg) {
  const int c = blockIdx.z, g = blockIdx.y;
  if (c >= chunks.n) return;
  const ChunkDev ch = chunks.c[c];
  const int rg = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
  const int G = nq / nkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int rows_total = ch.len * G;
  const int rbase = (rg * kPrefillWaves + wave) * 16;
  if (rbase >= rows_total) return;
  const int kv_len = ch.start_pos + ch.len;
  const int ld = (nq + 2 * nkv) * D;

  const int row = rbase + l16;
  const bool valid = row < rows_total;
  const int tok = valid ? row / G : 0;
  const int hl_ = row % G;
  const int row_limit = valid ? ch.start_pos + tok : -1;
  bf16x8 qf[D / 32];
  const bf16* qp = qkv + (size_t)(ch.row0 + tok) * ld + (size_t)(g * G + hl_) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = valid ? as_bf16x8(ld16(qp + ks * 32 + q * 8)) : as_bf16x8(u32x4{0, 0, 0, 0});

  // keys the wave needs: 0 .. last valid row's position; this workgroup's segment
  const int last_row = min(rbase + 16, rows_total) - 1;
  const int k_stop = ch.start_pos + last_row / G + 1;
  const int k0 = sp * seg;
  const int k1 = min(k_stop, k0 + seg);
  if (k0 >= k1) return;  // none of this wave's rows reaches this segment

  AttnAcc<D> a;
  a.m = -INFINITY;
  a.l = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) a.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  attend_segment<D>(a, qf, row_limit, k0, k1, kv_len, ch.block_table, ch.n_blocks, kv, g, l16, q);
  const float l_tot = row_total(a.l);
  if (!valid) return;
  const int h = g * G + hl_;
  const int n_parts = min(nsplit, (row_limit + 1 + seg - 1) / seg);
  if (sp >= n_parts) return;  // this row has no key in the segment
  const int grow = ch.row0 + tok;
  if (n_parts == 1) {
    store_row<D>(a, l_tot, attn + (size_t)grow * nq * D + (size_t)h * D, q);
    return;
  }
  const size_t pidx = ((size_t)grow * nq + h) * nsplit + sp;
  store_partial<D>(a, l_tot, o_part + pidx * D, ml_part + pidx * 2, q);
}

template <int D>
__device__ void merge_unit_p(const float* __restrict__ o_part, const float* __restrict__ ml_part,
                             size_t base, int n_parts, bf16* __restrict__ orow) {
  float mmax = -INFINITY;
  for (int p = 0; p < n_parts; ++p) mmax = fmaxf(mmax, ml_part[(base + p) * 2]);
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  float lsum = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float mp = ml_part[(base + p) * 2];
    if (mp == -INFINITY) continue;
    const float w = exp2f(mp - mmax);
    lsum += w * ml_part[(base + p) * 2 + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += w * o_part[(base + p) * D + threadIdx.x * PER + i];
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[threadIdx.x * PER + i] = f2bf(o[i] * inv);
}

// one 64-thread block per (chunk row, q head)
template <int D>
__global__ __launch_bounds__(64) void prefill_merge_kernel(int nq, ChunkList chunks,
                                                           const float* __restrict__ o_part,
                                                           const float* __restrict__ ml_part,
                                                           int nsplit, int seg,
                                                           bf16* __restrict__ attn) {
  const int h = blockIdx.x, grow = blockIdx.y;
  int c = 0;
  while (c + 1 < chunks.n && grow >= chunks.c[c + 1].row0) ++c;
  const int pos = chunks.c[c].start_pos + (grow - chunks.c[c].row0);
  const int n_parts = min(nsplit, (pos + 1 + seg - 1) / seg);
  if (n_parts <= 1) return;
  merge_unit_p<D>(o_part, ml_part, ((size_t)grow * nq + h) * nsplit, n_parts,
                  attn + (size_t)grow * nq * D + (size_t)h * D);
}

// Key split: only when the chunk rows give fewer than 256 workgroups, into
// segments of >= 256 keys (multiples of 32), aiming at ~512 workgroups.
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
  *nsplit = (max_keys + sg - 1) / sg;
  if (*nsplit < 1) *nsplit = 1;
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

template <int D>
static void launch_p(const bf16* qkv, int nq, int nkv, const ChunkList& chunks, const KvDev& kv,
                     bf16* attn, float* o_part, float* ml_part, int ns, int sg, hipStream_t s) {
  const int G = nq / nkv;
  int max_len = 0;
  for (int i = 0; i < chunks.n; ++i) max_len = max(max_len, chunks.c[i].len);
  const int gx = (max_len * G + kPrefillRows - 1) / kPrefillRows;
  if (gx == 0) return;
  hipLaunchKernelGGL(prefill_attn_kernel<D>, dim3(gx * ns, nkv, chunks.n),
                     dim3(64 * kPrefillWaves), 0, s, qkv, nq, nkv, chunks, kv, attn, o_part,
                     ml_part, ns, sg);
  if (ns > 1)
    hipLaunchKernelGGL(prefill_merge_kernel<D>, dim3(nq, chunks.n_rows), dim3(64), 0, s, nq,
                       chunks, o_part, ml_part, ns, sg, attn);
}

hipError_t launch_prefill_attention(const bf16* qkv, int nq, int nkv, int d,
                                    const ChunkList& chunks, const KvDev& kv, bf16* attn,
                                    void* ws, hipStream_t s) {
  if (chunks.n == 0 || chunks.n_rows == 0) return hipSuccess;
  int ns = 1, sg = 1 << 30;
  if (ws) prefill_split(chunks, nq, nkv, &ns, &sg);
  if (ns <= 1) {
    ns = 1;
    sg = 1 << 30;
  }
  float* o_part = reinterpret_cast<float*>(ws);
  float* ml_part = ns > 1 ? o_part + (size_t)ns * chunks.n_rows * nq * d : nullptr;
  if (d == 128)
    launch_p<128>(qkv, nq, nkv, chunks, kv, attn, o_part, ml_part, ns, sg, s);
  else
    launch_p<64>(qkv, nq, nkv, chunks, kv, attn, o_part, ml_part, ns, sg, s);
  return hipGetLastError();
}

}  // namespace hl

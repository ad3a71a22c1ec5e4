// Paged GQA decode attention (PagedAttention-style reads of each request's
// pages through its block table), split-K over fixed 256-key partitions,
// followed by a log-sum-exp merge of the partitions.
//
// One wave per (decode j, kv head g, partition): the G query heads sharing kv
// head g are the MFMA tile's rows (G <= 16; unused rows hold zero queries).
// The kernel is bound by HBM: every K and V byte of the context is read once,
// as 16- and 8-byte vector loads, with the next 32 keys in flight while the
// current ones are multiplied.  A decode whose context fits one partition
// writes its output directly; the others leave (o, m, l) per partition for
// the merge.
#include "attn_common.h"

namespace hl {

template <int D>
__global__ __launch_bounds__(64) void decode_attn_kernel(
    const bf16* __restrict__ qkv, int row0, int nq, int nkv, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_tables, int max_blocks, KvDev kv, float* __restrict__ o_part,
    float* __restrict__ ml_part, int max_parts, bf16* __restrict__ attn) {
  const int part = blockIdx.x, g = blockIdx.y, j = blockIdx.z;
  const int G = nq / nkv;
  const int lane = threadIdx.x, l16 = lane & 15, q = lane >> 4;

  const int ctx = ctx_lens[j];
  const int n_keys = ctx + 1;
  const int k0 = part * kDecodePart;
  if (k0 >= n_keys) return;
  const int k1 = min(n_keys, k0 + kDecodePart);
  const int n_parts = (n_keys + kDecodePart - 1) / kDecodePart;

  const int ld = (nq + 2 * nkv) * D;
  const bf16* qrow = qkv + (size_t)(row0 + j) * ld + (size_t)(g * G) * D;
  bf16x8 qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qf[ks] = l16 < G ? as_bf16x8(ld16(qrow + l16 * D + ks * 32 + q * 8))
                     : as_bf16x8(u32x4{0, 0, 0, 0});

  AttnAcc<D> a;
  a.m = -INFINITY;
  a.l = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) a.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  attend_segment<D>(a, qf, ctx, k0, k1, n_keys, block_tables + (size_t)j * max_blocks, max_blocks,
                    kv, g, l16, q);
  const float l_tot = row_total(a.l);
  if (l16 >= G) return;
  const int h = g * G + l16;
  if (n_parts == 1) {
    store_row<D>(a, l_tot, attn + (size_t)(row0 + j) * nq * D + (size_t)h * D, q);
    return;
  }
  const size_t pidx = ((size_t)j * nq + h) * max_parts + part;
  store_partial<D>(a, l_tot, o_part + pidx * D, ml_part + pidx * 2, q);
}

// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p over the partitions a
// unit (row, head) used; units with a single partition were written directly.
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
    if (mp == -INFINITY) continue;  // no visible key in this partition
    const float w = exp2f(mp - mmax);
    lsum += w * ml_part[(base + p) * 2 + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += w * o_part[(base + p) * D + threadIdx.x * PER + i];
  }
  const float inv = 1.f / lsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[threadIdx.x * PER + i] = f2bf(o[i] * inv);
}

template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    int row0, int nq, const int32_t* __restrict__ ctx_lens, const float* __restrict__ o_part,
    const float* __restrict__ ml_part, int max_parts, bf16* __restrict__ attn) {
  const int h = blockIdx.x, j = blockIdx.y;
  const int n_parts = min(max_parts, (ctx_lens[j] + 1 + kDecodePart - 1) / kDecodePart);
  if (n_parts <= 1) return;
  merge_unit<D>(o_part, ml_part, ((size_t)j * nq + h) * max_parts, n_parts,
                attn + (size_t)(row0 + j) * nq * D + (size_t)h * D);
}

static int parts_for(int max_ctx) { return (max_ctx + 1 + kDecodePart - 1) / kDecodePart; }

size_t decode_workspace_bytes(int n_decodes, int nq, int d, int max_ctx) {
  const size_t parts = (size_t)parts_for(max_ctx);
  return (size_t)n_decodes * nq * parts * (d + 2) * sizeof(float) + 256;
}

template <int D>
static void launch_d(const bf16* qkv, int row0, int nq, int nkv, const DecDev& dec,
                     const KvDev& kv, bf16* attn, float* o_part, float* ml_part, int parts,
                     hipStream_t s) {
  hipLaunchKernelGGL(decode_attn_kernel<D>, dim3(parts, nkv, dec.n), dim3(64), 0, s, qkv, row0, nq,
                     nkv, dec.ctx_lens, dec.block_tables, dec.max_blocks, kv, o_part, ml_part,
                     parts, attn);
  if (parts > 1)
    hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(nq, dec.n), dim3(64), 0, s, row0, nq,
                       dec.ctx_lens, o_part, ml_part, parts, attn);
}

hipError_t launch_decode_attention(const bf16* qkv, int row0, int nq, int nkv, int d,
                                   const DecDev& dec, const KvDev& kv, bf16* attn, void* ws,
                                   hipStream_t s) {
  if (dec.n == 0) return hipSuccess;
  const int parts = parts_for(dec.max_ctx);
  float* o_part = reinterpret_cast<float*>(ws);
  float* ml_part = o_part + (size_t)dec.n * nq * parts * d;
  if (d == 128)
    launch_d<128>(qkv, row0, nq, nkv, dec, kv, attn, o_part, ml_part, parts, s);
  else
    launch_d<64>(qkv, row0, nq, nkv, dec, kv, attn, o_part, ml_part, parts, s);
  return hipGetLastError();
}

}  // namespace hl

// Paged GQA decode attention (PagedAttention-style reads of each request's
// pages through its block table), split-K over fixed 256-key partitions,
// followed by a log-sum-exp merge of the partitions.
//
// One wave per (decode j, kv head g, partition).  The G query heads that
// share kv head g are the 16 columns of an MFMA tile (G <= 16; unused
// columns hold zero queries), so:
//   S^T[key][head] = K[key][:] . q[head][:]   -- A = K rows (token-major page)
//   O^T[dim][head] += V^T[dim][key] P^T[key][head]  -- A = V^T (page stores V
//                                                      dimension-major)
// The probabilities that lane l holds after the first product are exactly
// the B operand it needs for the second, so no data moves between lanes
// except the per-head max.  The kernel is bound by HBM: every K and V byte
// of the context is read once, as 16- and 8-byte vector loads.
#include "kernels.h"

namespace hl {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ __launch_bounds__(64) void decode_attn_kernel(
    const bf16* __restrict__ qkv, int row0, int nq, int nkv, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_tables, int max_blocks, KvDev kv, float* __restrict__ o_part,
    float* __restrict__ ml_part, int max_parts, bf16* __restrict__ attn) {
  constexpr int KS = D / 32;   // k-steps of the score product
  constexpr int DB = D / 16;   // 16-row blocks of O^T
  constexpr int P = 16;        // page size
  const int part = blockIdx.x, g = blockIdx.y, j = blockIdx.z;
  const int G = nq / nkv;
  const int lane = threadIdx.x, l16 = lane & 15, q = lane >> 4;

  const int n_keys = ctx_lens[j] + 1;
  const int k_begin = part * kDecodePart;
  if (k_begin >= n_keys) return;
  const int k_end = min(n_keys, k_begin + kDecodePart);
  const int n_parts = (n_keys + kDecodePart - 1) / kDecodePart;
  const int32_t* bt = block_tables + (size_t)j * max_blocks;

  // q of head (g*G + l16), as B fragments of S^T = K Q^T
  const int ld = (nq + 2 * nkv) * D;
  const bf16* qrow = qkv + (size_t)(row0 + j) * ld + (size_t)(g * G) * D;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = l16 < G ? as_bf16x8(ld16(qrow + l16 * D + ks * 32 + q * 8)) : as_bf16x8(u32x4{0, 0, 0, 0});

  const float scale = kLog2e * rsqrtf((float)D);
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = k_begin; t0 < k_end; t0 += 2 * P) {
    // the two pages of this step (page -1: beyond the context)
    int page[2];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const int t = t0 + hp * P, blk = t / P;
      int pg = -1;
      if (t < k_end && blk < max_blocks) pg = bt[blk];
      page[hp] = (pg >= 0 && pg < kv.num_pages) ? pg : -1;
    }
    // issue every load of the step: K rows (16 B) and V^T pieces (8 B)
    u32x4 kf[2][KS];
    u32x2 vf[2][DB];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const bf16* kp = page[hp] >= 0 ? kv.k_page(page[hp], g) : nullptr;
      const bf16* vp = page[hp] >= 0 ? kv.v_page(page[hp], g) : nullptr;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[hp][ks] = kp ? ld16(kp + l16 * D + ks * 32 + q * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vf[hp][db] = vp ? ld8(vp + (db * 16 + l16) * P + 4 * q) : u32x2{0, 0};
    }
    // scores: lane holds keys t0 + 16 hp + 4q + r of head l16
    f32x4 s[2];
    float smax = -INFINITY;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      s[hp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[hp] = mfma16x16x32(as_bf16x8(kf[hp][ks]), qf[ks], s[hp]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + hp * P + 4 * q + r;
        s[hp][r] = t < k_end ? s[hp][r] * scale : -INFINITY;
        smax = fmaxf(smax, s[hp][r]);
      }
    }
    smax = fmaxf(smax, __shfl_xor(smax, 16));
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    const float m_new = fmaxf(m_run, smax);
    const float alpha = exp2f(m_run - m_new);  // m_run = -inf on the first step -> 0
    m_run = m_new;
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = exp2f(s[hp][r] - m_new);
        psum += p[r];
      }
      pk[hp * 2 + 0] = pack2(p[0], p[1]);
      pk[hp * 2 + 1] = pack2(p[2], p[3]);
    }
    l_run = l_run * alpha + psum;
    const bf16x8 pf = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
    // zero V of keys past the context (their slots may hold anything)
    uint32_t vmask[2][2];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const int t = t0 + hp * P + 4 * q;
      vmask[hp][0] = (t + 0 < k_end ? 0x0000ffffu : 0u) | (t + 1 < k_end ? 0xffff0000u : 0u);
      vmask[hp][1] = (t + 2 < k_end ? 0x0000ffffu : 0u) | (t + 3 < k_end ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] *= alpha;
      const u32x4 va = {vf[0][db][0] & vmask[0][0], vf[0][db][1] & vmask[0][1],
                        vf[1][db][0] & vmask[1][0], vf[1][db][1] & vmask[1][1]};
      acc[db] = mfma16x16x32(as_bf16x8(va), pf, acc[db]);
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (l16 >= G) return;
  const int h = g * G + l16;
  if (n_parts == 1) {
    const float inv = 1.f / l_tot;
    bf16* orow = attn + (size_t)(row0 + j) * nq * D + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      u32x2 o;
      o[0] = pack2(acc[db][0] * inv, acc[db][1] * inv);
      o[1] = pack2(acc[db][2] * inv, acc[db][3] * inv);
      *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * q) = o;
    }
    return;
  }
  const size_t pidx = ((size_t)j * nq + h) * max_parts + part;
  float* op = o_part + pidx * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(op + db * 16 + 4 * q) = acc[db];
  if (q == 0) {
    ml_part[pidx * 2 + 0] = m_run;
    ml_part[pidx * 2 + 1] = l_tot;
  }
}

// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    int row0, int nq, const int32_t* __restrict__ ctx_lens, const float* __restrict__ o_part,
    const float* __restrict__ ml_part, int max_parts, bf16* __restrict__ attn) {
  const int h = blockIdx.x, j = blockIdx.y;
  const int n_parts = min(max_parts, (ctx_lens[j] + 1 + kDecodePart - 1) / kDecodePart);
  if (n_parts <= 1) return;
  const size_t base = ((size_t)j * nq + h) * max_parts;
  float mmax = -INFINITY;
  for (int p = 0; p < n_parts; ++p) mmax = fmaxf(mmax, ml_part[(base + p) * 2]);
  float lsum = 0.f;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float w = exp2f(ml_part[(base + p) * 2] - mmax);
    lsum += w * ml_part[(base + p) * 2 + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] += w * o_part[(base + p) * D + threadIdx.x * PER + i];
  }
  const float inv = 1.f / lsum;
  bf16* orow = attn + (size_t)(row0 + j) * nq * D + (size_t)h * D + threadIdx.x * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[i] = f2bf(o[i] * inv);
}

static int parts_for(int max_ctx) { return (max_ctx + 1 + kDecodePart - 1) / kDecodePart; }

size_t decode_workspace_bytes(int n_decodes, int nq, int d, int max_ctx) {
  const size_t parts = (size_t)parts_for(max_ctx);
  return (size_t)n_decodes * nq * parts * (d + 2) * sizeof(float) + 256;
}

hipError_t launch_decode_attention(const bf16* qkv, int row0, int nq, int nkv, int d,
                                   const DecDev& dec, const KvDev& kv, bf16* attn, void* ws,
                                   hipStream_t s) {
  if (dec.n == 0) return hipSuccess;
  const int parts = parts_for(dec.max_ctx);
  float* o_part = reinterpret_cast<float*>(ws);
  float* ml_part = o_part + (size_t)dec.n * nq * parts * d;
  dim3 grid(parts, nkv, dec.n);
  if (d == 128) {
    hipLaunchKernelGGL(decode_attn_kernel<128>, grid, dim3(64), 0, s, qkv, row0, nq, nkv,
                       dec.ctx_lens, dec.block_tables, dec.max_blocks, kv, o_part, ml_part, parts,
                       attn);
    if (parts > 1)
      hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(nq, dec.n), dim3(64), 0, s, row0, nq,
                         dec.ctx_lens, o_part, ml_part, parts, attn);
  } else {
    hipLaunchKernelGGL(decode_attn_kernel<64>, grid, dim3(64), 0, s, qkv, row0, nq, nkv,
                       dec.ctx_lens, dec.block_tables, dec.max_blocks, kv, o_part, ml_part, parts,
                       attn);
    if (parts > 1)
      hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(nq, dec.n), dim3(64), 0, s, row0, nq,
                         dec.ctx_lens, o_part, ml_part, parts, attn);
  }
  return hipGetLastError();
}

}  // namespace hl

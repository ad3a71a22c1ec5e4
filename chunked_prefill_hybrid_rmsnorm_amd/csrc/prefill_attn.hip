// Chunk-prefill attention: row i of a chunk (position start_pos + i) attends
// keys 0 .. start_pos + i of its request -- the KV that earlier chunks left in
// the pages plus the chunk's own keys, causally -- read through the chunk's
// block table.  Because every chunk re-reads the KV of all earlier chunks,
// prefilling a prompt in N chunks reads chunk KV N(N-1)/2 extra times; the
// kernel reads each needed page once per (workgroup, kv head) and leaves that
// cost visible rather than hiding it in a cache of its own.
//
// GQA packing: the rows of an MFMA tile are (token, q head) pairs of one kv
// head, row = token * G + head, so one K/V fragment serves all G heads.
//   S^T[key][row] = K[key][:] . q[row][:]           (A = K, token-major page)
//   O^T[dim][row] += V^T[dim][key] P^T[key][row]    (A = V^T, dim-major page)
// Online softmax in base 2; lane l owns row l%16 of each row block.
#include "kernels.h"

namespace hl {

constexpr float kLog2eP = 1.4426950408889634f;
constexpr int kPrefillRB = 2;      // 16-row blocks per wave
constexpr int kPrefillWaves = 4;   // waves per workgroup

template <int D, int RB>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_attn_kernel(
    const bf16* __restrict__ qkv, int nq, int nkv, ChunkList chunks, KvDev kv,
    bf16* __restrict__ attn) {
  constexpr int KS = D / 32, DB = D / 16, P = 16;
  const int c = blockIdx.z, g = blockIdx.y;
  if (c >= chunks.n) return;
  const ChunkDev ch = chunks.c[c];
  const int G = nq / nkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int rows_total = ch.len * G;
  const int rbase = (blockIdx.x * kPrefillWaves + wave) * (16 * RB);
  if (rbase >= rows_total) return;
  const int kv_len = ch.start_pos + ch.len;
  const int ld = (nq + 2 * nkv) * D;

  // this lane's row in each block: token, head, position
  int tok[RB], pos[RB];
  bf16x8 qf[RB][KS];
  int pos_max = 0;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rbase + rb * 16 + l16;
    const bool valid = row < rows_total;
    tok[rb] = valid ? row / G : -1;
    const int hl = row % G;
    pos[rb] = valid ? ch.start_pos + tok[rb] : kv_len - 1;
    const bf16* qp = qkv + (size_t)(ch.row0 + (valid ? tok[rb] : 0)) * ld + (size_t)(g * G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[rb][ks] = valid ? as_bf16x8(ld16(qp + ks * 32 + q * 8)) : as_bf16x8(u32x4{0, 0, 0, 0});
  }
  {
    const int last_row = min(rbase + 16 * RB, rows_total) - 1;
    pos_max = ch.start_pos + last_row / G;
  }
  const int k_stop = pos_max + 1;  // keys [0, k_stop) cover every row of the wave

  const float scale = kLog2eP * rsqrtf((float)D);
  float m_run[RB], l_run[RB];
  f32x4 acc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[rb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int t0 = 0; t0 < k_stop; t0 += 2 * P) {
    int page[2];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const int t = t0 + hp * P, blk = t / P;
      int pg = -1;
      if (t < k_stop && blk < ch.n_blocks) pg = ch.block_table[blk];
      page[hp] = (pg >= 0 && pg < kv.num_pages) ? pg : -1;
    }
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
    // V of keys at or past the end of the request's KV is zeroed
    uint32_t vmask[2][2];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const int t = t0 + hp * P + 4 * q;
      vmask[hp][0] = (t + 0 < kv_len ? 0x0000ffffu : 0u) | (t + 1 < kv_len ? 0xffff0000u : 0u);
      vmask[hp][1] = (t + 2 < kv_len ? 0x0000ffffu : 0u) | (t + 3 < kv_len ? 0xffff0000u : 0u);
    }
    bf16x8 pf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 s[2];
      float smax = -INFINITY;
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        s[hp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[hp] = mfma16x16x32(as_bf16x8(kf[hp][ks]), qf[rb][ks], s[hp]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + hp * P + 4 * q + r;
          s[hp][r] = t <= pos[rb] ? s[hp][r] * scale : -INFINITY;
          smax = fmaxf(smax, s[hp][r]);
        }
      }
      // every row sees key 0 in the first step, so m_new is finite
      smax = fmaxf(smax, __shfl_xor(smax, 16));
      smax = fmaxf(smax, __shfl_xor(smax, 32));
      const float m_new = fmaxf(m_run[rb], smax);
      const float alpha = exp2f(m_run[rb] - m_new);
      m_run[rb] = m_new;
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
      l_run[rb] = l_run[rb] * alpha + psum;
      pf[rb] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[rb][db] *= alpha;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x4 va = {vf[0][db][0] & vmask[0][0], vf[0][db][1] & vmask[0][1],
                        vf[1][db][0] & vmask[1][0], vf[1][db][1] & vmask[1][1]};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb][db] = mfma16x16x32(as_bf16x8(va), pf[rb], acc[rb][db]);
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (tok[rb] < 0) continue;
    const int row = rbase + rb * 16 + l16;
    const int h = g * G + row % G;
    const float inv = 1.f / l_tot;
    bf16* orow = attn + (size_t)(ch.row0 + tok[rb]) * nq * D + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      u32x2 o;
      o[0] = pack2(acc[rb][db][0] * inv, acc[rb][db][1] * inv);
      o[1] = pack2(acc[rb][db][2] * inv, acc[rb][db][3] * inv);
      *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * q) = o;
    }
  }
}

hipError_t launch_prefill_attention(const bf16* qkv, int nq, int nkv, int d,
                                    const ChunkList& chunks, const KvDev& kv, bf16* attn,
                                    hipStream_t s) {
  if (chunks.n == 0 || chunks.n_rows == 0) return hipSuccess;
  const int G = nq / nkv;
  int max_len = 0;
  for (int i = 0; i < chunks.n; ++i) max_len = max(max_len, chunks.c[i].len);
  const int rows_per_wg = 16 * kPrefillRB * kPrefillWaves;
  const int gx = (max_len * G + rows_per_wg - 1) / rows_per_wg;
  if (gx == 0) return hipSuccess;
  dim3 grid(gx, nkv, chunks.n);
  if (d == 128)
    hipLaunchKernelGGL((prefill_attn_kernel<128, kPrefillRB>), grid, dim3(64 * kPrefillWaves), 0,
                       s, qkv, nq, nkv, chunks, kv, attn);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<64, kPrefillRB>), grid, dim3(64 * kPrefillWaves), 0,
                       s, qkv, nq, nkv, chunks, kv, attn);
  return hipGetLastError();
}

}  // namespace hl

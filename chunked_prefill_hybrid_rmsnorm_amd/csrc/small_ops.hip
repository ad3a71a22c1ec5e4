// Row metadata, RMSNorm and RoPE + KV append: the HBM-bound small steps of
// the hybrid-batch layer.
#include "kernels.h"

namespace hl {

// ----------------------------------------------------------------- slots
// Row r < n_rows of the chunks: position start_pos + (r - row0) of its chunk;
// decode row j: position ctx_lens[j].  Slot = page * page_size + offset with
// page = block_table[pos / page_size] (PagedAttention addressing).
__global__ void slot_map_kernel(ChunkList chunks, DecDev dec, int page_size, int num_pages,
                                int32_t* __restrict__ pos_out, int32_t* __restrict__ slot_out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  const int total = chunks.n_rows + dec.n;
  if (r >= total) return;
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
  pos_out[r] = pos;
  slot_out[r] = (page >= 0 && page < num_pages) ? page * page_size + pos % page_size : -1;
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
// One 256-thread block per row; 8 bf16 per thread per step (16-byte loads).
constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ g, bf16* __restrict__ y, int rows,
    int hidden, float eps) {
  const int r = blockIdx.x;
  bf16* yr = y + (size_t)r * hidden;
  const int tid = threadIdx.x;
  if (r >= rows) {  // padding row: zero dummy token
    for (int c = tid * 8; c < hidden; c += kNormThreads * 8)
      *reinterpret_cast<u32x4*>(yr + c) = u32x4{0, 0, 0, 0};
    return;
  }
  const bf16* xr = x + (size_t)r * hidden;
  float ss = 0.f;
  for (int c = tid * 8; c < hidden; c += kNormThreads * 8) {
    u32x4 v = ld16(xr + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = __uint_as_float(v[i] << 16), b = __uint_as_float(v[i] & 0xffff0000u);
      ss += a * a + b * b;
    }
  }
  __shared__ float part[kNormThreads / kWave];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += part[i];
  const float inv = rsqrtf(tot / (float)hidden + eps);
  for (int c = tid * 8; c < hidden; c += kNormThreads * 8) {
    u32x4 v = ld16(xr + c), gv = ld16(g + c), o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = __uint_as_float(v[i] << 16) * inv * __uint_as_float(gv[i] << 16);
      float b = __uint_as_float(v[i] & 0xffff0000u) * inv * __uint_as_float(gv[i] & 0xffff0000u);
      o[i] = pack2(a, b);
    }
    *reinterpret_cast<u32x4*>(yr + c) = o;
  }
}

hipError_t launch_rmsnorm(const bf16* x, const bf16* g, bf16* y, int rows, int rows_padded,
                          int hidden, float eps, hipStream_t s) {
  if (rows_padded == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows_padded), dim3(kNormThreads), 0, s, x, g, y, rows,
                     hidden, eps);
  return hipGetLastError();
}

// ----------------------------------------------------------------- RoPE + append
// One block per row.  Pair i (< d/2) of a head rotates (u_i, u_{i+d/2}) by
// pos * theta^(-2i/d); the angle and its sine/cosine are taken in fp64 so
// long positions lose no precision.  Rotated q and k go back into qkv; K and
// V go to the row's slot (V dimension-major inside the page).
__global__ __launch_bounds__(256) void rope_kv_append_kernel(
    bf16* __restrict__ qkv, const int32_t* __restrict__ pos_in, const int32_t* __restrict__ slot_in,
    int nq, int nkv, int d, float theta, KvDev kv) {
  const int r = blockIdx.x;
  const int half = d >> 1;
  const int ld = (nq + 2 * nkv) * d;
  bf16* row = qkv + (size_t)r * ld;
  const int pos = pos_in[r];
  const int slot = slot_in[r];
  const int page = slot >= 0 ? slot / kv.page_size : -1;
  const int off = slot >= 0 ? slot % kv.page_size : 0;
  const double ln_theta = log((double)theta);
  // rotations of the nq q heads and the nkv k heads
  for (int p = threadIdx.x; p < (nq + nkv) * half; p += blockDim.x) {
    const int h = p / half, i = p % half;
    const double ang = (double)pos * exp(-2.0 * (double)i / (double)d * ln_theta);
    double sd, cd;
    sincos(ang, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    bf16* u = row + h * d;
    const float a = bf2f(u[i]), b = bf2f(u[i + half]);
    const bf16 ra = f2bf(a * c - b * s), rb = f2bf(a * s + b * c);
    u[i] = ra;
    u[i + half] = rb;
    if (h >= nq && page >= 0) {
      bf16* kp = kv.k_page(page, h - nq) + (size_t)off * d;
      kp[i] = ra;
      kp[i + half] = rb;
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
  hipLaunchKernelGGL(rope_kv_append_kernel, dim3(rows), dim3(256), 0, s, qkv, pos, slot, nq, nkv,
                     d, theta, kv);
  return hipGetLastError();
}

}  // namespace hl

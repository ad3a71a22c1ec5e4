// Shared device helpers for the hybrid-batch layer kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hybrid_layer.h"

namespace hl {

typedef uint16_t bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16 f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16, h);
}

// two fp32 -> two bf16 (round to nearest even) in one 32-bit word, a low
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// D = A(16x32) * B(32x16) + C.  Lane l supplies A[l%16][8*(l/16) .. +8] and
// B[8*(l/16) .. +8][l%16]; it receives C[4*(l/16) + r][l%16], r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 a, const bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// inclusive prefix sum over the wave's lanes
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): `lds` is the
// wave-uniform base and lane i's bytes land at lds + 16 i, no registers involved.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)lds, 16, 0, 0);
}

// s_waitcnt with only the vector-memory counter: wait until at most n remain.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

// Chunk descriptors passed by value to kernels.
struct ChunkDev {
  int32_t len, start_pos, row0, n_blocks;
  const int32_t* block_table;
};
struct ChunkList {
  int32_t n;
  int32_t n_rows;  // sum of len
  ChunkDev c[HL_MAX_CHUNKS];
};

// Per-launch view of the paged KV cache.  Page layout, bf16:
//   K: [n_kv][page_size][head_dim]   (token-major)
//   V: [n_kv][head_dim][page_size]   (dimension-major, i.e. transposed)
// K block first, then V block; one page is 2 * n_kv * page_size * head_dim.
struct KvDev {
  bf16* data;
  int32_t num_pages, n_kv, head_dim, page_size;
  __device__ __forceinline__ size_t page_elems() const {
    return (size_t)2 * n_kv * page_size * head_dim;
  }
  __device__ __forceinline__ bf16* k_page(int page, int g) const {
    return data + (size_t)page * page_elems() + (size_t)g * page_size * head_dim;
  }
  __device__ __forceinline__ bf16* v_page(int page, int g) const {
    return data + (size_t)page * page_elems() + (size_t)(n_kv + g) * page_size * head_dim;
  }
};

}  // namespace hl

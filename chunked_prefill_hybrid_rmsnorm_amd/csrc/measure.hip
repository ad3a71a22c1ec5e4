// Measurement aid: the HBM read rate a plain streaming kernel attains on this
// GPU, the attainable bandwidth the memory-bound kernels of the layer are
// read against beside the 8 TB/s of the data sheet.
#include <hip/hip_runtime.h>

#include "common.h"
#include "hybrid_layer.h"

namespace hl {

constexpr int kReadWgs = 8192;  // workgroups of 256 lanes
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per lane
constexpr size_t kReadQuantum = (size_t)kReadWgs * 256 * kReadUnroll * 16;  // 256 MiB

// Every lane streams 16-byte non-temporal loads, kReadUnroll at a time,
// grid-stride over n16 16-byte words (a multiple of the grid's lanes x
// kReadUnroll); workgroup b stores the XOR of every 32-bit word it read to
// sink[b] (one plain store per workgroup, so no two workgroups meet on a word).
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t nth = (size_t)gridDim.x * blockDim.x;
  u32x4 x = {0, 0, 0, 0};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += kReadUnroll * nth) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * nth);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u];
  }
  uint32_t w = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) w ^= __shfl_xor(w, o);
  __shared__ uint32_t wave_x[4];
  if ((threadIdx.x & 63) == 0) wave_x[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = wave_x[0] ^ wave_x[1] ^ wave_x[2] ^ wave_x[3];
}

}  // namespace hl

using namespace hl;

extern "C" int hl_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return HL_ERR_NULL;
  if (bytes == 0 || bytes % kReadQuantum || (reinterpret_cast<uintptr_t>(buf) & 15))
    return HL_ERR_SHAPE;
  hipLaunchKernelGGL(read_stream_kernel, dim3(kReadWgs), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? HL_OK : HL_ERR_LAUNCH;
}

// The two steps a batching loop adds around the layers: the embedding lookup
// of each batch row's input token, and the greedy choice of the next token
// from the LM head's logits.  Both are plain definitions (a row gather; an
// argmax with ties to the lowest id).
#include "hybrid_layer.h"
#include "kernels.h"

namespace hl {

// Row r's token: row_tok[r] >= 0 is a prompt token id; row_tok[r] = -(q+1)
// reads the last token chosen for request q (last_tok[q], q < n_last).  Ids
// and request slots out of range are clamped, so a bad entry reads a real row
// instead of memory past the arrays.  8 bf16 per thread per step.
__global__ __launch_bounds__(256) void embed_rows_kernel(const bf16* __restrict__ table,
                                                         int vocab, int hidden,
                                                         const int32_t* __restrict__ row_tok,
                                                         const int32_t* __restrict__ last_tok,
                                                         int n_last, bf16* __restrict__ out) {
  const int r = blockIdx.x;
  const int t = row_tok[r];
  int id = t;
  if (t < 0) id = n_last > 0 ? last_tok[min(-(t + 1), n_last - 1)] : 0;
  id = min(max(id, 0), vocab - 1);
  const bf16* src = table + (size_t)id * hidden;
  bf16* dst = out + (size_t)r * hidden;
  for (int c = threadIdx.x * 8; c < hidden; c += 256 * 8)
    *reinterpret_cast<u32x4*>(dst + c) = ld16(src + c);
}

// One 256-thread block per row with 0 <= sample_req[r] < n_last: the id of
// the largest logit (ties: the lowest id; NaN never wins; a row with no
// number picks 0) goes to last_tok[sample_req[r]] and, when 0 <= sample_pos[r]
// < n_out, to out_tokens[sample_pos[r]].
__global__ __launch_bounds__(256) void argmax_rows_kernel(const bf16* __restrict__ logits,
                                                          int vocab,
                                                          const int32_t* __restrict__ sample_req,
                                                          const int32_t* __restrict__ sample_pos,
                                                          int32_t* __restrict__ last_tok,
                                                          int n_last,
                                                          int32_t* __restrict__ out_tokens,
                                                          int n_out) {
  const int r = blockIdx.x;
  const int q = sample_req[r];
  if (q < 0 || q >= n_last) return;
  const bf16* row = logits + (size_t)r * vocab;
  float best = -INFINITY;
  int best_id = vocab;  // past the end: loses every tie
  for (int v = threadIdx.x; v < vocab; v += 256) {
    const float x = bf2f(row[v]);
    if (x > best) {  // strictly greater: the first (lowest) id of a tie stays
      best = x;
      best_id = v;
    }
  }
  // wave reduction: larger value wins, equal values go to the lower id
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oi = __shfl_xor(best_id, o);
    if (ob > best || (ob == best && oi < best_id)) {
      best = ob;
      best_id = oi;
    }
  }
  __shared__ float sb[4];
  __shared__ int si[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sb[wave] = best;
    si[wave] = best_id;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (sb[w] > best || (sb[w] == best && si[w] < best_id)) {
        best = sb[w];
        best_id = si[w];
      }
    if (best_id >= vocab) best_id = 0;  // every logit NaN or -inf
    last_tok[q] = best_id;
    const int p = sample_pos[r];
    if (p >= 0 && p < n_out) out_tokens[p] = best_id;
  }
}

}  // namespace hl

using namespace hl;

extern "C" {

int hl_embed_rows(const hl_bf16* table, int32_t vocab, int32_t hidden, const int32_t* row_tok,
                  const int32_t* last_tok, int32_t n_last, int32_t rows, hl_bf16* out,
                  hipStream_t stream) {
  if (rows < 0 || vocab <= 0 || hidden <= 0 || hidden % 8 || n_last < 0) return HL_ERR_SHAPE;
  if (rows == 0) return HL_OK;
  if (!table || !row_tok || !out || (n_last > 0 && !last_tok)) return HL_ERR_NULL;
  hipLaunchKernelGGL(embed_rows_kernel, dim3(rows), dim3(256), 0, stream,
                     reinterpret_cast<const bf16*>(table), vocab, hidden, row_tok, last_tok, n_last,
                     reinterpret_cast<bf16*>(out));
  return hipGetLastError() == hipSuccess ? HL_OK : HL_ERR_LAUNCH;
}

int hl_argmax_rows(const hl_bf16* logits, int32_t rows, int32_t vocab, const int32_t* sample_req,
                   const int32_t* sample_pos, int32_t* last_tok, int32_t n_last,
                   int32_t* out_tokens, int32_t n_out, hipStream_t stream) {
  if (rows < 0 || vocab <= 0 || n_last < 0 || n_out < 0) return HL_ERR_SHAPE;
  if (rows == 0) return HL_OK;
  if (!logits || !sample_req || !sample_pos || !last_tok || !out_tokens) return HL_ERR_NULL;
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(rows), dim3(256), 0, stream,
                     reinterpret_cast<const bf16*>(logits), vocab, sample_req, sample_pos, last_tok,
                     n_last, out_tokens, n_out);
  return hipGetLastError() == hipSuccess ? HL_OK : HL_ERR_LAUNCH;
}

}  // extern "C"

// Internal launchers shared by the C-ABI layer (api.hip) and the kernels.
#pragma once
#include "common.h"

namespace hl {

struct DecDev {
  int32_t n;
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t max_ctx;
};

// positions / slots of rows [0, chunks.n_rows + dec.n)
hipError_t launch_slot_map(const ChunkList& chunks, const DecDev& dec, int page_size,
                           int num_pages, int32_t* pos, int32_t* slot, hipStream_t s);

hipError_t launch_rmsnorm(const bf16* x, const bf16* g, bf16* y, int rows, int rows_padded,
                          int hidden, float eps, hipStream_t s);

enum GemmEpilogue { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2 };
// c = a w^T (+ residual) / swiglu(a w_gate^T, a w_up^T).  ws holds split-K
// partials (gemm_workspace_bytes); with ws == nullptr K is not split.
// Launchers of two kernels record `mid` (when not null) on the stream between
// the first and the second, also when the second is not needed.
size_t gemm_workspace_bytes(GemmEpilogue epi, int m_padded, int n, int k);
// act = silu(a w_gate^T) * (a w_up^T) with one wave per SIMD and the
// accumulators in AGPRs (gemm_agpr.hip): 288- (or 256-, rows256) row tiles
// of 112 outputs, no K split.
hipError_t launch_swiglu_agpr(const bf16* a, const bf16* wg, const bf16* wu, bf16* act, int mp,
                              int f, int k, bool rows256, hipStream_t s);
// One-wave-per-SIMD plain / residual GEMM (gemm_agpr.hip): BM = 288 (or 256
// with rows256) x 32 fn weight rows per tile, fn in {4, 5, 7}; with splits > 1
// it writes fp32 partials [splits][mp][n] to `part` instead of c.
hipError_t launch_gemm_agpr(GemmEpilogue epi, int fn, const bf16* a, const bf16* w, bf16* c,
                            const bf16* r, float* part, int m, int mp, int n, int k, int splits,
                            bool rows256, hipStream_t s);
hipError_t launch_gemm(GemmEpilogue epi, const bf16* a, const bf16* w, const bf16* w2, bf16* c,
                       const bf16* residual, void* ws, int m, int m_padded, int n, int k,
                       hipStream_t s, hipEvent_t mid = nullptr);
// K splits launch_gemm would use for this shape with a workspace
int gemm_splits(GemmEpilogue epi, int m_padded, int n, int k);
// Plain-store GEMM that leaves its split-K partials in ws for a consumer that
// reduces them itself (gemm_splits(...) > 1 planes of [m_padded][n] fp32)
hipError_t launch_gemm_partials(const bf16* a, const bf16* w, void* ws, int m, int m_padded, int n,
                                int k, hipStream_t s);

// h = a w^T + residual (rows < m) followed by y = RMSNorm(h; g, eps) (rows
// < m_padded, pad rows zero); with split K the norm runs inside the reduce.
hipError_t launch_gemm_residual_norm(const bf16* a, const bf16* w, bf16* h, const bf16* residual,
                                     const bf16* g, bf16* y, float eps, void* ws, int m,
                                     int m_padded, int n, int k, hipStream_t s,
                                     hipEvent_t mid = nullptr);

hipError_t launch_rope_kv_append(bf16* qkv, const int32_t* pos, const int32_t* slot, int rows,
                                 int nq, int nkv, int d, float theta, const KvDev& kv,
                                 hipStream_t s);
// theta^(-2 i / d) for the rotation pairs of a head (d / 2 <= kRopeMaxPairs),
// computed on the host in fp64 and passed by value
constexpr int kRopeMaxPairs = 64;
struct RopeFreq {
  double inv[kRopeMaxPairs];
};

// RoPE on q / k and KV append, each row's position, slot and cos / sin
// resolved in the kernel; with `part` (split-K partials of the QKV
// projection, `splits` planes of Mp rows) the rows are first formed from them
// and rows [rows, Mp) of qkv are zeroed.
hipError_t launch_rope_append_wide(bf16* qkv, const float* part, int splits, int rows, int Mp,
                                   int nq, int nkv, int d, float theta, const ChunkList& chunks,
                                   const DecDev& dec, const KvDev& kv, hipStream_t s);

// ws (prefill_workspace_bytes) holds key-split partials; nullptr: no split.
size_t prefill_workspace_bytes(const ChunkList& chunks, int nq, int nkv, int d);
size_t prefill_workspace_bound(int rows, int nq, int nkv, int d);
hipError_t launch_prefill_attention(const bf16* qkv, int nq, int nkv, int d,
                                    const ChunkList& chunks, const KvDev& kv, bf16* attn,
                                    void* ws, hipStream_t s);

size_t decode_workspace_bytes(int n_decodes, int nq, int nkv, int d, int max_ctx);
// Prefill rows and decode rows in one launch (plus one merge when keys were
// split); pf_ws / dc_ws as for the two launchers below.
hipError_t launch_attention(const bf16* qkv, int nq, int nkv, int d, const ChunkList& chunks,
                            const DecDev& dec, int dec_row0, const KvDev& kv, bf16* attn,
                            void* pf_ws, void* dc_ws, hipStream_t s, hipEvent_t mid = nullptr);
hipError_t launch_decode_attention(const bf16* qkv, int row0, int nq, int nkv, int d,
                                   const DecDev& dec, const KvDev& kv, bf16* attn, void* ws,
                                   hipStream_t s);

}  // namespace hl

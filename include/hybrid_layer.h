/*
 * hybrid_layer.h -- C ABI of the MI355X (gfx950) hybrid-batch decoder layer.
 *
 * One call runs one pre-norm GQA decoder layer over a *hybrid batch*: the
 * rows of one or more prefill chunks followed by one row per piggybacked
 * decode, stacked into a single [M = Lp + Bd, H] matrix.
 *
 * Where the operation comes from (pages on SARATHI / Sarathi-Serve):
 *  - chunked prefill: a prompt is cut into fixed-size chunks computed over
 *    several iterations; each chunk must attend to the KV of the earlier
 *    chunks (intelliparadigm.com article, section 3.1; Sarathi-Serve digest,
 *    section 2, Q2 item 1);
 *  - decode-maximal batching: one chunk plus decodes form one batch
 *    (intelliparadigm.com section 3.2; SARATHI summary on gitcode.csdn.net,
 *    part 2 item 2);
 *  - the linear layers run once on the concatenated [Lp+Bd, H] matrix,
 *    attention is split by pointer offset into the prefill part and the
 *    paged decode part, and results land in preallocated contiguous memory
 *    for the next layer (gitcode.csdn.net part 2 item 3,
 *    "merge / split / merge"; intelliparadigm.com section 3.3);
 *  - each chunk keeps its own position ids so positions run on across
 *    chunks (intelliparadigm.com section 6.1);
 *  - the hybrid batch rows are padded to a tile multiple with dummy rows
 *    (intelliparadigm.com section 4.3; gitcode.csdn.net part 3 item 3).
 *
 * Conventions shared by every entry point:
 *  - bf16 values are passed as uint16_t bit patterns (hl_bf16);
 *  - every pointer to data is a DEVICE pointer owned by the caller unless
 *    stated otherwise; the library allocates nothing, frees nothing and keeps
 *    no pointer after it returns; its only global state is a per-device
 *    cache of the attention kernel's occupancy, filled on first use and safe
 *    to fill from several threads, so calls on different streams with
 *    different workspaces may run concurrently;
 *  - calls only enqueue work on `stream` (0 = the null stream) and return;
 *    none synchronises except hl_validate_metadata;
 *  - return value: HL_OK (0) or a negative HL_ERR_* code; nothing is
 *    enqueued when a check fails; no exception crosses the ABI.
 */
#ifndef HYBRID_LAYER_H
#define HYBRID_LAYER_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HL_OK 0
#define HL_ERR_NULL (-1)        /* a required pointer is NULL */
#define HL_ERR_SHAPE (-2)       /* sizes inconsistent or not multiples the kernels need */
#define HL_ERR_UNSUPPORTED (-3) /* head_dim not 64/128, page_size not 16, too many chunks,
                                   a weight matrix of 4 GiB or more */
#define HL_ERR_WORKSPACE (-4)   /* ws_bytes smaller than hl_workspace_bytes() */
#define HL_ERR_LAUNCH (-5)      /* a kernel launch failed (hipGetLastError) */
#define HL_ERR_METADATA (-6)    /* hl_validate_metadata found a bad table entry */
#define HL_ERR_HIP (-7)         /* a HIP runtime call failed */

#define HL_MAX_CHUNKS 16

typedef uint16_t hl_bf16;

/* Layer shape.  hidden, ffn and n_q_heads*head_dim must be multiples of 64,
 * hidden at most 16384 (HL_ERR_UNSUPPORTED); n_q_heads a multiple of
 * n_kv_heads; head_dim 64 or 128; page_size 16. */
typedef struct {
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, ffn, page_size;
  float rms_eps;    /* added to mean(x^2) inside the square root */
  float rope_theta; /* RoPE base */
} hl_config;

/* Layer weights, bf16, every matrix [out, in] row-major (the GEMMs compute
 * y = x W^T).  w_qkv stacks n_q_heads q heads, then n_kv_heads k heads, then
 * n_kv_heads v heads, head_dim rows each. */
typedef struct {
  const hl_bf16* w_qkv;  /* [(nq + 2 nkv) d, H] */
  const hl_bf16* w_o;    /* [H, nq d] */
  const hl_bf16* w_gate; /* [F, H] */
  const hl_bf16* w_up;   /* [F, H] */
  const hl_bf16* w_down; /* [H, F] */
  const hl_bf16* g_attn; /* [H] RMSNorm gain before attention */
  const hl_bf16* g_ffn;  /* [H] RMSNorm gain before the FFN */
} hl_weights;

/* One prefill chunk: `len` rows holding positions start_pos .. start_pos+len-1
 * of one request.  block_table (device, int32 [n_blocks]) maps position p to
 * page block_table[p / page_size]; it must cover positions [0, start_pos+len):
 * tokens before start_pos are already cached (earlier chunks). */
typedef struct {
  int32_t len;
  int32_t start_pos;
  const int32_t* block_table;
  int32_t n_blocks;
} hl_chunk;

/* Piggybacked decodes, one row each.  Decode j has ctx_lens[j] cached tokens;
 * its new token sits at position ctx_lens[j], is appended there and attends
 * ctx_lens[j] + 1 keys.  block_tables is device int32 [n, max_blocks].
 * Row j of block_tables must cover positions [0, ctx_lens[j]] (device
 * contents are trusted; hl_validate_metadata checks them).  max_ctx is a
 * HOST-side upper bound of ctx_lens: it sizes the decode workspace and caps
 * how many key slices the decode attention cuts all decodes' keys into, with
 * no device read.  Every key of every decode is visited whatever max_ctx
 * says; an underestimate only makes the slices longer. */
typedef struct {
  int32_t n;
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t max_ctx;
} hl_decodes;

/* Paged KV cache of one layer (device).  num_pages pages; page layout bf16:
 *   K: [n_kv][page_size][head_dim]  token-major,
 *   V: [n_kv][head_dim][page_size]  dimension-major (V transposed per page),
 * K block first, then V block: 2 * n_kv * page_size * head_dim per page.
 * K is stored after the rotary embedding.  Updated in place. */
typedef struct {
  hl_bf16* data;
  int32_t num_pages;
} hl_kv;

/* Optional intermediate buffers (device, nullable).  A non-NULL pointer
 * replaces the workspace region of that intermediate, so the caller sees it
 * without a copy.  Rows: Mp = M rounded up to `pad`.
 *   xn1 [Mp, H], qkv [Mp, (nq+2nkv) d] (q and k after RoPE), attn [Mp, nq d],
 *   h [Mp, H] (rows >= M unwritten), xn2 [Mp, H], act [Mp, F]. */
typedef struct {
  hl_bf16 *xn1, *qkv, *attn, *h, *xn2, *act;
} hl_taps;

/* Text for an HL_* code (static storage). */
const char* hl_error_string(int code);

/* Bytes of workspace hl_layer_forward needs for at most max_rows rows
 * (chunk rows + decodes), max_decodes decodes with contexts up to max_ctx, and
 * row padding `pad` (positive multiple of 16).  Host only.  Nondecreasing in
 * max_rows, max_decodes and max_ctx: a workspace of this size serves every
 * call with at most that many rows, decodes and cached tokens. */
int hl_workspace_bytes(const hl_config* cfg, int32_t max_rows, int32_t max_decodes,
                       int32_t max_ctx, int32_t pad, size_t* bytes);

/* One decoder-layer forward over the hybrid batch.
 *   x   [M, H] input rows: chunk rows in chunk order, then one row per decode;
 *   out [M, H] output rows (must not alias x);
 *   ws  device workspace of ws_bytes >= hl_workspace_bytes(cfg, M, dec->n,
 *       dec->max_ctx, pad), 256-byte aligned;
 *   pad row padding: the GEMMs run on Mp = ceil(M/pad)*pad rows, the pad rows
 *       being zero dummy tokens that write no KV and reach no output.
 * Steps, all on `stream`: RMSNorm; fused QKV GEMM; each row's position and
 * KV slot, RoPE on q and k and append of K/V into the pages; attention -- the
 * chunk-prefill rows (causal within the chunk, paged KV of earlier chunks)
 * and the paged split-K decode rows in one launch; O GEMM + residual and
 * RMSNorm; gate/up GEMM + SwiGLU; down GEMM + residual.  Writes exactly M KV
 * slots. */
int hl_layer_forward(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                     const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                     const hl_kv* kv, hl_bf16* out, void* ws, size_t ws_bytes, int32_t pad,
                     const hl_taps* taps, hipStream_t stream);

/* The same forward, recording stage_events[i] (caller-created HIP events,
 * HL_N_STAGES + 1 of them) on `stream` before kernel slot i and stage_events
 * [HL_N_STAGES] after the last, so that the caller can time every kernel of
 * the real sequence.  A slot holds at most one kernel; a slot whose kernel is
 * not needed for this batch (a split-K reduce or a key-split merge that the
 * launch shape makes unnecessary) times as an empty interval.  hl_stage_name(i)
 * names slot i. */
#define HL_N_STAGES 11
int hl_layer_forward_timed(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                           const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                           const hl_kv* kv, hl_bf16* out, void* ws, size_t ws_bytes, int32_t pad,
                           const hl_taps* taps, hipEvent_t* stage_events, hipStream_t stream);
const char* hl_stage_name(int stage);

/* Cross-layer fusion of the first RMSNorm.  In a stack of layers the input
 * of layer l + 1 is the output of layer l, which the results of a layer are
 * written for (preallocated contiguous memory handed to the next layer:
 * gitcode.csdn.net SARATHI summary, part 2 item 3).  Layer l's last kernel,
 * the split-K reduce of the down projection, holds whole output rows, so it
 * can also store layer l + 1's normalised input, and layer l + 1 skips its
 * own RMSNorm launch.  Fields (device pointers, each may be NULL):
 *   xn_in   [Mp, H]: RMSNorm(x) * g_attn of THIS layer with eps =
 *           cfg->rms_eps and pad rows zero, as the previous call's xn_next
 *           left it (not checked).  When set, the layer's own RMSNorm is not
 *           run (its stage slot times empty) and taps->xn1 is not written.
 *   g_next  [H]: gain of the RMSNorm applied to this layer's output (the
 *           next layer's g_attn, or the model's final norm).
 *   xn_next [Mp, H]: receives RMSNorm(out) * g_next with eps =
 *           cfg->rms_eps, pad rows zero; required when g_next is set and
 *           must alias none of x, out, xn_in (HL_ERR_SHAPE).
 * Mp = M rounded up to `pad`, as for the taps. */
typedef struct {
  const hl_bf16* xn_in;
  const hl_bf16* g_next;
  hl_bf16* xn_next;
} hl_chain;

/* hl_layer_forward with the cross-layer RMSNorm fusion above (chain NULL:
 * the same as hl_layer_forward) and, when stage_events is not NULL, the stage
 * events of hl_layer_forward_timed.  Workspace as for hl_layer_forward. */
int hl_layer_forward_chain(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                           const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                           const hl_kv* kv, hl_bf16* out, void* ws, size_t ws_bytes, int32_t pad,
                           const hl_taps* taps, const hl_chain* chain, hipEvent_t* stage_events,
                           hipStream_t stream);

/* hl_layer_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a device array inside
 * the library, HL_NOALLOC_SCRATCH_BYTES (160 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends; this call allocates
 * and frees nothing.  Every other argument as for hl_layer_forward.
 * Errors: HL_ERR_WORKSPACE (nothing enqueued) when the batch needs more than
 * HL_NOALLOC_SCRATCH_BYTES, i.e. hl_workspace_bytes(cfg, M, dec->n,
 * dec->max_ctx, pad) > HL_NOALLOC_SCRATCH_BYTES; HL_ERR_UNSUPPORTED when
 * `stream` belongs to a device other than the current one; HL_ERR_HIP when
 * the array's device address cannot be looked up.  No part of the array
 * needs to start at zero: every region is written before it is read within
 * one call.  All calls on one GPU share the array, so calls that overlap in
 * time on one GPU (different streams, or threads) race and give wrong
 * results; calls on one stream run in order and are safe. */
#define HL_NOALLOC_SCRATCH_BYTES (160u << 20)
int hl_layer_forward_noalloc(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                             const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                             const hl_kv* kv, hl_bf16* out, int32_t pad, const hl_taps* taps,
                             hipStream_t stream);

/* Row positions and KV slots of a hybrid batch (PagedAttention addressing:
 * slot = block_table[pos / page_size] * page_size + pos % page_size).
 * positions, slots: device int32 [M], M = sum of chunk lens + dec->n.  A row
 * whose block-table index is out of range gets slot -1. */
int hl_slot_mapping(const hl_config* cfg, const hl_chunk* chunks, int32_t n_chunks,
                    const hl_decodes* dec, int32_t num_pages, int32_t* positions,
                    int32_t* slots, hipStream_t stream);

/* Debug check of the metadata (synchronises `stream`, copies the tables to
 * the host): every page id needed is in [0, num_pages), block tables are long
 * enough, ctx_lens <= max_ctx, and no two requests share a page. */
int hl_validate_metadata(const hl_config* cfg, const hl_chunk* chunks, int32_t n_chunks,
                         const hl_decodes* dec, int32_t num_pages, hipStream_t stream);

/* ---- single steps, same kernels as hl_layer_forward (for per-step checks) */

/* y[r] = x[r] / sqrt(mean(x[r]^2) + eps) * g for r < rows; y[r] = 0 for
 * rows <= r < rows_padded.  x [rows, hidden], y [rows_padded, hidden]. */
int hl_rmsnorm(const hl_bf16* x, const hl_bf16* g, hl_bf16* y, int32_t rows,
               int32_t rows_padded, int32_t hidden, float eps, hipStream_t stream);

/* c[m, n] = sum_k a[m, k] w[n, k] (+ residual[m, n]) in fp32, rounded to bf16.
 * a [m_padded, k], w [n, k], c and residual [*, n] row-major.  Without a
 * residual all m_padded rows are written; with one only the first m rows.
 * k multiple of 64, n multiple of 64, m_padded multiple of 16.  ws (device,
 * 16-byte aligned, ws_bytes >= hl_gemm_workspace_bytes) lets the kernel split
 * K over more workgroups; with ws == NULL K is not split (same results up to
 * fp32 summation order).  HL_ERR_UNSUPPORTED when a or w spans 4 GiB or more
 * (max(m_padded, n) * k * 2 bytes). */
int hl_gemm_bf16(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, const hl_bf16* residual,
                 int32_t m, int32_t m_padded, int32_t n, int32_t k, void* ws, size_t ws_bytes,
                 hipStream_t stream);
int hl_gemm_workspace_bytes(int32_t m_padded, int32_t n, int32_t k, size_t* bytes);

/* act[m, f] = silu(sum_k a[m,k] w_gate[f,k]) * sum_k a[m,k] w_up[f,k] for
 * m < m_padded; silu(z) = z / (1 + exp(-z)).  a [m_padded, k],
 * w_gate/w_up [f, k], act [m_padded, f].  HL_ERR_UNSUPPORTED when a or a
 * weight spans 4 GiB or more. */
int hl_gemm_swiglu(const hl_bf16* a, const hl_bf16* w_gate, const hl_bf16* w_up, hl_bf16* act,
                   int32_t m_padded, int32_t f, int32_t k, hipStream_t stream);

/* RoPE on the q and k heads of qkv rows [0, rows) at positions[r] (rotate-half
 * pairing of element i with i + d/2, angle pos * theta^(-2i/d)), written back
 * in place, and append of K (rotated) and V into kv at slots[r].  A row whose
 * slot is negative or names a page >= kv->num_pages is rotated but writes no
 * KV.  qkv [rows, (nq + 2nkv) d]. */
int hl_rope_kv_append(const hl_config* cfg, hl_bf16* qkv, const int32_t* positions,
                      const int32_t* slots, int32_t rows, const hl_kv* kv, hipStream_t stream);

/* Chunk-prefill attention.  Chunk c's rows start at row sum_{i<c} len_i of
 * qkv (q already rotated, its own K/V already appended); row i of the chunk
 * (position start_pos + i) attends keys 0 .. start_pos + i through the
 * chunk's block table.  Writes attn rows of the chunks ([*, nq d]).  ws
 * (device, 16-byte aligned, >= hl_prefill_workspace_bytes) lets the kernel
 * split long key ranges over more workgroups; ws == NULL: no split. */
int hl_prefill_attention(const hl_config* cfg, const hl_bf16* qkv, const hl_chunk* chunks,
                         int32_t n_chunks, const hl_kv* kv, hl_bf16* attn, void* ws,
                         size_t ws_bytes, hipStream_t stream);
int hl_prefill_workspace_bytes(const hl_config* cfg, const hl_chunk* chunks, int32_t n_chunks,
                               size_t* bytes);

/* Paged decode attention.  The 32-key steps of all decodes are cut into equal
 * slices, one per wave, and decodes split over slices are merged afterwards.
 * Decode j reads its q from qkv row row0 + j and writes attn row row0 + j.
 * ws (device, 16-byte aligned, HL_ERR_WORKSPACE otherwise) needs
 * hl_decode_workspace_bytes(cfg, dec->n, dec->max_ctx). */
int hl_decode_attention(const hl_config* cfg, const hl_bf16* qkv, int32_t row0,
                        const hl_decodes* dec, const hl_kv* kv, hl_bf16* attn, void* ws,
                        size_t ws_bytes, hipStream_t stream);
int hl_decode_workspace_bytes(const hl_config* cfg, int32_t n_decodes, int32_t max_ctx,
                              size_t* bytes);

/* ---------------------------------------------------------------------------
 * Around the layers, for a batching loop (Sarathi-Serve digest, Algorithm 3:
 * each iteration runs one hybrid batch and every decode row, and every chunk
 * that finishes its prompt, yields one new token; greedy choice).
 */

/* out[r] = table[id_r] for r < rows, where id_r = row_tok[r] when >= 0, else
 * last_tok[-(row_tok[r] + 1)] (the token last chosen for that request slot).
 * table [vocab, hidden] bf16 (hidden a multiple of 8), out [rows, hidden];
 * row_tok [rows] and last_tok [n_last] are device int32.  Ids outside
 * [0, vocab) and slots outside [0, n_last) are clamped to the nearest valid
 * one (no read past the arrays).  last_tok may be NULL when n_last == 0. */
int hl_embed_rows(const hl_bf16* table, int32_t vocab, int32_t hidden, const int32_t* row_tok,
                  const int32_t* last_tok, int32_t n_last, int32_t rows, hl_bf16* out,
                  hipStream_t stream);

/* Greedy next token of the rows that sample: for each r < rows with
 * 0 <= sample_req[r] < n_last, the id of the largest of logits[r][0..vocab)
 * (ties: the lowest id; NaN never wins; a row with no number gives 0) is
 * written to last_tok[sample_req[r]] and, when 0 <= sample_pos[r] < n_out, to
 * out_tokens[sample_pos[r]].  logits [rows, vocab] bf16; every other array is
 * device int32.  Rows with sample_req[r] < 0 are skipped. */
int hl_argmax_rows(const hl_bf16* logits, int32_t rows, int32_t vocab, const int32_t* sample_req,
                   const int32_t* sample_pos, int32_t* last_tok, int32_t n_last,
                   int32_t* out_tokens, int32_t n_out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Measurement aid.
 */

/* Reads the `bytes` bytes at buf once, with the plainest streaming pattern
 * (16-byte non-temporal vector loads, 8192 workgroups of 256 lanes, eight
 * loads in flight per lane).  Workgroup b stores the XOR of the 32-bit words
 * it read to sink[b], so the XOR of sink[0..8192) is that of the whole
 * buffer.  Timed over buffers larger than the 256 MB MALL it gives the HBM
 * read rate this GPU attains, the bandwidth term of the roofline
 * (Sarathi-Serve digest, section 4) as measured rather than as specified.
 * buf device, 16-byte aligned; bytes a positive multiple of 256 MiB
 * (HL_ERR_SHAPE otherwise); sink device uint32 [8192]. */
int hl_read_stream(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HYBRID_LAYER_H */

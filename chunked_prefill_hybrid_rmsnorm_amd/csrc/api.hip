// C ABI of the hybrid-batch decoder layer: argument checks, workspace
// layout and the sequence of kernels on the caller's stream.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "kernels.h"

using namespace hl;

// Workspace of hl_layer_forward_noalloc: a device array of fixed size, one
// copy per GPU, held from the module's load on that GPU to the end of the
// process.  Host code never passes its name to a kernel (on the host the name
// is only a stand-in); it passes the device address looked up per device.
static __device__ __align__(256) char scratch[HL_NOALLOC_SCRATCH_BYTES];

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The GEMM copies address A and W by 32-bit byte offsets.
bool gemm_fits_offsets(int m_padded, int n, int k) {
  return (size_t)std::max(m_padded, n) * k * 2 <= UINT32_MAX;
}
int round_up(int x, int m) { return (x + m - 1) / m * m; }

int check_config(const hl_config* c) {
  if (!c) return HL_ERR_NULL;
  if (c->head_dim != 64 && c->head_dim != 128) return HL_ERR_UNSUPPORTED;
  if (c->page_size != 16) return HL_ERR_UNSUPPORTED;
  if (c->hidden <= 0 || c->ffn <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0)
    return HL_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads) return HL_ERR_SHAPE;
  if (c->n_q_heads / c->n_kv_heads > 16) return HL_ERR_UNSUPPORTED;
  if (c->hidden % 64 || c->ffn % 64 || (c->n_q_heads * c->head_dim) % 64) return HL_ERR_SHAPE;
  // the row-wise RMSNorm kernels hold a row in the registers of 256 threads
  if (c->hidden > 16384) return HL_ERR_UNSUPPORTED;
  // the GEMM copies address each weight matrix by 32-bit byte offsets
  const size_t nqkv = (size_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
  if (std::max({nqkv, (size_t)c->ffn, (size_t)c->n_q_heads * c->head_dim}) * c->hidden * 2 >
      UINT32_MAX)
    return HL_ERR_UNSUPPORTED;
  return HL_OK;
}

struct Layout {
  int Mp;
  size_t xn1, qkv, attn, h, xn2, act, dec, pre, gemm, total;
};

Layout make_layout(const hl_config* c, int rows, int n_dec, int max_ctx, int pad) {
  Layout L{};
  L.Mp = round_up(std::max(rows, 1), pad);
  const size_t Mp = L.Mp;
  const size_t H = c->hidden, F = c->ffn, d = c->head_dim;
  const size_t nqkv = (size_t)(c->n_q_heads + 2 * c->n_kv_heads) * d;
  size_t o = 0;
  L.xn1 = o;  o = align256(o + Mp * H * 2);
  L.qkv = o;  o = align256(o + Mp * nqkv * 2);
  L.attn = o; o = align256(o + Mp * c->n_q_heads * d * 2);
  L.h = o;    o = align256(o + Mp * H * 2);
  L.xn2 = o;  o = align256(o + Mp * H * 2);
  L.act = o;  o = align256(o + Mp * F * 2);
  // The attention partials (decode and prefill key splits) and the GEMMs'
  // split-K partials share one region: the QKV partials are consumed by the
  // RoPE step before attention writes its partials, and the merge has read
  // those before the O projection writes its own.
  L.dec = o;
  o = align256(o + (n_dec > 0
                        ? decode_workspace_bytes(n_dec, c->n_q_heads, c->n_kv_heads, d, max_ctx)
                        : 0));
  L.pre = o;
  o = align256(o + prefill_workspace_bound(rows, c->n_q_heads, c->n_kv_heads, (int)d));
  L.gemm = L.dec;
  const int nqd = c->n_q_heads * c->head_dim;
  const size_t g = std::max({gemm_workspace_bytes(EPI_STORE, L.Mp, (int)nqkv, (int)H),
                             gemm_workspace_bytes(EPI_RESIDUAL, L.Mp, (int)H, nqd),
                             gemm_workspace_bytes(EPI_RESIDUAL, L.Mp, (int)H, (int)F),
                             gemm_workspace_bytes(EPI_SWIGLU, L.Mp, (int)F, (int)H)});
  L.total = std::max(o, L.gemm + align256(g));
  return L;
}

// Bytes a call with `rows` rows needs.  The split-K partials of the GEMMs are
// not monotone in the row count (a second row tile halves the splits), so
// their share is the largest over every padded row count up to this one;
// every other part grows with rows, decodes and max_ctx.  A workspace sized
// for max_rows therefore serves every call with fewer rows.
size_t workspace_need(const hl_config* c, int rows, int n_dec, int max_ctx, int pad) {
  const Layout L = make_layout(c, rows, n_dec, max_ctx, pad);
  const int H = c->hidden, F = c->ffn, nqd = c->n_q_heads * c->head_dim;
  const int nqkv = (c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
  size_t g = 0;
  for (int mp = pad; mp <= L.Mp; mp += pad)
    g = std::max({g, gemm_workspace_bytes(EPI_STORE, mp, nqkv, H),
                  gemm_workspace_bytes(EPI_RESIDUAL, mp, H, nqd),
                  gemm_workspace_bytes(EPI_RESIDUAL, mp, H, F),
                  gemm_workspace_bytes(EPI_SWIGLU, mp, F, H)});
  return std::max(L.total, L.gemm + align256(g));
}

// Device address of `scratch` on the device that runs `stream`, looked up
// once per device (with that device current) and kept.  Threads that race on
// the first call store the same address.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HL_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return HL_ERR_HIP;
    if (sdev != dev) return HL_ERR_UNSUPPORTED;  // the lookup below is per current device
  }
  if (dev < 0 || dev >= kMaxDevices) return HL_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HL_ERR_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return HL_OK;
}

int fill_chunks(const hl_chunk* chunks, int n_chunks, ChunkList* cl) {
  if (n_chunks < 0) return HL_ERR_SHAPE;
  if (n_chunks > HL_MAX_CHUNKS) return HL_ERR_UNSUPPORTED;
  if (n_chunks > 0 && !chunks) return HL_ERR_NULL;
  memset(cl, 0, sizeof(*cl));
  cl->n = n_chunks;
  int row = 0;
  for (int i = 0; i < n_chunks; ++i) {
    const hl_chunk& c = chunks[i];
    if (c.len < 0 || c.start_pos < 0 || c.n_blocks < 0) return HL_ERR_SHAPE;
    if (c.len > 0 && !c.block_table) return HL_ERR_NULL;
    cl->c[i] = ChunkDev{c.len, c.start_pos, row, c.n_blocks, c.block_table};
    row += c.len;
  }
  cl->n_rows = row;
  return HL_OK;
}

int fill_decodes(const hl_decodes* d, DecDev* dd) {
  memset(dd, 0, sizeof(*dd));
  if (!d || d->n == 0) return HL_OK;
  if (d->n < 0 || d->max_blocks <= 0 || d->max_ctx < 0) return HL_ERR_SHAPE;
  if (!d->ctx_lens || !d->block_tables) return HL_ERR_NULL;
  *dd = DecDev{d->n, d->ctx_lens, d->block_tables, d->max_blocks, d->max_ctx};
  return HL_OK;
}

KvDev make_kv(const hl_config* c, const hl_kv* kv) {
  return KvDev{kv->data, kv->num_pages, c->n_kv_heads, c->head_dim, c->page_size};
}

}  // namespace

extern "C" {

const char* hl_error_string(int code) {
  switch (code) {
    case HL_OK: return "ok";
    case HL_ERR_NULL: return "required pointer is NULL";
    case HL_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case HL_ERR_UNSUPPORTED: return "unsupported configuration (head_dim, page_size, group or chunk count)";
    case HL_ERR_WORKSPACE: return "workspace too small";
    case HL_ERR_LAUNCH: return "kernel launch failed";
    case HL_ERR_METADATA: return "invalid metadata (page id, block table or context length)";
    case HL_ERR_HIP: return "HIP runtime call failed";
  }
  return "unknown error";
}

int hl_workspace_bytes(const hl_config* cfg, int32_t max_rows, int32_t max_decodes,
                       int32_t max_ctx, int32_t pad, size_t* bytes) {
  int e = check_config(cfg);
  if (e) return e;
  if (!bytes) return HL_ERR_NULL;
  if (max_rows < 0 || max_decodes < 0 || max_ctx < 0 || pad <= 0 || pad % 16) return HL_ERR_SHAPE;
  *bytes = workspace_need(cfg, max_rows, max_decodes, max_ctx, pad);
  return HL_OK;
}

int hl_decode_workspace_bytes(const hl_config* cfg, int32_t n_decodes, int32_t max_ctx,
                              size_t* bytes) {
  int e = check_config(cfg);
  if (e) return e;
  if (!bytes) return HL_ERR_NULL;
  if (n_decodes < 0 || max_ctx < 0) return HL_ERR_SHAPE;
  *bytes = decode_workspace_bytes(n_decodes, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim,
                                  max_ctx);
  return HL_OK;
}

static const char* const kStageNames[HL_N_STAGES] = {
    "rmsnorm1",     "gemm_qkv",  "rope_kv_append",   "attention",
    "attention_merge", "gemm_o", "gemm_o_reduce_rmsnorm2", "gemm_gate_up",
    "gemm_gate_up_reduce", "gemm_down", "gemm_down_reduce"};

const char* hl_stage_name(int stage) {
  return (stage >= 0 && stage < HL_N_STAGES) ? kStageNames[stage] : "";
}

static int layer_forward_impl(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                              const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                              const hl_kv* kv, hl_bf16* out, void* ws, size_t ws_bytes,
                              int32_t pad, const hl_taps* taps, const hl_chain* chain,
                              hipStream_t stream, hipEvent_t* ev) {
  int e = check_config(cfg);
  if (e) return e;
  if (!w || !x || !kv || !out || !ws || !kv->data) return HL_ERR_NULL;
  if (!w->w_qkv || !w->w_o || !w->w_gate || !w->w_up || !w->w_down || !w->g_attn || !w->g_ffn)
    return HL_ERR_NULL;
  if (pad <= 0 || pad % 16 || kv->num_pages <= 0) return HL_ERR_SHAPE;
  if ((const void*)x == (const void*)out) return HL_ERR_SHAPE;
  const hl_chain no_chain{};
  const hl_chain& chn = chain ? *chain : no_chain;
  if (chn.g_next && !chn.xn_next) return HL_ERR_NULL;
  if (chn.g_next && ((const void*)chn.xn_next == (const void*)x ||
                     (const void*)chn.xn_next == (const void*)out ||
                     (const void*)chn.xn_next == (const void*)chn.xn_in))
    return HL_ERR_SHAPE;
  ChunkList cl;
  if ((e = fill_chunks(chunks, n_chunks, &cl))) return e;
  DecDev dd;
  if ((e = fill_decodes(dec, &dd))) return e;
  const int M = cl.n_rows + dd.n;
  if (M == 0) return HL_ERR_SHAPE;
  const Layout L = make_layout(cfg, M, dd.n, dd.max_ctx, pad);
  if (ws_bytes < workspace_need(cfg, M, dd.n, dd.max_ctx, pad)) return HL_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return HL_ERR_WORKSPACE;

  char* base = static_cast<char*>(ws);
  auto pick = [&](hl_bf16* tap, size_t off) {
    return tap ? reinterpret_cast<bf16*>(tap) : reinterpret_cast<bf16*>(base + off);
  };
  const hl_taps none{};
  const hl_taps& t = taps ? *taps : none;
  bf16* xn1 = pick(t.xn1, L.xn1);
  bf16* qkv = pick(t.qkv, L.qkv);
  bf16* attn = pick(t.attn, L.attn);
  bf16* h = pick(t.h, L.h);
  bf16* xn2 = pick(t.xn2, L.xn2);
  bf16* act = pick(t.act, L.act);

  const int H = cfg->hidden, F = cfg->ffn, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  const int d = cfg->head_dim, Mp = L.Mp;
  const int nqkv = (nq + 2 * nkv) * d;
  const KvDev kvd = make_kv(cfg, kv);
  const bf16* xin = reinterpret_cast<const bf16*>(x);

  hipError_t r;
#define HL_TRY(call)                      \
  do {                                    \
    if ((r = (call)) != hipSuccess) return HL_ERR_LAUNCH; \
  } while (0)
  int stage = 0;
  auto mark = [&]() {
    if (ev && hipEventRecord(ev[stage], stream) != hipSuccess) return false;
    ++stage;
    return true;
  };
  // event between the two kernels of a two-kernel step (its slot boundary)
  auto mid = [&]() -> hipEvent_t {
    hipEvent_t m = ev ? ev[stage] : nullptr;
    ++stage;
    return m;
  };
#define HL_MARK() \
  do {            \
    if (!mark()) return HL_ERR_HIP; \
  } while (0)
  HL_MARK();
  // RMSNorm of the input rows (pad rows -> 0), unless the previous layer's
  // down-projection reduce already left it in chain->xn_in
  if (chn.xn_in)
    xn1 = const_cast<bf16*>(reinterpret_cast<const bf16*>(chn.xn_in));
  else
    HL_TRY(launch_rmsnorm(xin, reinterpret_cast<const bf16*>(w->g_attn), xn1, M, Mp, H,
                          cfg->rms_eps, stream));
  HL_MARK();
  // fused QKV projection on the stacked rows; with split K its partials are
  // summed by the RoPE / append kernel that follows
  void* gws = base + L.gemm;
  const int qkv_splits = gemm_splits(EPI_STORE, Mp, nqkv, H);
  if (qkv_splits > 1)
    HL_TRY(launch_gemm_partials(xn1, reinterpret_cast<const bf16*>(w->w_qkv), gws, M, Mp, nqkv, H,
                                stream));
  else
    HL_TRY(launch_gemm(EPI_STORE, xn1, reinterpret_cast<const bf16*>(w->w_qkv), nullptr, qkv,
                       nullptr, gws, M, Mp, nqkv, H, stream));
  HL_MARK();
  // each row's position and KV slot, RoPE on q and k, append K and V
  HL_TRY(launch_rope_append_wide(qkv, qkv_splits > 1 ? reinterpret_cast<const float*>(gws) : nullptr,
                                 qkv_splits, M, Mp, nq, nkv, d, cfg->rope_theta, cl, dd, kvd,
                                 stream));
  HL_MARK();
  // chunk-prefill attention (rows [0, Lp)) and paged decode attention
  // (rows [Lp, M)) in one launch
  HL_TRY(launch_attention(qkv, nq, nkv, d, cl, dd, cl.n_rows, kvd, attn, base + L.pre,
                          base + L.dec, stream, mid()));
  HL_MARK();
  // O projection + residual, then RMSNorm (fused into the split-K reduce)
  HL_TRY(launch_gemm_residual_norm(attn, reinterpret_cast<const bf16*>(w->w_o), h, xin,
                                   reinterpret_cast<const bf16*>(w->g_ffn), xn2, cfg->rms_eps, gws,
                                   M, Mp, H, nq * d, stream, mid()));
  HL_MARK();
  // gate/up projection + SwiGLU
  HL_TRY(launch_gemm(EPI_SWIGLU, xn2, reinterpret_cast<const bf16*>(w->w_gate),
                     reinterpret_cast<const bf16*>(w->w_up), act, nullptr, gws, M, Mp, F, H,
                     stream, mid()));
  HL_MARK();
  // down projection + residual; with chain->g_next the split-K reduce also
  // forms the next RMSNorm of the output rows (the next layer's input norm)
  if (chn.g_next)
    HL_TRY(launch_gemm_residual_norm(act, reinterpret_cast<const bf16*>(w->w_down),
                                     reinterpret_cast<bf16*>(out), h,
                                     reinterpret_cast<const bf16*>(chn.g_next),
                                     reinterpret_cast<bf16*>(chn.xn_next), cfg->rms_eps, gws, M,
                                     Mp, H, F, stream, mid()));
  else
    HL_TRY(launch_gemm(EPI_RESIDUAL, act, reinterpret_cast<const bf16*>(w->w_down), nullptr,
                       reinterpret_cast<bf16*>(out), h, gws, M, Mp, H, F, stream, mid()));
  HL_MARK();
#undef HL_MARK
#undef HL_TRY
  return HL_OK;
}

int hl_layer_forward(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                     const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                     const hl_kv* kv, hl_bf16* out, void* ws, size_t ws_bytes, int32_t pad,
                     const hl_taps* taps, hipStream_t stream) {
  return layer_forward_impl(cfg, w, x, chunks, n_chunks, dec, kv, out, ws, ws_bytes, pad, taps,
                            nullptr, stream, nullptr);
}

int hl_layer_forward_chain(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                           const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                           const hl_kv* kv, hl_bf16* out, void* ws, size_t ws_bytes, int32_t pad,
                           const hl_taps* taps, const hl_chain* chain, hipEvent_t* stage_events,
                           hipStream_t stream) {
  if (stage_events)
    for (int i = 0; i <= HL_N_STAGES; ++i)
      if (!stage_events[i]) return HL_ERR_NULL;
  return layer_forward_impl(cfg, w, x, chunks, n_chunks, dec, kv, out, ws, ws_bytes, pad, taps,
                            chain, stream, stage_events);
}

int hl_layer_forward_timed(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                           const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                           const hl_kv* kv, hl_bf16* out, void* ws, size_t ws_bytes, int32_t pad,
                           const hl_taps* taps, hipEvent_t* stage_events, hipStream_t stream) {
  if (!stage_events) return HL_ERR_NULL;
  for (int i = 0; i <= HL_N_STAGES; ++i)
    if (!stage_events[i]) return HL_ERR_NULL;
  return layer_forward_impl(cfg, w, x, chunks, n_chunks, dec, kv, out, ws, ws_bytes, pad, taps,
                            nullptr, stream, stage_events);
}

int hl_layer_forward_noalloc(const hl_config* cfg, const hl_weights* w, const hl_bf16* x,
                             const hl_chunk* chunks, int32_t n_chunks, const hl_decodes* dec,
                             const hl_kv* kv, hl_bf16* out, int32_t pad, const hl_taps* taps,
                             hipStream_t stream) {
  // the size check comes first, so an oversized call fails before any
  // runtime call (same checks and order as hl_layer_forward otherwise)
  int e = check_config(cfg);
  if (e) return e;
  if (pad <= 0 || pad % 16) return HL_ERR_SHAPE;
  ChunkList cl;
  if ((e = fill_chunks(chunks, n_chunks, &cl))) return e;
  DecDev dd;
  if ((e = fill_decodes(dec, &dd))) return e;
  const int M = cl.n_rows + dd.n;
  if (M == 0) return HL_ERR_SHAPE;
  if (workspace_need(cfg, M, dd.n, dd.max_ctx, pad) > (size_t)HL_NOALLOC_SCRATCH_BYTES)
    return HL_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((e = scratch_address(stream, &ws))) return e;
  return layer_forward_impl(cfg, w, x, chunks, n_chunks, dec, kv, out, ws,
                            (size_t)HL_NOALLOC_SCRATCH_BYTES, pad, taps, nullptr, stream, nullptr);
}

int hl_slot_mapping(const hl_config* cfg, const hl_chunk* chunks, int32_t n_chunks,
                    const hl_decodes* dec, int32_t num_pages, int32_t* positions, int32_t* slots,
                    hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  if (!positions || !slots) return HL_ERR_NULL;
  ChunkList cl;
  if ((e = fill_chunks(chunks, n_chunks, &cl))) return e;
  DecDev dd;
  if ((e = fill_decodes(dec, &dd))) return e;
  if (launch_slot_map(cl, dd, cfg->page_size, num_pages, positions, slots, stream) != hipSuccess)
    return HL_ERR_LAUNCH;
  return HL_OK;
}

int hl_validate_metadata(const hl_config* cfg, const hl_chunk* chunks, int32_t n_chunks,
                         const hl_decodes* dec, int32_t num_pages, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  ChunkList cl;
  if ((e = fill_chunks(chunks, n_chunks, &cl))) return e;
  DecDev dd;
  if ((e = fill_decodes(dec, &dd))) return e;
  if (hipStreamSynchronize(stream) != hipSuccess) return HL_ERR_HIP;
  const int P = cfg->page_size;
  std::vector<int> owner(std::max(num_pages, 0), -1);
  auto claim = [&](int page, int req) {
    if (page < 0 || page >= num_pages) return false;
    if (owner[page] != -1 && owner[page] != req) return false;
    owner[page] = req;
    return true;
  };
  int req = 0;
  for (int i = 0; i < cl.n; ++i, ++req) {
    const ChunkDev& c = cl.c[i];
    const int need = (c.start_pos + c.len + P - 1) / P;
    if (need > c.n_blocks) return HL_ERR_METADATA;
    if (need == 0) continue;
    std::vector<int32_t> bt(need);
    if (hipMemcpy(bt.data(), c.block_table, need * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return HL_ERR_HIP;
    for (int b = 0; b < need; ++b)
      if (!claim(bt[b], req)) return HL_ERR_METADATA;
  }
  if (dd.n > 0) {
    std::vector<int32_t> ctx(dd.n), bts((size_t)dd.n * dd.max_blocks);
    if (hipMemcpy(ctx.data(), dd.ctx_lens, dd.n * 4, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(bts.data(), dd.block_tables, bts.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return HL_ERR_HIP;
    for (int j = 0; j < dd.n; ++j, ++req) {
      if (ctx[j] < 0 || ctx[j] > dd.max_ctx) return HL_ERR_METADATA;
      const int need = ctx[j] / P + 1;
      if (need > dd.max_blocks) return HL_ERR_METADATA;
      for (int b = 0; b < need; ++b)
        if (!claim(bts[(size_t)j * dd.max_blocks + b], req)) return HL_ERR_METADATA;
    }
  }
  return HL_OK;
}

int hl_rmsnorm(const hl_bf16* x, const hl_bf16* g, hl_bf16* y, int32_t rows, int32_t rows_padded,
               int32_t hidden, float eps, hipStream_t stream) {
  if (!x || !g || !y) return HL_ERR_NULL;
  if (rows < 0 || rows_padded < rows || hidden <= 0 || hidden % 8) return HL_ERR_SHAPE;
  return launch_rmsnorm(reinterpret_cast<const bf16*>(x), reinterpret_cast<const bf16*>(g),
                        reinterpret_cast<bf16*>(y), rows, rows_padded, hidden, eps, stream) ==
                 hipSuccess
             ? HL_OK
             : HL_ERR_LAUNCH;
}

int hl_gemm_workspace_bytes(int32_t m_padded, int32_t n, int32_t k, size_t* bytes) {
  if (!bytes) return HL_ERR_NULL;
  if (m_padded < 0 || m_padded % 16 || n <= 0 || n % 64 || k <= 0 || k % 64) return HL_ERR_SHAPE;
  *bytes = std::max(gemm_workspace_bytes(EPI_STORE, m_padded, n, k),
                    gemm_workspace_bytes(EPI_RESIDUAL, m_padded, n, k));
  return HL_OK;
}

int hl_gemm_bf16(const hl_bf16* a, const hl_bf16* w, hl_bf16* c, const hl_bf16* residual,
                 int32_t m, int32_t m_padded, int32_t n, int32_t k, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  if (!a || !w || !c) return HL_ERR_NULL;
  if (m < 0 || m_padded < m || m_padded % 16 || n <= 0 || n % 64 || k <= 0 || k % 64)
    return HL_ERR_SHAPE;
  if (!gemm_fits_offsets(m_padded, n, k)) return HL_ERR_UNSUPPORTED;
  const GemmEpilogue epi = residual ? EPI_RESIDUAL : EPI_STORE;
  const size_t need = gemm_workspace_bytes(epi, m_padded, n, k);
  if (ws && ws_bytes < need) return HL_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 15) return HL_ERR_WORKSPACE;
  return launch_gemm(epi, reinterpret_cast<const bf16*>(a), reinterpret_cast<const bf16*>(w),
                     nullptr, reinterpret_cast<bf16*>(c), reinterpret_cast<const bf16*>(residual),
                     need ? ws : nullptr, m, m_padded, n, k, stream) == hipSuccess
             ? HL_OK
             : HL_ERR_LAUNCH;
}

int hl_gemm_swiglu(const hl_bf16* a, const hl_bf16* w_gate, const hl_bf16* w_up, hl_bf16* act,
                   int32_t m_padded, int32_t f, int32_t k, hipStream_t stream) {
  if (!a || !w_gate || !w_up || !act) return HL_ERR_NULL;
  if (m_padded < 0 || m_padded % 16 || f <= 0 || f % 64 || k <= 0 || k % 64) return HL_ERR_SHAPE;
  if (!gemm_fits_offsets(m_padded, f, k)) return HL_ERR_UNSUPPORTED;
  return launch_gemm(EPI_SWIGLU, reinterpret_cast<const bf16*>(a),
                     reinterpret_cast<const bf16*>(w_gate), reinterpret_cast<const bf16*>(w_up),
                     reinterpret_cast<bf16*>(act), nullptr, nullptr, m_padded, m_padded, f, k,
                     stream) ==
                 hipSuccess
             ? HL_OK
             : HL_ERR_LAUNCH;
}

int hl_rope_kv_append(const hl_config* cfg, hl_bf16* qkv, const int32_t* positions,
                      const int32_t* slots, int32_t rows, const hl_kv* kv, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  if (!qkv || !positions || !slots || !kv || !kv->data) return HL_ERR_NULL;
  if (rows < 0) return HL_ERR_SHAPE;
  return launch_rope_kv_append(reinterpret_cast<bf16*>(qkv), positions, slots, rows,
                               cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->rope_theta,
                               make_kv(cfg, kv), stream) == hipSuccess
             ? HL_OK
             : HL_ERR_LAUNCH;
}

int hl_prefill_workspace_bytes(const hl_config* cfg, const hl_chunk* chunks, int32_t n_chunks,
                               size_t* bytes) {
  int e = check_config(cfg);
  if (e) return e;
  if (!bytes) return HL_ERR_NULL;
  ChunkList cl;
  if ((e = fill_chunks(chunks, n_chunks, &cl))) return e;
  *bytes = prefill_workspace_bytes(cl, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim);
  return HL_OK;
}

int hl_prefill_attention(const hl_config* cfg, const hl_bf16* qkv, const hl_chunk* chunks,
                         int32_t n_chunks, const hl_kv* kv, hl_bf16* attn, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  if (!qkv || !kv || !kv->data || !attn) return HL_ERR_NULL;
  ChunkList cl;
  if ((e = fill_chunks(chunks, n_chunks, &cl))) return e;
  const size_t need = prefill_workspace_bytes(cl, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim);
  if (ws && ws_bytes < need) return HL_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 15) return HL_ERR_WORKSPACE;
  return launch_prefill_attention(reinterpret_cast<const bf16*>(qkv), cfg->n_q_heads,
                                  cfg->n_kv_heads, cfg->head_dim, cl, make_kv(cfg, kv),
                                  reinterpret_cast<bf16*>(attn), need ? ws : nullptr,
                                  stream) == hipSuccess
             ? HL_OK
             : HL_ERR_LAUNCH;
}

int hl_decode_attention(const hl_config* cfg, const hl_bf16* qkv, int32_t row0,
                        const hl_decodes* dec, const hl_kv* kv, hl_bf16* attn, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  if (!qkv || !kv || !kv->data || !attn) return HL_ERR_NULL;
  DecDev dd;
  if ((e = fill_decodes(dec, &dd))) return e;
  if (row0 < 0) return HL_ERR_SHAPE;
  if (dd.n == 0) return HL_OK;
  if (!ws) return HL_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) & 15) return HL_ERR_WORKSPACE;  // f32x4 partial stores
  if (ws_bytes <
      decode_workspace_bytes(dd.n, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, dd.max_ctx))
    return HL_ERR_WORKSPACE;
  return launch_decode_attention(reinterpret_cast<const bf16*>(qkv), row0, cfg->n_q_heads,
                                 cfg->n_kv_heads, cfg->head_dim, dd, make_kv(cfg, kv),
                                 reinterpret_cast<bf16*>(attn), ws, stream) == hipSuccess
             ? HL_OK
             : HL_ERR_LAUNCH;
}

}  // extern "C"

"""Thin ctypes binding of ``libhybrid_layer.so`` (C ABI in include/hybrid_layer.h).

Argument marshalling only: torch tensors supply device memory and the
stream, every step of the layer runs in the library's HIP kernels.  The
library must have been built (``python -m chunked_prefill_hybrid_rmsnorm_amd.build``);
loading fails loudly otherwise -- there is no fallback.

Also here: conversion of the KV pages between the logical layout
``[num_pages, 2, n_kv, page_size, head_dim]`` and the library's page layout,
in which V is stored dimension-major (``[n_kv, head_dim, page_size]``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhybrid_layer.so")
_lib = None

HL_OK = 0
HL_ERR_WORKSPACE = -4
HL_MAX_CHUNKS = 16
HL_NOALLOC_SCRATCH_BYTES = 160 << 20


class HLError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {error_string(code)} ({code})")
        self.code = code


class hl_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class hl_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")]


class hl_chunk(ctypes.Structure):
    _fields_ = [("len", ctypes.c_int32), ("start_pos", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("n_blocks", ctypes.c_int32)]


class hl_decodes(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("ctx_lens", ctypes.c_void_p),
                ("block_tables", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32)]


class hl_kv(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("num_pages", ctypes.c_int32)]


class hl_taps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("xn1", "qkv", "attn", "h", "xn2", "act")]


class hl_chain(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("xn_in", "g_next", "xn_next")]


_P = ctypes.POINTER
_c = ctypes
_SIGS = {
    "hl_error_string": (_c.c_char_p, [_c.c_int]),
    "hl_workspace_bytes": (_c.c_int, [_P(hl_config), _c.c_int32, _c.c_int32, _c.c_int32,
                                      _c.c_int32, _P(_c.c_size_t)]),
    "hl_decode_workspace_bytes": (_c.c_int, [_P(hl_config), _c.c_int32, _c.c_int32,
                                             _P(_c.c_size_t)]),
    "hl_layer_forward": (_c.c_int, [_P(hl_config), _P(hl_weights), _c.c_void_p, _P(hl_chunk),
                                    _c.c_int32, _P(hl_decodes), _P(hl_kv), _c.c_void_p,
                                    _c.c_void_p, _c.c_size_t, _c.c_int32, _P(hl_taps),
                                    _c.c_void_p]),
    "hl_layer_forward_timed": (_c.c_int, [_P(hl_config), _P(hl_weights), _c.c_void_p,
                                          _P(hl_chunk), _c.c_int32, _P(hl_decodes), _P(hl_kv),
                                          _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_int32,
                                          _P(hl_taps), _P(_c.c_void_p), _c.c_void_p]),
    "hl_layer_forward_chain": (_c.c_int, [_P(hl_config), _P(hl_weights), _c.c_void_p,
                                          _P(hl_chunk), _c.c_int32, _P(hl_decodes), _P(hl_kv),
                                          _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_int32,
                                          _P(hl_taps), _P(hl_chain), _P(_c.c_void_p),
                                          _c.c_void_p]),
    "hl_layer_forward_noalloc": (_c.c_int, [_P(hl_config), _P(hl_weights), _c.c_void_p,
                                            _P(hl_chunk), _c.c_int32, _P(hl_decodes), _P(hl_kv),
                                            _c.c_void_p, _c.c_int32, _P(hl_taps), _c.c_void_p]),
    "hl_stage_name": (_c.c_char_p, [_c.c_int]),
    "hl_slot_mapping": (_c.c_int, [_P(hl_config), _P(hl_chunk), _c.c_int32, _P(hl_decodes),
                                   _c.c_int32, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "hl_validate_metadata": (_c.c_int, [_P(hl_config), _P(hl_chunk), _c.c_int32,
                                        _P(hl_decodes), _c.c_int32, _c.c_void_p]),
    "hl_rmsnorm": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int32, _c.c_int32,
                              _c.c_int32, _c.c_float, _c.c_void_p]),
    "hl_gemm_bf16": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int32,
                                _c.c_int32, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_size_t,
                                _c.c_void_p]),
    "hl_gemm_workspace_bytes": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _P(_c.c_size_t)]),
    "hl_gemm_swiglu": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                  _c.c_int32, _c.c_int32, _c.c_int32, _c.c_void_p]),
    "hl_embed_rows": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_void_p,
                                 _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_void_p]),
    "hl_argmax_rows": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_void_p,
                                  _c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_int32, _c.c_void_p]),
    "hl_read_stream": (_c.c_int, [_c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_void_p]),
    "hl_rope_kv_append": (_c.c_int, [_P(hl_config), _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                     _c.c_int32, _P(hl_kv), _c.c_void_p]),
    "hl_prefill_attention": (_c.c_int, [_P(hl_config), _c.c_void_p, _P(hl_chunk), _c.c_int32,
                                        _P(hl_kv), _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                        _c.c_void_p]),
    "hl_prefill_workspace_bytes": (_c.c_int, [_P(hl_config), _P(hl_chunk), _c.c_int32,
                                              _P(_c.c_size_t)]),
    "hl_decode_attention": (_c.c_int, [_P(hl_config), _c.c_void_p, _c.c_int32, _P(hl_decodes),
                                       _P(hl_kv), _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                       _c.c_void_p]),
}
EXPORTED = tuple(_SIGS)


def lib_path() -> str:
    return _LIB_PATH


def load(path: Optional[str] = None):
    """Load the library (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} is missing "
                           "(run python -m chunked_prefill_hybrid_rmsnorm_amd.build)")
    try:  # share torch's HIP runtime (streams and events cross the ABI)
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def error_string(code: int) -> str:
    return load().hl_error_string(code).decode()


def _check(rc: int, where: str):
    if rc != HL_OK:
        raise HLError(rc, where)


# ----------------------------------------------------------------- helpers
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_config(shape) -> hl_config:
    return hl_config(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                     shape.page_size, shape.rms_eps, shape.rope_theta)


def kv_to_library_layout(kv: np.ndarray) -> np.ndarray:
    """[num_pages, 2, n_kv, P, d] -> library pages (V transposed per page)."""
    pages = kv.shape[0]
    k = kv[:, 0]                                   # [pages, nkv, P, d]
    v = np.ascontiguousarray(kv[:, 1].transpose(0, 1, 3, 2))  # [pages, nkv, d, P]
    return np.concatenate([k.reshape(pages, -1), v.reshape(pages, -1)], axis=1).reshape(kv.shape)


def kv_from_library_layout(buf: np.ndarray, n_kv: int, page_size: int, head_dim: int) -> np.ndarray:
    pages = buf.shape[0]
    flat = buf.reshape(pages, 2, n_kv * page_size * head_dim)
    k = flat[:, 0].reshape(pages, n_kv, page_size, head_dim)
    v = flat[:, 1].reshape(pages, n_kv, head_dim, page_size).transpose(0, 1, 3, 2)
    return np.stack([k, v], axis=1)


def bits_to_device(a: np.ndarray, device="cuda"):
    """Upload bf16 bit patterns (uint16) as a torch.bfloat16 device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def device_to_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def int32_to_device(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


# ----------------------------------------------------------------- raw entry points
def hl_workspace_bytes(cfg: hl_config, max_rows: int, max_decodes: int, max_ctx: int,
                       pad: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().hl_workspace_bytes(ctypes.byref(cfg), max_rows, max_decodes, max_ctx, pad,
                                     ctypes.byref(out)), "hl_workspace_bytes")
    return out.value


def hl_decode_workspace_bytes(cfg: hl_config, n_decodes: int, max_ctx: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().hl_decode_workspace_bytes(ctypes.byref(cfg), n_decodes, max_ctx,
                                            ctypes.byref(out)), "hl_decode_workspace_bytes")
    return out.value


def _chunk_array(chunks: Sequence[hl_chunk]):
    arr = (hl_chunk * max(1, len(chunks)))(*chunks)
    return arr, len(chunks)


def hl_layer_forward(cfg, weights: hl_weights, x, chunks: Sequence[hl_chunk], dec: hl_decodes,
                     kv: hl_kv, out, ws, ws_bytes: int, pad: int,
                     taps: Optional[hl_taps] = None, stream=None):
    arr, n = _chunk_array(chunks)
    rc = load().hl_layer_forward(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), arr, n,
                                 ctypes.byref(dec), ctypes.byref(kv), _ptr(out), _ptr(ws),
                                 ws_bytes, pad, ctypes.byref(taps) if taps is not None else None,
                                 _stream(stream))
    _check(rc, "hl_layer_forward")


def hl_layer_forward_noalloc(cfg, weights: hl_weights, x, chunks: Sequence[hl_chunk],
                             dec: hl_decodes, kv: hl_kv, out, pad: int,
                             taps: Optional[hl_taps] = None, stream=None) -> int:
    """The layer call on the library's own device workspace; returns the HL
    code (0, or HL_ERR_WORKSPACE when the batch needs more than the fixed
    workspace) and raises on any other error."""
    arr, n = _chunk_array(chunks)
    rc = load().hl_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), arr,
                                         n, ctypes.byref(dec), ctypes.byref(kv), _ptr(out), pad,
                                         ctypes.byref(taps) if taps is not None else None,
                                         _stream(stream))
    if rc not in (HL_OK, HL_ERR_WORKSPACE):
        _check(rc, "hl_layer_forward_noalloc")
    return rc


N_STAGES = 11


def stage_names():
    return [load().hl_stage_name(i).decode() for i in range(N_STAGES)]


def hl_layer_forward_timed(cfg, weights: hl_weights, x, chunks, dec: hl_decodes, kv: hl_kv, out,
                           ws, ws_bytes: int, pad: int, events, taps=None, stream=None):
    """``events``: N_STAGES + 1 torch.cuda.Event objects (timing enabled)."""
    arr, n = _chunk_array(chunks)
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    rc = load().hl_layer_forward_timed(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), arr, n,
                                       ctypes.byref(dec), ctypes.byref(kv), _ptr(out), _ptr(ws),
                                       ws_bytes, pad,
                                       ctypes.byref(taps) if taps is not None else None, handles,
                                       _stream(stream))
    _check(rc, "hl_layer_forward_timed")


def hl_layer_forward_chain(cfg, weights: hl_weights, x, chunks, dec: hl_decodes, kv: hl_kv, out,
                           ws, ws_bytes: int, pad: int, xn_in=None, g_next=None, xn_next=None,
                           events=None, taps=None, stream=None):
    """The layer call with the cross-layer RMSNorm fusion: ``xn_in`` (this
    layer's normalised input, from the previous call's ``xn_next``) replaces
    the layer's own first RMSNorm; with ``g_next`` the down projection's
    reduce also writes RMSNorm(out) * g_next into ``xn_next``.  ``events``:
    None or N_STAGES + 1 torch.cuda.Event objects."""
    arr, n = _chunk_array(chunks)
    chain = hl_chain(_ptr(xn_in), _ptr(g_next), _ptr(xn_next))
    handles = None
    if events is not None:
        handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    rc = load().hl_layer_forward_chain(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), arr, n,
                                       ctypes.byref(dec), ctypes.byref(kv), _ptr(out), _ptr(ws),
                                       ws_bytes, pad,
                                       ctypes.byref(taps) if taps is not None else None,
                                       ctypes.byref(chain), handles, _stream(stream))
    _check(rc, "hl_layer_forward_chain")


def hl_slot_mapping(cfg, chunks, dec, num_pages, positions, slots, stream=None):
    arr, n = _chunk_array(chunks)
    _check(load().hl_slot_mapping(ctypes.byref(cfg), arr, n, ctypes.byref(dec), num_pages,
                                  _ptr(positions), _ptr(slots), _stream(stream)),
           "hl_slot_mapping")


def hl_validate_metadata(cfg, chunks, dec, num_pages, stream=None) -> int:
    arr, n = _chunk_array(chunks)
    return load().hl_validate_metadata(ctypes.byref(cfg), arr, n, ctypes.byref(dec), num_pages,
                                       _stream(stream))


def hl_rmsnorm(x, g, y, rows, rows_padded, hidden, eps, stream=None):
    _check(load().hl_rmsnorm(_ptr(x), _ptr(g), _ptr(y), rows, rows_padded, hidden, eps,
                             _stream(stream)), "hl_rmsnorm")


def hl_gemm_workspace_bytes(m_padded, n, k) -> int:
    out = ctypes.c_size_t(0)
    _check(load().hl_gemm_workspace_bytes(m_padded, n, k, ctypes.byref(out)),
           "hl_gemm_workspace_bytes")
    return out.value


def hl_gemm_bf16(a, w, c, residual, m, m_padded, n, k, ws=None, ws_bytes=0, stream=None):
    _check(load().hl_gemm_bf16(_ptr(a), _ptr(w), _ptr(c), _ptr(residual), m, m_padded, n, k,
                               _ptr(ws), ws_bytes, _stream(stream)), "hl_gemm_bf16")


def hl_gemm_swiglu(a, w_gate, w_up, act, m_padded, f, k, stream=None):
    _check(load().hl_gemm_swiglu(_ptr(a), _ptr(w_gate), _ptr(w_up), _ptr(act), m_padded, f, k,
                                 _stream(stream)), "hl_gemm_swiglu")


def hl_embed_rows(table, vocab, hidden, row_tok, last_tok, rows, out, stream=None):
    n_last = 0 if last_tok is None else last_tok.numel()
    _check(load().hl_embed_rows(_ptr(table), vocab, hidden, _ptr(row_tok), _ptr(last_tok), n_last,
                                rows, _ptr(out), _stream(stream)), "hl_embed_rows")


def hl_argmax_rows(logits, rows, vocab, sample_req, sample_pos, last_tok, out_tokens,
                   stream=None):
    _check(load().hl_argmax_rows(_ptr(logits), rows, vocab, _ptr(sample_req), _ptr(sample_pos),
                                 _ptr(last_tok), last_tok.numel(), _ptr(out_tokens),
                                 out_tokens.numel(), _stream(stream)), "hl_argmax_rows")


def hl_read_stream(buf, nbytes, sink, stream=None):
    _check(load().hl_read_stream(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "hl_read_stream")


def hl_rope_kv_append(cfg, qkv, positions, slots, rows, kv: hl_kv, stream=None):
    _check(load().hl_rope_kv_append(ctypes.byref(cfg), _ptr(qkv), _ptr(positions), _ptr(slots),
                                    rows, ctypes.byref(kv), _stream(stream)), "hl_rope_kv_append")


def hl_prefill_workspace_bytes(cfg, chunks) -> int:
    arr, n = _chunk_array(chunks)
    out = ctypes.c_size_t(0)
    _check(load().hl_prefill_workspace_bytes(ctypes.byref(cfg), arr, n, ctypes.byref(out)),
           "hl_prefill_workspace_bytes")
    return out.value


def hl_prefill_attention(cfg, qkv, chunks, kv: hl_kv, attn, ws=None, ws_bytes=0, stream=None):
    arr, n = _chunk_array(chunks)
    _check(load().hl_prefill_attention(ctypes.byref(cfg), _ptr(qkv), arr, n, ctypes.byref(kv),
                                       _ptr(attn), _ptr(ws), ws_bytes, _stream(stream)),
           "hl_prefill_attention")


def hl_decode_attention(cfg, qkv, row0, dec: hl_decodes, kv: hl_kv, attn, ws, ws_bytes,
                        stream=None):
    _check(load().hl_decode_attention(ctypes.byref(cfg), _ptr(qkv), row0, ctypes.byref(dec),
                                      ctypes.byref(kv), _ptr(attn), _ptr(ws), ws_bytes,
                                      _stream(stream)), "hl_decode_attention")


# ----------------------------------------------------------------- device-side batch
class DeviceBatch:
    """A generated hybrid batch uploaded to the GPU, with the structs that
    describe it to the library.  Keeps every tensor alive while the structs
    point at them."""

    def __init__(self, hb, device="cuda", pad: int = 16, weights=None):
        import torch
        self.hb = hb
        self.shape = hb.shape
        self.cfg = make_config(hb.shape)
        self.pad = pad
        if weights is None:
            weights = upload_weights(hb.weights, device)
        self.wt, self.weights = weights
        self.x = bits_to_device(hb.x, device)
        self.M = hb.x.shape[0]
        self.out = torch.empty_like(self.x)
        self.kv_t = bits_to_device(kv_to_library_layout(hb.kv_pages), device)
        self.kv = hl_kv(self.kv_t.data_ptr(), hb.kv_pages.shape[0])
        self.bt_t = [int32_to_device(c.block_table, device) for c in hb.chunks]
        self.chunks = [hl_chunk(c.length, c.start_pos, t.data_ptr(), len(c.block_table))
                       for c, t in zip(hb.chunks, self.bt_t)]
        d = hb.decodes
        if d.n:
            self.ctx_t = int32_to_device(d.ctx_lens, device)
            self.dbt_t = int32_to_device(d.block_tables, device)
            self.dec = hl_decodes(d.n, self.ctx_t.data_ptr(), self.dbt_t.data_ptr(), d.max_blocks,
                                  d.max_ctx)
        else:
            self.dec = hl_decodes(0, None, None, 0, 0)
        self.ws_bytes = hl_workspace_bytes(self.cfg, self.M, d.n, d.max_ctx if d.n else 0, pad)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    @property
    def Mp(self) -> int:
        return -(-self.M // self.pad) * self.pad

    def make_taps(self):
        import torch
        s, Mp = self.shape, self.Mp
        dev = self.x.device
        e = lambda n: torch.zeros((Mp, n), dtype=torch.bfloat16, device=dev)
        self.tap_t = {"xn1": e(s.hidden), "qkv": e(s.qkv_rows), "attn": e(s.n_q_heads * s.head_dim),
                      "h": e(s.hidden), "xn2": e(s.hidden), "act": e(s.ffn)}
        return hl_taps(*(self.tap_t[k].data_ptr() for k in ("xn1", "qkv", "attn", "h", "xn2", "act")))

    def forward(self, taps: Optional[hl_taps] = None, stream=None):
        hl_layer_forward(self.cfg, self.weights, self.x, self.chunks, self.dec, self.kv, self.out,
                         self.ws, self.ws_bytes, self.pad, taps, stream)

    def kv_logical(self) -> np.ndarray:
        s = self.shape
        return kv_from_library_layout(device_to_bits(self.kv_t), s.n_kv_heads, s.page_size,
                                      s.head_dim)


def upload_weights(w, device="cuda"):
    t = {k: bits_to_device(v, device) for k, v in w.as_dict().items()}
    return t, hl_weights(*(t[k].data_ptr() for k in
                           ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")))

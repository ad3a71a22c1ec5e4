"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/hybrid_layer.h declares, and rejects bad arguments before touching
the device."""
import ctypes
import os
import re

import pytest

from chunked_prefill_hybrid_rmsnorm_amd import binding as B
from chunked_prefill_hybrid_rmsnorm_amd.inputs import MISTRAL_7B, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hybrid_layer.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hl_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        from chunked_prefill_hybrid_rmsnorm_amd.build import build
        build()
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert set(names) == set(B.EXPORTED)


def test_stage_slots_match_header(lib):
    """The binding's slot count is the header's, every slot has a distinct
    name, and the slots out of range have none."""
    n = int(re.search(r"#define\s+HL_N_STAGES\s+(\d+)", open(HEADER).read()).group(1))
    assert n == B.N_STAGES
    names = B.stage_names()
    assert len(names) == n and len(set(names)) == n and all(names)
    assert lib.hl_stage_name(n) == b"" and lib.hl_stage_name(-1) == b""


def test_error_strings(lib):
    for code in range(0, -8, -1):
        assert B.error_string(code) not in ("", "unknown error")
    assert B.error_string(-99) == "unknown error"


def test_workspace_bytes_host_only(lib):
    cfg = B.make_config(MISTRAL_7B)
    ws = B.hl_workspace_bytes(cfg, 288, 32, 2048, 16)
    # activations alone: xn1, xn2, h [Mp,H], qkv, attn, act, all bf16
    acts = 288 * 2 * (3 * 4096 + 6144 + 4096 + 14336)
    assert ws >= acts
    # decode partials share the region of the GEMM split-K partials
    assert ws >= B.hl_workspace_bytes(cfg, 288, 0, 0, 16)
    assert B.hl_workspace_bytes(cfg, 257, 0, 0, 256) > B.hl_workspace_bytes(cfg, 257, 0, 0, 16)


def _cfg(**kw):
    c = B.make_config(TINY)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -3), (dict(page_size=32), -3), (dict(n_kv_heads=3), -2),
    (dict(hidden=100), -2), (dict(ffn=1000), -2), (dict(n_q_heads=32, n_kv_heads=1), -3),
    # a weight matrix of 4 GiB or more (the GEMM copies use 32-bit byte offsets)
    (dict(hidden=65536, ffn=32768), -3),
])
def test_config_errors(lib, kw, code):
    out = ctypes.c_size_t(0)
    assert lib.hl_workspace_bytes(ctypes.byref(_cfg(**kw)), 10, 1, 10, 16, ctypes.byref(out)) == code


def test_bad_pad_and_null(lib):
    out = ctypes.c_size_t(0)
    cfg = _cfg()
    assert lib.hl_workspace_bytes(ctypes.byref(cfg), 10, 1, 10, 24, ctypes.byref(out)) == -2
    assert lib.hl_workspace_bytes(None, 10, 1, 10, 16, ctypes.byref(out)) == -1
    assert lib.hl_workspace_bytes(ctypes.byref(cfg), 10, 1, 10, 16, None) == -1


def test_layer_forward_rejects_before_launch(lib):
    """Every failing check returns before a kernel is enqueued (fake,
    never-dereferenced pointers are safe here)."""
    cfg = _cfg()
    fake = 0x1000
    w = B.hl_weights(*([fake] * 7))
    kv = B.hl_kv(fake, 10)
    ch = (B.hl_chunk * 1)(B.hl_chunk(4, 0, fake, 1))
    dec = B.hl_decodes(0, None, None, 0, 0)
    f = lib.hl_layer_forward
    # workspace too small
    assert f(ctypes.byref(cfg), ctypes.byref(w), fake, ch, 1, ctypes.byref(dec), ctypes.byref(kv),
             fake + 4096, fake, 16, 16, None, None) == -4
    # x aliases out
    assert f(ctypes.byref(cfg), ctypes.byref(w), fake, ch, 1, ctypes.byref(dec), ctypes.byref(kv),
             fake, fake, 1 << 30, 16, None, None) == -2
    # no rows
    empty = (B.hl_chunk * 1)(B.hl_chunk(0, 0, fake, 1))
    assert f(ctypes.byref(cfg), ctypes.byref(w), fake, empty, 1, ctypes.byref(dec),
             ctypes.byref(kv), fake + 4096, fake, 1 << 30, 16, None, None) == -2
    # too many chunks
    many = (B.hl_chunk * 17)(*([B.hl_chunk(1, 0, fake, 1)] * 17))
    assert f(ctypes.byref(cfg), ctypes.byref(w), fake, many, 17, ctypes.byref(dec),
             ctypes.byref(kv), fake + 4096, fake, 1 << 30, 16, None, None) == -3
    # null weight pointer
    w0 = B.hl_weights(*([fake] * 6 + [0]))
    assert f(ctypes.byref(cfg), ctypes.byref(w0), fake, ch, 1, ctypes.byref(dec),
             ctypes.byref(kv), fake + 4096, fake, 1 << 30, 16, None, None) == -1
    # decode block table missing
    bad_dec = B.hl_decodes(2, fake, None, 4, 30)
    assert f(ctypes.byref(cfg), ctypes.byref(w), fake, ch, 1, ctypes.byref(bad_dec),
             ctypes.byref(kv), fake + 4096, fake, 1 << 30, 16, None, None) == -1


def test_layer_forward_chain_rejects_before_launch(lib):
    """The stack-call fields are checked on the host before any launch (fake,
    never-dereferenced pointers)."""
    cfg = _cfg()
    fake = 0x1000
    w = B.hl_weights(*([fake] * 7))
    kv = B.hl_kv(fake, 10)
    ch = (B.hl_chunk * 1)(B.hl_chunk(4, 0, fake, 1))
    dec = B.hl_decodes(0, None, None, 0, 0)
    f = lib.hl_layer_forward_chain
    x, out, ws = fake, fake + 4096, fake + 8192

    def call(chain, events=None):
        return f(ctypes.byref(cfg), ctypes.byref(w), x, ch, 1, ctypes.byref(dec), ctypes.byref(kv),
                 out, ws, 1 << 30, 16, None, ctypes.byref(chain) if chain else None, events, None)

    # g_next without xn_next
    assert call(B.hl_chain(None, fake + 12288, None)) == -1
    # xn_next aliasing out, x or xn_in
    assert call(B.hl_chain(None, fake + 12288, out)) == -2
    assert call(B.hl_chain(None, fake + 12288, x)) == -2
    assert call(B.hl_chain(fake + 16384, fake + 12288, fake + 16384)) == -2
    # a stage-event array with a missing event
    events = (ctypes.c_void_p * (B.N_STAGES + 1))()
    assert call(B.hl_chain(None, None, None), events) == -1
    # hidden beyond what the row-wise RMSNorm kernels hold
    big = B.hl_config(16384 + 64, 8, 8, 128, 1024, 16, 1e-5, 1e4)
    assert f(ctypes.byref(big), ctypes.byref(w), x, ch, 1, ctypes.byref(dec), ctypes.byref(kv),
             out, ws, 1 << 30, 16, None, None, None, None) == -3


def test_gemm_entries_reject_before_launch(lib):
    """Shape errors and operands of 4 GiB or more come back before any launch
    (fake device pointers, no GPU needed)."""
    fake = ctypes.c_void_p(0x1000)
    g = lib.hl_gemm_bf16
    assert g(fake, fake, fake, None, 16, 16, 100, 64, None, 0, None) == -2   # n % 64
    assert g(fake, fake, fake, None, 16, 16, 65536, 65536, None, 0, None) == -3  # w: 8 GiB
    assert g(fake, fake, fake, None, 65536, 65536, 64, 65536, None, 0, None) == -3  # a: 8 GiB
    s = lib.hl_gemm_swiglu
    assert s(fake, fake, fake, fake, 16, 65536, 65536, None) == -3
    assert s(None, fake, fake, fake, 16, 64, 64, None) == -1


@pytest.mark.parametrize("mp,n,k,splits", [(64, 6144, 4096, 5), (64, 10240, 8192, 3),
                                             (32, 4608, 4096, 7), (128, 4096, 4096, 8),
                                             (288, 6144, 4096, 4)])
def test_gemm_split_counts(lib, mp, n, k, splits):
    """The GEMM workspace is the fp32 partials of the chosen split count:
    small batches take the most splits (up to 8, any count) that keep one
    round of 256 workgroups and >= 8 k-steps each for the plain epilogue
    (48, 80 and 36 column tiles of 128: 5, 3 and 7 splits; 32 tiles: 8);
    288-row tiles keep powers of two."""
    assert B.hl_gemm_workspace_bytes(mp, n, k) == splits * mp * n * 4


def test_read_stream_rejects_before_launch(lib):
    """The streaming-read measurement entry checks its arguments before any
    launch (fake device pointers, no GPU needed)."""
    fake = ctypes.c_void_p(0x1000)
    f = lib.hl_read_stream
    assert f(None, 256 << 20, fake, None) == -1
    assert f(fake, 256 << 20, None, None) == -1
    assert f(fake, 0, fake, None) == -2
    assert f(fake, (256 << 20) + 16, fake, None) == -2   # not a multiple of 256 MiB
    assert f(ctypes.c_void_p(0x1008), 256 << 20, fake, None) == -2   # not 16-byte aligned


def test_kv_layout_roundtrip():
    import numpy as np
    rng = np.random.default_rng(0)
    kv = rng.integers(0, 65535, size=(3, 2, 2, 16, 64), dtype=np.uint16)
    lib_layout = B.kv_to_library_layout(kv)
    back = B.kv_from_library_layout(lib_layout, 2, 16, 64)
    np.testing.assert_array_equal(back, kv)
    # V of page 1, kv head 1, token 5, dim 7 sits at dim-major offset 7*16+5
    flat = lib_layout.reshape(3, -1)
    v_base = 2 * 16 * 64 + 1 * 64 * 16
    assert flat[1, v_base + 7 * 16 + 5] == kv[1, 1, 1, 5, 7]


def test_cost_model_slots_are_library_slots(lib):
    from chunked_prefill_hybrid_rmsnorm_amd import profiling
    from chunked_prefill_hybrid_rmsnorm_amd import roofline as rl
    s = rl.layer_stages(4096, 32, 8, 128, 14336, [256], [768], [1000] * 32)
    assert [x.name for x in s] == B.stage_names() == list(profiling.SLOTS)


@pytest.mark.parametrize("shape_name", ["TINY", "MISTRAL_7B", "LLAMA2_70B", "LLAMA2_70B_TP8",
                                        "MISTRAL_7B_TP4"])
@pytest.mark.parametrize("pad", [16, 128])
def test_workspace_bytes_is_nondecreasing(lib, shape_name, pad):
    """A workspace sized for max_rows serves every call with fewer rows: the
    size never drops as rows, decodes or contexts grow (the GEMMs' split-K
    partials alone would drop where a second row tile halves the splits, e.g.
    288 -> 304 rows of the Mistral-shaped down projection)."""
    from chunked_prefill_hybrid_rmsnorm_amd import inputs as I
    cfg = B.make_config(getattr(I, shape_name))
    prev = 0
    for rows in range(1, 1200, 3 if pad == 16 else 7):
        ws = B.hl_workspace_bytes(cfg, rows, 0, 0, pad)
        assert ws >= prev, (rows, ws, prev)
        prev = ws
    top = B.hl_workspace_bytes(cfg, 1200, 64, 4096, pad)
    for rows, dec, ctx in [(273, 0, 0), (288, 32, 2048), (576, 64, 4096), (1, 1, 1), (1200, 64, 4096)]:
        assert B.hl_workspace_bytes(cfg, rows, dec, ctx, pad) <= top
    for dec in range(0, 65, 8):
        assert B.hl_workspace_bytes(cfg, 600, dec, 4096, pad) <= B.hl_workspace_bytes(cfg, 600, dec + 1, 4096, pad)
    for ctx in range(0, 5000, 250):
        assert B.hl_workspace_bytes(cfg, 600, 64, ctx, pad) <= B.hl_workspace_bytes(cfg, 600, 64, ctx + 1, pad)


def test_noalloc_limit_matches_header(lib):
    """The fixed device workspace of hl_layer_forward_noalloc: the header's
    size is the binding's, and the Mistral- and Llama-2-70B-shaped batches fit
    it while a far larger batch does not (checked on the host sizes only)."""
    from chunked_prefill_hybrid_rmsnorm_amd import inputs as I
    text = open(HEADER).read()
    m = re.search(r"#define\s+HL_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.HL_NOALLOC_SCRATCH_BYTES
    lim = B.HL_NOALLOC_SCRATCH_BYTES
    assert B.hl_workspace_bytes(B.make_config(I.MISTRAL_7B), 288, 32, 2048, 16) <= lim
    assert B.hl_workspace_bytes(B.make_config(I.LLAMA2_70B), 576, 64, 4096, 16) <= lim
    assert B.hl_workspace_bytes(B.make_config(I.LLAMA2_70B), 4096, 64, 4096, 16) > lim


def test_noalloc_rejects_oversized_batch_before_any_runtime_call(lib):
    """An oversized batch comes back HL_ERR_WORKSPACE from the host checks
    alone (fake pointers, no GPU touched)."""
    from chunked_prefill_hybrid_rmsnorm_amd import inputs as I
    cfg = B.make_config(I.LLAMA2_70B)
    fake = 0x1000
    w = B.hl_weights(*([fake] * 7))
    kv = B.hl_kv(fake, 10)
    ch = (B.hl_chunk * 1)(B.hl_chunk(4096, 0, fake, 256))
    dec = B.hl_decodes(0, None, None, 0, 0)
    assert lib.hl_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), fake, ch, 1,
                                        ctypes.byref(dec), ctypes.byref(kv), fake + 4096, 16,
                                        None, None) == -4

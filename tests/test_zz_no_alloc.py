"""hl_layer_forward_noalloc, the layer call on the library's own fixed device
workspace (for callers that cannot allocate), against hl_layer_forward with a
caller workspace on the same inputs: two calls in a row, the second with a
smaller batch (the array keeps the first call's contents), each bit for bit
equal in output rows and KV pages, and the second also against the oracle."""
import numpy as np
import pytest

from chunked_prefill_hybrid_rmsnorm_amd import binding as B
from chunked_prefill_hybrid_rmsnorm_amd.inputs import mistral_batch, tiny_batch
from tests.gpu_helpers import check_layer, require_gpu, run_oracle, tap_f64

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16)


def _both(hb):
    """(out, pages) of hl_layer_forward and of hl_layer_forward_noalloc, each
    from the same starting pages."""
    import torch
    db = B.DeviceBatch(hb)
    assert db.ws_bytes <= B.HL_NOALLOC_SCRATCH_BYTES
    kv0 = db.kv_t.clone()
    db.forward()
    torch.cuda.synchronize()
    ref_out, ref_kv = db.out.clone(), db.kv_t.clone()
    db.kv_t.copy_(kv0)
    db.out.fill_(0)
    torch.cuda.synchronize()
    rc = B.hl_layer_forward_noalloc(db.cfg, db.weights, db.x, db.chunks, db.dec, db.kv, db.out,
                                    db.pad)
    assert rc == B.HL_OK
    torch.cuda.synchronize()
    return db, ref_out, ref_kv


def test_noalloc_matches_workspace_call_twice_then_smaller():
    require_gpu()
    print("no-alloc: mistral-shaped batch (M=288), then the tiny batch (M=68)", flush=True)
    for hb, oracle in ((mistral_batch(seed=5), False), (tiny_batch(seed=6), True)):
        db, ref_out, ref_kv = _both(hb)
        assert _bits(db.out).equal(_bits(ref_out)), "output differs from hl_layer_forward"
        assert _bits(db.kv_t).equal(_bits(ref_kv)), "pages differ from hl_layer_forward"
        if oracle:
            check_layer(hb, {"out": tap_f64(db.out, db.M), "kv": db.kv_logical()},
                        run_oracle(hb), taps=False)


def test_noalloc_rejects_a_batch_beyond_its_workspace():
    """A batch whose workspace exceeds the fixed array returns HL_ERR_WORKSPACE
    and writes nothing."""
    import torch
    require_gpu()
    hb = mistral_batch(seed=7, prior_kv="none")
    db = B.DeviceBatch(hb)
    big_pad = 4096  # pads the GEMM rows to 4096: far more workspace than the array holds
    need = B.hl_workspace_bytes(db.cfg, db.M, hb.decodes.n, hb.decodes.max_ctx, big_pad)
    assert need > B.HL_NOALLOC_SCRATCH_BYTES
    db.out.fill_(0)
    kv0 = db.kv_t.clone()
    torch.cuda.synchronize()
    rc = B.hl_layer_forward_noalloc(db.cfg, db.weights, db.x, db.chunks, db.dec, db.kv, db.out,
                                    big_pad)
    torch.cuda.synchronize()
    assert rc == B.HL_ERR_WORKSPACE
    assert int(np.count_nonzero(B.device_to_bits(db.out))) == 0
    assert _bits(db.kv_t).equal(_bits(kv0))

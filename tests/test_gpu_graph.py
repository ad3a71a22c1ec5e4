"""The layer call recorded into a HIP graph and replayed (GPU).

The library issues only kernel launches on the caller's stream (no memsets,
no allocations, no host synchronisation), so one layer call can be captured
and replayed.  Every replay, with ordinary eager work between replays, must
match the eager call bit for bit (output rows and KV pages) and the oracle
within the parity tolerance."""
import pytest

from chunked_prefill_hybrid_rmsnorm_amd import binding as B
from chunked_prefill_hybrid_rmsnorm_amd.inputs import mistral_batch
from tests.gpu_helpers import check_layer, require_gpu, run_oracle, tap_f64

pytestmark = pytest.mark.gpu


def test_layer_graph_replays_match_eager():
    import torch
    require_gpu()
    print("mistral-shaped hybrid batch, seed 1: eager call, capture, 4 replays", flush=True)
    hb = mistral_batch(seed=1)
    ref = run_oracle(hb)
    db = B.DeviceBatch(hb)
    kv0 = db.kv_t.clone()
    db.forward()  # eager (also settles every one-time host-side query before capture)
    torch.cuda.synchronize()
    out_ref, kv_ref = db.out.clone(), db.kv_t.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        db.forward()  # launches on the capture stream (the current stream here)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        db.out.zero_()
        db.kv_t.copy_(kv0)  # the call appends the batch's K/V; start from the same pages
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # bit patterns: slots that hold no token carry NaN fill, which never equals itself
        bits = lambda t: t.view(torch.int16)
        assert torch.equal(bits(db.out), bits(out_ref)), f"replay {rep}: output differs from the eager call"
        assert torch.equal(bits(db.kv_t), bits(kv_ref)), f"replay {rep}: pages differ from the eager call"
        print(f"replay {rep} against the oracle", flush=True)
        check_layer(hb, {"out": tap_f64(db.out, db.M), "kv": db.kv_logical()}, ref, taps=False)


def test_chained_call_graph_replays_match_eager():
    """The call as it runs inside a layer stack (previous layer's normalised
    input in, next layer's out), captured and replayed: output, pages and the
    next layer's normalised input bit-identical to the eager call."""
    import torch
    require_gpu()
    print("llama70-shaped hybrid batch, chained call: eager, capture, 3 replays", flush=True)
    from chunked_prefill_hybrid_rmsnorm_amd.inputs import llama70_batch
    hb = llama70_batch(seed=2)
    db = B.DeviceBatch(hb)
    H = hb.shape.hidden
    xn_in = torch.empty((db.Mp, H), dtype=torch.bfloat16, device="cuda")
    B.hl_rmsnorm(db.x, db.wt["g_attn"], xn_in, db.M, db.Mp, H, hb.shape.rms_eps)
    xn_next = torch.empty_like(xn_in)
    kv0 = db.kv_t.clone()

    def call():
        B.hl_layer_forward_chain(db.cfg, db.weights, db.x, db.chunks, db.dec, db.kv, db.out, db.ws,
                                 db.ws_bytes, db.pad, xn_in=xn_in, g_next=db.wt["g_ffn"],
                                 xn_next=xn_next)

    call()
    torch.cuda.synchronize()
    out_ref, kv_ref, xn_ref = db.out.clone(), db.kv_t.clone(), xn_next.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)
    for rep in range(3):
        db.out.zero_()
        xn_next.zero_()
        db.kv_t.copy_(kv0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(db.out), bits(out_ref)), f"replay {rep}: output differs"
        assert torch.equal(bits(db.kv_t), bits(kv_ref)), f"replay {rep}: pages differ"
        assert torch.equal(bits(xn_next), bits(xn_ref)), f"replay {rep}: next-layer norm differs"

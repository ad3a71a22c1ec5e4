"""Token-budget sweep of the layer on the Mistral-7B shape.

The pages choose the chunk size (the token budget) by profiling the layer
once: up to a point, adding prefill tokens to a decode batch costs little
because the linear layers stream their weights whether they multiply few rows
or many; past it the time grows with the rows.  This script measures that
curve for the library on the GPU it runs on:

1. the Lp x Bd grid: a chunk of Lp tokens from position 0 plus Bd decodes
   with contexts U{128..4096}, Lp in {128, 192, 256, 257, 384, 512}, Bd in
   {0, 16, 64, 128};
2. the 256-vs-257 step at padding granularity 16, 128 and 256 (Bd = 0);
3. a 2048-token prompt prefilled in N in {1, 2, 4, 8, 16} equal chunks over N
   calls: the sum over the N calls, the attention share of it, and the bytes
   the chunks re-read from earlier chunks' pages, C N (N - 1) / 2 kvB;
4. a scan of Lp = 16 ... 1024 in steps of 16 (Bd = 0).  The time climbs in
   steps, where the GEMMs need one more row tile; the last Lp before each
   step (a plateau end) is where a token budget gets the most rows for the
   time, so those are the candidates for the budget;
5. the Bd decodes alone (Lp = 0), so that the grid's piggybacked decodes can
   be set against a separate decode call: what adding Bd decodes to a chunk
   costs (hybrid minus chunk alone) against what they cost on their own.
   The pages' case for piggybacking is that the first is much smaller,
   because the decode rows ride on the chunk's weight stream.

Inputs are seeded and synthetic (weights N(0, 0.02), activations and cached
K/V N(0, 1)); one page pool holds every request, so each point only changes
the metadata handed to the library.  Two weight copies alternate between
calls so the weights stream from HBM each call.

    python -m chunked_prefill_hybrid_rmsnorm_amd.sweep --md profiles/token_budget_mistral7b.md
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import Dict, List

import numpy as np

from . import binding as B
from .inputs import MISTRAL_7B, _fill_cached, _normal_bf16, draw_weights, pages_for

LPS = (128, 192, 256, 257, 384, 512)
BDS = (0, 16, 64, 128)
PADS = (16, 128, 256)
NS = (1, 2, 4, 8, 16)
PROMPT = 2048
SCAN = tuple(range(16, 1025, 16))
CTX_RANGE = (128, 4096)
LP_MAX = 1024


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Pool:
    """Every request of the sweep in one page pool on the device."""

    def __init__(self, seed: int = 0):
        import torch
        s = MISTRAL_7B
        P = s.page_size
        rng = np.random.default_rng(seed)
        self.shape = s
        self.cfg = B.make_config(s)
        w = draw_weights(rng, s, 0.02, False)
        self.weights = [B.upload_weights(w), B.upload_weights(w)]
        bd_max = max(BDS)
        self.ctx = rng.integers(CTX_RANGE[0], CTX_RANGE[1], size=bd_max, endpoint=True).astype(np.int32)
        need_dec = [pages_for(int(c) + 1, P) for c in self.ctx]
        n_chunk, n_prompt = pages_for(LP_MAX, P), pages_for(PROMPT, P)
        num_pages = n_chunk + n_prompt + sum(need_dec)
        perm = rng.permutation(num_pages).astype(np.int32)
        self.chunk_bt = perm[:n_chunk].copy()
        self.prompt_bt = perm[n_chunk:n_chunk + n_prompt].copy()
        cur = n_chunk + n_prompt
        self.max_blocks = max(need_dec)
        bts = np.zeros((bd_max, self.max_blocks), dtype=np.int32)
        for j, nb in enumerate(need_dec):
            bts[j, :nb] = perm[cur:cur + nb]
            cur += nb
        log(f"pool: {num_pages} pages, {bd_max} decodes with {int(self.ctx.sum())} cached tokens")
        kv = np.zeros((num_pages, 2, s.n_kv_heads, P, s.head_dim), dtype=np.uint16)
        for j in range(bd_max):
            _fill_cached(rng, kv, bts[j], int(self.ctx[j]), P)
        self.kv_t = B.bits_to_device(B.kv_to_library_layout(kv))
        del kv
        self.kv = B.hl_kv(self.kv_t.data_ptr(), num_pages)
        self.chunk_bt_t = B.int32_to_device(self.chunk_bt)
        self.prompt_bt_t = B.int32_to_device(self.prompt_bt)
        self.ctx_t = B.int32_to_device(self.ctx)
        self.bt_t = B.int32_to_device(bts)
        rows = LP_MAX + bd_max
        self.x = B.bits_to_device(_normal_bf16(rng, (max(rows, PROMPT), s.hidden), 1.0))
        self.out = torch.empty_like(self.x)
        self.ws_bytes = B.hl_workspace_bytes(self.cfg, max(rows, PROMPT), bd_max, int(self.ctx.max()),
                                             max(PADS))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")

    def decodes(self, bd: int) -> B.hl_decodes:
        if bd == 0:
            return B.hl_decodes(0, None, None, 0, 0)
        return B.hl_decodes(bd, self.ctx_t.data_ptr(), self.bt_t.data_ptr(), self.max_blocks,
                            int(self.ctx[:bd].max()))

    def chunk(self, lp: int) -> List[B.hl_chunk]:
        if lp == 0:
            return []
        return [B.hl_chunk(lp, 0, self.chunk_bt_t.data_ptr(), len(self.chunk_bt))]

    def prompt_chunk(self, c: int, k: int) -> List[B.hl_chunk]:
        return [B.hl_chunk(c, k * c, self.prompt_bt_t.data_ptr(), len(self.prompt_bt))]

    def call(self, i: int, chunks, dec, x, out, pad: int, events=None) -> None:
        wt = self.weights[i % 2][1]
        if events is None:
            B.hl_layer_forward(self.cfg, wt, x, chunks, dec, self.kv, out, self.ws, self.ws_bytes,
                               pad)
        else:
            B.hl_layer_forward_timed(self.cfg, wt, x, chunks, dec, self.kv, out, self.ws,
                                     self.ws_bytes, pad, events)


def timed(fn, n: int, warm: int) -> float:
    """Average ms per fn(i) call, HIP events on the current stream."""
    import torch
    for i in range(warm):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def point(pool: Pool, lp: int, bd: int, pad: int, n: int, warm: int) -> float:
    chunks, dec = pool.chunk(lp), pool.decodes(bd)
    M = lp + bd
    x, out = pool.x[:M], pool.out[:M]
    return timed(lambda i: pool.call(i, chunks, dec, x, out, pad), n, warm)


def n_chunk_prefill(pool: Pool, nc: int, reps: int) -> Dict[str, float]:
    """One prompt prefilled in nc calls: ms for the whole sequence, and the
    attention + merge share from the library's per-step events."""
    import torch
    c = PROMPT // nc
    calls = [(pool.prompt_chunk(c, k), pool.x[k * c:(k + 1) * c], pool.out[k * c:(k + 1) * c])
             for k in range(nc)]
    none = pool.decodes(0)

    def seq(i):
        for k, (ch, x, out) in enumerate(calls):
            pool.call(i * nc + k, ch, none, x, out, 16)

    ms = timed(seq, reps, 2)
    names = B.stage_names()
    a0, a1 = names.index("attention"), names.index("attention_merge")
    att = 0.0
    for r in range(reps):
        for k, (ch, x, out) in enumerate(calls):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
            for e in ev:  # the HIP event exists once recorded
                e.record()
            pool.call(r * nc + k, ch, none, x, out, 16, events=ev)
            torch.cuda.synchronize()
            att += ev[a0].elapsed_time(ev[a1 + 1])
    return {"ms": ms, "attention_ms": att / reps}


def n_chunk_counter_pass(args) -> None:
    """The N-chunk prefill alone, for a rocprofv3 --pmc FETCH_SIZE pass.  A
    256 MiB device copy comes first (the byte counters' scale); then, for
    each N, one marker kernel (a one-element fill) and `seq_reps` runs of
    the N calls, so the counter file splits into the N groups at the
    markers."""
    import torch
    torch.cuda.set_device(0)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    torch.empty_like(src).copy_(src)
    torch.cuda.synchronize()
    del src
    pool = Pool(args.seed)
    none = pool.decodes(0)
    marker = torch.empty(1, dtype=torch.float32, device="cuda")
    point(pool, 256, 0, 16, 5, 0)
    for nc in NS:
        marker.fill_(float(nc))
        c = PROMPT // nc
        for r in range(args.seq_reps):
            for k in range(nc):
                pool.call(r * nc + k, pool.prompt_chunk(c, k), none, pool.x[k * c:(k + 1) * c],
                          pool.out[k * c:(k + 1) * c], 16)
    torch.cuda.synchronize()
    log(f"N-chunk counter pass: N in {NS}, {args.seq_reps} runs each")


def run(args) -> dict:
    import torch
    torch.cuda.set_device(0)
    log("building the page pool ...")
    pool = Pool(args.seed)
    kvB = pool.shape.kv_bytes_per_token
    log("warming up ...")
    point(pool, 256, 32, 16, args.warm_calls, 0)
    res: dict = {"grid": {}, "pad_step": {}, "n_chunks": {}, "scan": {}, "decode_only": {}}
    for lp in LPS:
        for bd in BDS:
            ms = point(pool, lp, bd, 16, args.steps, args.warmup)
            res["grid"][f"{lp},{bd}"] = ms
            log(f"  Lp={lp:4d} Bd={bd:4d}: {ms * 1e3:7.1f} us")
    for bd in BDS[1:]:
        ms = point(pool, 0, bd, 16, args.steps, args.warmup)
        res["decode_only"][str(bd)] = ms
        log(f"  Lp=   0 Bd={bd:4d}: {ms * 1e3:7.1f} us")
    for lp in (256, 257):
        for pad in PADS:
            ms = point(pool, lp, 0, pad, args.steps, args.warmup)
            res["pad_step"][f"{lp},{pad}"] = ms
            log(f"  Lp={lp} pad={pad}: {ms * 1e3:7.1f} us")
    for nc in NS:
        r = n_chunk_prefill(pool, nc, args.seq_reps)
        c = PROMPT // nc
        r["reread_bytes"] = c * nc * (nc - 1) // 2 * kvB
        res["n_chunks"][str(nc)] = r
        log(f"  N={nc:2d}: {r['ms'] * 1e3:8.1f} us, attention {r['attention_ms'] * 1e3:7.1f} us, "
            f"re-read {r['reread_bytes'] / 1e6:6.1f} MB")
    for lp in SCAN:
        res["scan"][str(lp)] = point(pool, lp, 0, 16, args.steps, args.warmup)
    res["plateau_ends"] = plateau_ends(res["scan"])
    log(f"  plateau ends (last Lp before a step of > {STEP:.0%}): {res['plateau_ends']}")
    return res


STEP = 0.15  # a rise of more than this between neighbouring scan points is a step


def plateau_ends(scan: Dict[str, float]) -> List[int]:
    """Scan points followed by a step in the layer time, and the last point."""
    lps = sorted(int(k) for k in scan)
    ends = [a for a, b in zip(lps, lps[1:]) if scan[str(b)] > (1 + STEP) * scan[str(a)]]
    return ends + [lps[-1]]


def write_md(path: str, res: dict, command: str) -> None:
    us = lambda ms: f"{ms * 1e3:.1f}"
    L = ["# Token-budget sweep, Mistral-7B-shaped layer", "",
         "Command (run from the repository root):", "", f"    {command}", "",
         "One layer call per point: a chunk of Lp tokens from position 0 plus Bd decodes with "
         "contexts U{128..4096}; seeded synthetic inputs; two weight copies alternate.", "",
         "## Layer time (us) over the Lp x Bd grid (pad 16)", "",
         "| Lp \\ Bd | " + " | ".join(str(b) for b in BDS) + " |",
         "|---|" + "---:|" * len(BDS)]
    for lp in LPS:
        L.append(f"| {lp} | " + " | ".join(us(res["grid"][f"{lp},{bd}"]) for bd in BDS) + " |")
    L += ["", "Tokens/s per layer (M = Lp + Bd real rows):", "",
          "| Lp \\ Bd | " + " | ".join(str(b) for b in BDS) + " |",
          "|---|" + "---:|" * len(BDS)]
    for lp in LPS:
        L.append(f"| {lp} | " + " | ".join(
            f"{(lp + bd) / (res['grid'][f'{lp},{bd}'] * 1e-3) / 1e6:.2f} M" for bd in BDS) + " |")
    if res.get("decode_only"):
        L += ["", "## Piggybacked decodes against a separate decode call", "",
              "Cost of adding the Bd decodes to the chunk (hybrid call minus the chunk alone), "
              "against the Bd decodes in a call of their own (Lp = 0), us:", "",
              "| Lp \\ Bd | " + " | ".join(str(b) for b in BDS[1:]) + " |",
              "|---|" + "---:|" * len(BDS[1:]),
              "| alone (Lp = 0) | " + " | ".join(us(res["decode_only"][str(bd)])
                                                for bd in BDS[1:]) + " |"]
        for lp in LPS:
            base = res["grid"][f"{lp},0"]
            L.append(f"| {lp} | " + " | ".join(
                f"+{us(res['grid'][f'{lp},{bd}'] - base)} "
                f"({(res['grid'][f'{lp},{bd}'] - base) / res['decode_only'][str(bd)]:.2f})"
                for bd in BDS[1:]) + " |")
        L += ["", "In parentheses: the added cost as a fraction of the separate decode call."]
    L += ["", "## Tile step: 256 vs 257 rows (Bd = 0)", "",
          "| pad | Lp=256 us | Lp=257 us | step |", "|---:|---:|---:|---:|"]
    for pad in PADS:
        a, b = res["pad_step"][f"256,{pad}"], res["pad_step"][f"257,{pad}"]
        L.append(f"| {pad} | {us(a)} | {us(b)} | {100 * (b / a - 1):+.1f} % |")
    L += ["", f"## A {PROMPT}-token prompt prefilled in N chunks", "",
          "| N | chunk | all N calls, us | attention + merge, us | KV re-read from earlier chunks, closed form C N(N-1)/2 kvB |",
          "|---:|---:|---:|---:|---:|"]
    for nc in NS:
        r = res["n_chunks"][str(nc)]
        L.append(f"| {nc} | {PROMPT // nc} | {us(r['ms'])} | {us(r['attention_ms'])} | "
                 f"{r['reread_bytes'] / 1e6:.1f} MB |")
    L += ["", "## Scan of Lp (Bd = 0, pad 16)", "",
          f"Plateau ends (the last Lp before the layer time rises by more than {STEP:.0%} at the "
          f"next point, and the last point):", "",
          "| Lp | us | tokens/s |", "|---:|---:|---:|"]
    for lp in res["plateau_ends"]:
        t = res["scan"][str(lp)]
        L.append(f"| {lp} | {us(t)} | {lp / (t * 1e-3) / 1e6:.2f} M |")
    L += ["", "Every point:", "", "| Lp | us | tokens/s |", "|---:|---:|---:|"]
    for lp in SCAN:
        t = res["scan"][str(lp)]
        L.append(f"| {lp} | {us(t)} | {lp / (t * 1e-3) / 1e6:.2f} M |")
    with open(path, "w") as fh:
        fh.write("\n".join(L) + "\n")


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--warm-calls", type=int, default=200)
    p.add_argument("--seq-reps", type=int, default=5)
    p.add_argument("--md", help="write the tables as markdown here")
    p.add_argument("--json", help="write the raw numbers here")
    p.add_argument("--n-chunk-counters", action="store_true",
                   help="only run the N-chunk prefill, marked for a FETCH_SIZE counter pass")
    a = p.parse_args()
    if a.n_chunk_counters:
        n_chunk_counter_pass(a)
        return
    res = run(a)
    cmd = "python -m chunked_prefill_hybrid_rmsnorm_amd.sweep " + " ".join(sys.argv[1:])
    if a.md:
        write_md(a.md, res, cmd)
    if a.json:
        with open(a.json, "w") as fh:
            json.dump(res, fh, indent=1)
    print(json.dumps({"plateau_ends": res["plateau_ends"]}))


if __name__ == "__main__":
    main()

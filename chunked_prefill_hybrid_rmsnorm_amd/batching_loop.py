"""A model of L layers driven by stall-free batching (Sarathi-Serve digest,
Algorithm 3) through the library: one hybrid batch per iteration.

Every iteration: the scheduler forms the batch (decodes first, then prompt
chunks within the token budget); the library embeds the rows' input tokens
(prompt ids, or each decoding request's last generated token, kept on the
GPU), runs the L layer calls (each layer with its own page pool, all sharing
the block tables; each layer's input RMSNorm is formed by the previous
layer's last kernel, and the last layer's forms the final RMSNorm), the LM
head GEMM and the greedy choice of the rows that yield a token.  The host only counts tokens: the generated
ids stay on the GPU until the end (there is no end-of-sequence token), so the
host can queue iterations ahead of the GPU.

The measured workload: 32 Mistral-7B-shaped layers, random bf16 weights
(N(0, 0.02); unit gains), vocabulary 32000, 32 requests with prompt lengths
U{50..500} and prompt ids U{0..31999}, 100 generated tokens each, token budget
512.  It reports generated and total tokens/s and the per-iteration time
between tokens (p50 / p99).

    python -m chunked_prefill_hybrid_rmsnorm_amd.batching_loop
"""
from __future__ import annotations

import argparse
import json
import sys
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import binding as B
from .inputs import MISTRAL_7B, LayerShape, pages_for
from .scheduler import StallFreeScheduler


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Model:
    """Layer weights, embedding table, LM head and final gain on the GPU."""

    def __init__(self, shape: LayerShape, layers, table, lm, g_final):
        self.shape = shape
        self.cfg = B.make_config(shape)
        self.layers = layers            # [(tensors dict, hl_weights)]
        self.table, self.lm, self.g_final = table, lm, g_final
        self.vocab = table.shape[0]

    @classmethod
    def random(cls, shape: LayerShape, n_layers: int, vocab: int, seed: int = 0,
               std: float = 0.02) -> "Model":
        """Weights drawn on the GPU from a seeded generator."""
        import torch
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        H, F = shape.hidden, shape.ffn
        nqd = shape.n_q_heads * shape.head_dim

        def normal(*size):
            return (torch.randn(*size, generator=gen, device="cuda") * std).to(torch.bfloat16)

        ones = torch.ones(H, dtype=torch.bfloat16, device="cuda")
        layers = []
        for _ in range(n_layers):
            t = {"w_qkv": normal(shape.qkv_rows, H), "w_o": normal(H, nqd),
                 "w_gate": normal(F, H), "w_up": normal(F, H), "w_down": normal(H, F),
                 "g_attn": ones, "g_ffn": ones}
            layers.append((t, B.hl_weights(*(t[k].data_ptr() for k in
                                              ("w_qkv", "w_o", "w_gate", "w_up", "w_down",
                                               "g_attn", "g_ffn")))))
        return cls(shape, layers, normal(vocab, H), normal(vocab, H), ones)

    @classmethod
    def from_host(cls, shape: LayerShape, layer_weights, table_bits, lm_bits,
                  g_final_bits) -> "Model":
        """Weights given as bf16 bit arrays (``inputs.Weights`` per layer)."""
        layers = [B.upload_weights(w) for w in layer_weights]
        return cls(shape, layers, B.bits_to_device(table_bits), B.bits_to_device(lm_bits),
                   B.bits_to_device(g_final_bits))


@dataclass
class Record:
    """What one iteration ran and what it sampled (record mode)."""
    chunks: list
    decodes: list
    ctx_lens: list
    samples: list
    logits: np.ndarray  # float32 [len(samples), vocab], bf16 values


@dataclass
class RunStats:
    iterations: int
    seconds: float
    generated: int
    prompt_tokens: int
    tbt_ms: List[float]          # iterations that carried decodes
    iter_ms: List[float] = field(default_factory=list)


class BatchingLoop:
    def __init__(self, model: Model, prompts: List[np.ndarray], gen_len: int, budget: int,
                 pad: int = 16, seed: int = 0):
        import torch
        self.m = model
        s = model.shape
        self.prompts = [np.asarray(p, dtype=np.int32) for p in prompts]
        self.gen_len, self.budget, self.pad = gen_len, budget, pad
        n_req = len(prompts)
        P = s.page_size
        need = [pages_for(len(p) + gen_len, P) for p in self.prompts]
        self.max_blocks = max(need)
        perm = np.random.default_rng(seed).permutation(sum(need)).astype(np.int32)
        self.bt = np.full((n_req, self.max_blocks), -1, dtype=np.int32)
        cur = 0
        for i, nb in enumerate(need):
            self.bt[i, :nb] = perm[cur:cur + nb]
            cur += nb
        self.n_blocks = need
        self.bt_dev = [B.int32_to_device(self.bt[i]) for i in range(n_req)]
        self.num_pages = int(sum(need))
        page_elems = 2 * s.n_kv_heads * P * s.head_dim
        self.kv_t = [torch.zeros(self.num_pages * page_elems, dtype=torch.bfloat16, device="cuda")
                     for _ in model.layers]
        self.kv = [B.hl_kv(t.data_ptr(), self.num_pages) for t in self.kv_t]
        rows = max(budget, n_req)
        self.Mp_max = -(-rows // pad) * pad
        H, V = s.hidden, model.vocab
        self.x = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
        self.y = torch.empty_like(self.x)
        # normalised layer inputs, handed from one layer call to the next
        # (cross-layer RMSNorm fusion); the last holds the final norm
        self.xn = [torch.empty((self.Mp_max, H), dtype=torch.bfloat16, device="cuda")
                   for _ in range(2)]
        self.logits = torch.empty((self.Mp_max, V), dtype=torch.bfloat16, device="cuda")
        max_ctx = max(len(p) for p in self.prompts) + gen_len
        self.ws_bytes = B.hl_workspace_bytes(model.cfg, rows, n_req, max_ctx, pad)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        # the split count (and so the workspace) can differ with the padded rows
        self.gws_bytes = max(B.hl_gemm_workspace_bytes(mp, V, H)
                             for mp in range(pad, self.Mp_max + 1, pad))
        self.gws = torch.empty(max(self.gws_bytes, 256), dtype=torch.uint8, device="cuda")
        self.last_tok = torch.zeros(n_req, dtype=torch.int32, device="cuda")
        self.out_tokens = torch.full((n_req * gen_len,), -1, dtype=torch.int32, device="cuda")

    @staticmethod
    def _up(a: np.ndarray):
        import torch
        return torch.from_numpy(np.ascontiguousarray(a)).pin_memory().to("cuda", non_blocking=True)

    def run(self, record: bool = False, max_iterations: Optional[int] = None):
        """Run the loop to the end, or for at most ``max_iterations``
        iterations.  With ``record`` every iteration's batch and the logits of
        its sampled rows are kept (one synchronisation per iteration)."""
        import torch
        s, m = self.m.shape, self.m
        sched = StallFreeScheduler([len(p) for p in self.prompts], self.gen_len, self.budget,
                                   max_chunks=B.HL_MAX_CHUNKS)
        events, records = [], []
        while max_iterations is None or len(events) < max_iterations:
            b = sched.next_batch()
            if b is None:
                break
            M = b.n_rows
            Mp = -(-M // self.pad) * self.pad
            ids = np.empty(M, dtype=np.int32)
            row = 0
            for c in b.chunks:
                ids[row:row + c.length] = self.prompts[c.rid][c.start:c.start + c.length]
                row += c.length
            for k, r in enumerate(b.decodes):
                ids[row + k] = -(r + 1)
            sreq = np.full(M, -1, dtype=np.int32)
            spos = np.full(M, -1, dtype=np.int32)
            for r_, rid, k in b.samples:
                sreq[r_], spos[r_] = rid, rid * self.gen_len + k
            ctx = [sched.decode_context(r) for r in b.decodes]
            chunks = [B.hl_chunk(c.length, c.start, self.bt_dev[c.rid].data_ptr(),
                                 self.n_blocks[c.rid]) for c in b.chunks]
            ids_d, sreq_d, spos_d = self._up(ids), self._up(sreq), self._up(spos)
            if b.decodes:
                ctx_d = self._up(np.array(ctx, dtype=np.int32))
                bts_d = self._up(self.bt[b.decodes])
                dec = B.hl_decodes(len(b.decodes), ctx_d.data_ptr(), bts_d.data_ptr(),
                                   self.max_blocks, max(ctx))
            else:
                dec = B.hl_decodes(0, None, None, 0, 0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            x, y = self.x[:M], self.y[:M]
            B.hl_embed_rows(m.table, m.vocab, s.hidden, ids_d, self.last_tok, M, x)
            # layer l's first RMSNorm comes from layer l-1's down-projection
            # reduce; the last layer's reduce forms the final norm
            xa, xb = self.xn
            B.hl_rmsnorm(x, m.layers[0][0]["g_attn"], xa, M, Mp, s.hidden, s.rms_eps)
            for l, ((_, w), kv) in enumerate(zip(m.layers, self.kv)):
                g_next = m.layers[l + 1][0]["g_attn"] if l + 1 < len(m.layers) else m.g_final
                B.hl_layer_forward_chain(m.cfg, w, x, chunks, dec, kv, y, self.ws, self.ws_bytes,
                                         self.pad, xn_in=xa, g_next=g_next, xn_next=xb)
                x, y = y, x
                xa, xb = xb, xa
            B.hl_gemm_bf16(xa, m.lm, self.logits, None, Mp, Mp, m.vocab, s.hidden,
                           self.gws, self.gws_bytes)
            B.hl_argmax_rows(self.logits, M, m.vocab, sreq_d, spos_d, self.last_tok,
                             self.out_tokens)
            e1.record()
            events.append((e0, e1, bool(b.decodes)))
            if record:
                torch.cuda.synchronize()
                rows = [r_ for r_, _, _ in b.samples]
                lg = self.logits[rows].float().cpu().numpy()
                records.append(Record([(c.rid, c.start, c.length) for c in b.chunks],
                                      list(b.decodes), ctx, list(b.samples), lg))
            sched.commit(b)
        torch.cuda.synchronize()
        it_ms = [a.elapsed_time(z) for a, z, _ in events]
        total_ms = events[0][0].elapsed_time(events[-1][1]) if events else 0.0
        stats = RunStats(len(events), total_ms / 1e3, len(self.prompts) * self.gen_len,
                         int(sum(len(p) for p in self.prompts)),
                         [t for t, (_, _, d) in zip(it_ms, events) if d], it_ms)
        return stats, records

    def tokens(self) -> np.ndarray:
        return self.out_tokens.cpu().numpy().reshape(len(self.prompts), self.gen_len)


def cfg5_prompts(n: int, vocab: int, seed: int) -> List[np.ndarray]:
    rng = np.random.default_rng(seed)
    lens = rng.integers(50, 500, size=n, endpoint=True)
    return [rng.integers(0, vocab, size=int(l)).astype(np.int32) for l in lens]


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--requests", type=int, default=32)
    p.add_argument("--gen", type=int, default=100)
    p.add_argument("--budget", type=int, default=512)
    p.add_argument("--vocab", type=int, default=32000)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--repeats", type=int, default=2, help="runs (the first warms up)")
    a = p.parse_args()
    import torch
    torch.cuda.set_device(0)
    log(f"drawing {a.layers} Mistral-7B-shaped layers on the GPU ...")
    model = Model.random(MISTRAL_7B, a.layers, a.vocab, a.seed)
    prompts = cfg5_prompts(a.requests, a.vocab, a.seed + 1)
    stats = None
    for rep in range(a.repeats):
        loop = BatchingLoop(model, prompts, a.gen, a.budget, seed=a.seed)
        stats, _ = loop.run()
        toks = loop.tokens()
        assert (toks >= 0).all() and (toks < a.vocab).all(), "a token was not generated"
        log(f"run {rep}: {stats.iterations} iterations, {stats.seconds * 1e3:.1f} ms, "
            f"{stats.generated / stats.seconds:.0f} generated tokens/s")
        del loop
    tbt = np.array(stats.tbt_ms)
    res = {"metric": "generated tokens/s, 32-layer stall-free batching loop",
           "generated_tok_s": round(stats.generated / stats.seconds, 1),
           "total_tok_s": round((stats.generated + stats.prompt_tokens) / stats.seconds, 1),
           "seconds": round(stats.seconds, 4), "iterations": stats.iterations,
           "generated_tokens": stats.generated, "prompt_tokens": stats.prompt_tokens,
           "tbt_ms_p50": round(float(np.percentile(tbt, 50)), 3) if tbt.size else None,
           "tbt_ms_p99": round(float(np.percentile(tbt, 99)), 3) if tbt.size else None,
           "config": {"layers": a.layers, "requests": a.requests, "gen": a.gen,
                      "budget": a.budget, "vocab": a.vocab, "shape": "mistral7b",
                      "data": "synthetic, random weights"}}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

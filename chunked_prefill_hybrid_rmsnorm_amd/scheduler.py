"""Stall-free batching for a token budget (host side).

Sarathi-Serve digest, Algorithm 3 (the flow of one iteration): every
iteration forms one hybrid batch of at most ``budget`` rows --

1. one decode token for every admitted request whose prompt is fully
   prefilled (decodes are never held back by prefill);
2. the next chunk of the request whose prompt is partly prefilled, if any:
   ``min(prompt left, budget left)`` tokens (with new requests admitted only
   while budget is left, at most one prompt is ever partly prefilled);
3. new requests in arrival order while budget is left, each with a chunk of
   ``min(prompt, budget left)`` tokens, up to ``max_chunks`` chunks in the
   batch (the layer call's limit, HL_MAX_CHUNKS).

A chunk that completes its prompt yields the request's first generated token
from its last row; every decode row yields the next one.  A request leaves
after ``gen_len`` generated tokens (there is no end-of-sequence token), so
decode steps feed generated tokens 0 .. gen_len - 2.

Row order inside a batch is the library's: chunk rows (in chunk order), then
decode rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple


@dataclass
class Request:
    rid: int
    prompt_len: int
    gen_len: int
    prefilled: int = 0
    generated: int = 0

    @property
    def prefill_done(self) -> bool:
        return self.prefilled >= self.prompt_len

    @property
    def done(self) -> bool:
        return self.generated >= self.gen_len


@dataclass
class ChunkWork:
    rid: int
    start: int   # position of the chunk's first token
    length: int


@dataclass
class Batch:
    chunks: List[ChunkWork]
    decodes: List[int]                 # request ids, one row each
    # (row, request id, index of the generated token the row yields)
    samples: List[Tuple[int, int, int]] = field(default_factory=list)

    @property
    def n_chunk_rows(self) -> int:
        return sum(c.length for c in self.chunks)

    @property
    def n_rows(self) -> int:
        return self.n_chunk_rows + len(self.decodes)


class StallFreeScheduler:
    """Requests all arrive at the start, in ``prompt_lens`` order."""

    def __init__(self, prompt_lens: Sequence[int], gen_len: int, budget: int,
                 max_chunks: int = 16):
        if budget <= 0 or gen_len <= 0 or any(p <= 0 for p in prompt_lens):
            raise ValueError("budget, gen_len and every prompt length must be positive")
        if max_chunks <= 0:
            raise ValueError("max_chunks must be positive")
        self.budget = budget
        self.max_chunks = max_chunks
        self.reqs = [Request(i, int(p), gen_len) for i, p in enumerate(prompt_lens)]
        self.waiting: List[int] = list(range(len(self.reqs)))
        self.running: List[int] = []   # admitted and not finished, in admission order

    @property
    def finished(self) -> bool:
        return not self.waiting and not self.running

    def next_batch(self) -> Optional[Batch]:
        if self.finished:
            return None
        R = self.reqs
        decodes = [r for r in self.running if R[r].prefill_done]
        n_t = len(decodes)
        chunks: List[ChunkWork] = []
        partial = [r for r in self.running if not R[r].prefill_done]
        assert len(partial) <= 1, "more than one prompt partly prefilled"
        for r in partial:
            c = min(R[r].prompt_len - R[r].prefilled, self.budget - n_t)
            if c > 0:
                chunks.append(ChunkWork(r, R[r].prefilled, c))
                n_t += c
        # the layer call takes at most max_chunks chunks per batch
        while self.waiting and n_t < self.budget and len(chunks) < self.max_chunks:
            r = self.waiting.pop(0)
            self.running.append(r)
            c = min(R[r].prompt_len, self.budget - n_t)
            chunks.append(ChunkWork(r, 0, c))
            n_t += c
        b = Batch(chunks, decodes)
        row = 0
        for ch in chunks:
            row += ch.length
            if ch.start + ch.length == R[ch.rid].prompt_len:
                b.samples.append((row - 1, ch.rid, 0))
        for k, r in enumerate(decodes):
            b.samples.append((b.n_chunk_rows + k, r, R[r].generated))
        return b

    def decode_context(self, rid: int) -> int:
        """Cached tokens before a decode row of request ``rid`` (its position):
        the prompt plus every generated token but the one it feeds."""
        r = self.reqs[rid]
        return r.prompt_len + r.generated - 1

    def commit(self, b: Batch) -> None:
        R = self.reqs
        for ch in b.chunks:
            R[ch.rid].prefilled += ch.length
            if R[ch.rid].prefill_done:
                R[ch.rid].generated = 1
        for r in b.decodes:
            R[r].generated += 1
        self.running = [r for r in self.running if not R[r].done]


def max_batch(mem_gpu: int, mem_static: int, max_seq_len: int, kv_bytes_per_token: int,
              reserve: float = 0.0) -> int:
    """Most requests whose KV cache fits on the GPU at once.

    intelliparadigm.com article, section 4.1 (batch capacity): the batch size
    is the memory left after the model's parameters, divided by what one
    request's cache takes at the longest sequence,
    ``B = floor((MG - MS) / (L * mkv))`` with MG the GPU memory available, MS
    the parameters, L the longest sequence and mkv the KV bytes of one token
    (every layer).  The article keeps a share of the memory free against
    fragmentation (a fifth in its deployments); ``reserve`` is that share,
    taken off MG first.  Integer arithmetic, so the floor is exact.
    """
    if not 0.0 <= reserve < 1.0:
        raise ValueError("reserve must be in [0, 1)")
    if min(mem_gpu, mem_static, max_seq_len, kv_bytes_per_token) < 0 or \
            max_seq_len == 0 or kv_bytes_per_token == 0:
        raise ValueError("sizes must be non-negative and L, mkv positive")
    usable = mem_gpu - int(round(mem_gpu * reserve)) - mem_static
    return max(0, usable // (max_seq_len * kv_bytes_per_token))


def kv_bytes_per_token_model(shape, n_layers: int) -> int:
    """mkv of a model: one token's K and V for every kv head of every layer."""
    return shape.kv_bytes_per_token * n_layers

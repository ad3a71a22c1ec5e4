"""Batching-loop pieces around the layers -- TEST INFRASTRUCTURE ONLY.

Plain float64 numpy, like the layer oracle, and for the same users (tests,
smoke check, benchmark baseline).  One batch of the loop (Sarathi-Serve
digest, Algorithm 3: a hybrid batch per iteration; every decode row, and
every chunk's last row when the chunk completes its prompt, yields a token):

* the rows' input embeddings: a row gather from the table;
* the layers in turn, each with its own weights and paged KV (the layer
  oracle, ``layer_forward``);
* the final RMSNorm and the LM head (logits = xn · W_lmᵀ);
* the greedy choice: the index of the largest logit, the lowest index on
  ties.

Parity: pinned in ``tests/test_oracle_model.py`` -- the gather against a
one-hot product, the tie rule, and invariants of the composition (a prompt
prefilled in two calls equals one call; rows of a batch are independent of
each other).
"""
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .layer import layer_forward, rmsnorm


def embed(table: np.ndarray, ids: Sequence[int]) -> np.ndarray:
    """Rows ``table[ids[r]]`` (float64)."""
    return np.asarray(table, dtype=np.float64)[np.asarray(ids, dtype=np.int64)]


def greedy(logits: np.ndarray) -> np.ndarray:
    """Per row, the index of the largest value; on ties the lowest index."""
    logits = np.asarray(logits, dtype=np.float64)
    return np.argmax(logits, axis=-1)  # argmax returns the first maximum


def model_batch(shape, layers: List[Dict[str, np.ndarray]], table: np.ndarray, lm: np.ndarray,
                g_final: np.ndarray, ids: Sequence[int],
                chunks: Sequence[Tuple[int, int, Sequence[int]]], ctx_lens: Sequence[int],
                block_tables, kv_list: List[np.ndarray]) -> Tuple[np.ndarray, List[np.ndarray]]:
    """Logits of every row of one batch, and each layer's updated pages.

    ``ids`` are the rows' input tokens (chunk rows, then decode rows);
    ``chunks``, ``ctx_lens`` and ``block_tables`` are as for ``layer_forward``
    and shared by every layer (each layer has its own page pool in
    ``kv_list``)."""
    x = embed(table, ids)
    new_kv = []
    for w, kv in zip(layers, kv_list):
        r = layer_forward(shape, w, x, chunks, ctx_lens, block_tables, kv)
        x = r.out
        new_kv.append(r.kv_pages)
    xn = rmsnorm(x, g_final, shape.rms_eps)
    return xn @ np.asarray(lm, dtype=np.float64).T, new_kv

"""Turn generator output (bf16 bits) into the oracle's float64 arguments."""
import numpy as np

from chunked_prefill_hybrid_rmsnorm_amd.inputs import bf16_to_f32


def widen(bits):
    with np.errstate(invalid="ignore"):   # sentinel slots are NaN
        return bf16_to_f32(bits).astype(np.float64)


def oracle_weights(weights):
    return {k: widen(v) for k, v in weights.as_dict().items()}


def oracle_args(hb):
    """(shape, w, x, chunks, ctx_lens, block_tables, kv) for oracle.layer_forward."""
    chunks = [(c.length, c.start_pos, c.block_table) for c in hb.chunks]
    return (hb.shape, oracle_weights(hb.weights), widen(hb.x), chunks,
            [int(c) for c in hb.decodes.ctx_lens], hb.decodes.block_tables, widen(hb.kv_pages))

"""CPU oracle for the hybrid-batch decoder layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy.  It is what the HIP library is checked against
and nothing else: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP path and
imports nothing from the library package; its inputs are plain numpy arrays
(bf16 inputs arrive already widened).

Parity status of each function is stated in its docstring; the property
pins live in ``tests/test_oracle_*.py``.
"""
from .layer import (  # noqa: F401
    OracleResult,
    attention_row,
    layer_forward,
    prefix_reread_loads,
    rmsnorm,
    rope_rotate,
    silu,
    slot_of,
    swiglu_ffn,
)
from .model import embed, greedy, model_batch  # noqa: F401,E402

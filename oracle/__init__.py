"""fp64 CPU oracle for gated retention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library, and the library
never imports it.
"""
from .oracle import (  # noqa: F401
    build_oracle,
    oracle_decode_f64,
    oracle_max_threads,
    oracle_prefill_f64,
)
from .cross_attention import oracle_cross_attention_f64  # noqa: F401
from .output_gate import oracle_output_gate_f64  # noqa: F401
from .projection import log_sigmoid_f64, oracle_head_projection_f64  # noqa: F401
from .swa import oracle_swa_decode_f64, oracle_swa_prefill_f64, oracle_swa_ring_f64  # noqa: F401

"""Float64 CPU oracle for the In-Place TTT fast-weight prefill (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the HIP library and its binding never do.
"""
from .ipttt_oracle import (  # noqa: F401
    backward,
    chunk_ranges,
    conv_chunk,
    conv_chunk_backward,
    decode_steps,
    final_weight_entries,
    gate_up,
    initial_weight_grad_entries,
    prefill,
    prefill_prefix_form,
    prefill_prefix_form_stream,
    prefill_with_resets,
    silu,
    silu_grad,
    target_chunk,
)

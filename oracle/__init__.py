"""CPU reference (oracle) for SwiAttn routed dual-branch attention.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library and imports nothing from it.
"""
from .swiattn_ref import (  # noqa: F401
    anchor_key_range,
    attend_rows,
    compact,
    decode,
    decode_step,
    full_key_range,
    prefill,
    prefill_backward,
    prefill_backward_keys,
    prefill_backward_rows,
    regularizer,
    route,
    router_backward,
    softplus,
    swa_key_range,
)

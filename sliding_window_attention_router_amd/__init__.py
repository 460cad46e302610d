"""SwiAttn routed dual-branch attention on MI355X (gfx950).

The compute lives in the HIP shared library ``libswiattn.so`` (built from
``csrc/``); :mod:`.binding` marshals torch tensors into its C ABI.  Importing
this package does not load the library; the first call does, and raises if
the library has not been built.
"""
from .binding import (  # noqa: F401
    SwiAttnError,
    decode,
    decode_noalloc,
    decode_step,
    decode_workspace_size,
    lib,
    prefill,
    prefill_backward,
    prefill_branches,
    prefill_workspace_size,
    regularizer,
    route,
    router_backward,
)

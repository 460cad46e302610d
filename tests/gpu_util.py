"""Helpers for the GPU parity tests: device upload of seeded inputs, error
statistics, and the tolerances the tests enforce."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

# Attention outputs: max-abs error against the float64 reference on the same
# stored input values (bf16 inputs: 2e-2, float32 inputs: 1e-4).
TOL = {"bf16": 2e-2, "f32": 1e-4}
TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def ensure_built():
    from sliding_window_attention_router_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        from sliding_window_attention_router_amd import build

        build.build()
    binding.lib()


def dev(x, dtype=None, device="cuda"):
    """numpy -> torch on the GPU (values of bf16 arrays are bf16-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def diff_tolerance(diff_ref, n_channels, delta):
    """Bound on |diff_gpu - diff_ref| when every channel of both branch
    outputs is within delta of the reference:
    |sqrt(diff_gpu) - sqrt(diff_ref)| <= 2*delta*sqrt(n) (triangle
    inequality on the difference vector), hence
    |diff_gpu - diff_ref| <= 4*delta*sqrt(n*diff_ref) + 4*delta^2*n."""
    return 4 * delta * np.sqrt(n_channels * diff_ref) + 4 * delta * delta * n_channels

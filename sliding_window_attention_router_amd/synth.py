"""Seeded synthetic inputs for the SwiAttn hot path.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the method's arithmetic.  Tests feed the same arrays to the
HIP library and to the CPU reference, and the benchmark uses the same
recipes.

Shapes and statistics follow the workloads on the SwiAttn report (section 2:
1.5B model with a 1024-token window and a 32K context after YaRN; section 3:
mean full-attention ratio about 0.13, about 0.30 with the needle outside the
window and about 0.05 inside it).  The pages' evaluation suites need trained
weights and datasets; these synthetic inputs stand in for them.

All floating arrays are returned as float32 numpy arrays whose values are
exactly representable in the storage dtype ("bf16" values are float32 draws
rounded to bfloat16 by round-to-nearest-even), so converting them to a
torch.bfloat16 tensor is exact.
"""
from __future__ import annotations

import statistics
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "round_bf16",
    "tiny",
    "layer",
    "long_prefill",
    "structured",
    "structured_gate",
    "decode_cache",
    "Workload",
]


def round_bf16(x):
    """float32 -> float32 holding the nearest bfloat16 value (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.nan
    return out


def _normal(rng, shape, std=1.0, dtype="bf16"):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_bf16(x) if dtype == "bf16" else x


@dataclass
class Workload:
    name: str
    dtype: str  # "bf16" or "f32"
    W: int
    Q: np.ndarray = None  # [B,N,Hq,d]
    K: np.ndarray = None  # [B,N,Hkv,d]
    V: np.ndarray = None
    gate: np.ndarray = None  # uint8 [B,N,G]; None when the router makes it
    H: np.ndarray = None  # [B,N,hidden]
    r: np.ndarray = None  # [hidden,G]
    bias: np.ndarray = None  # float32 [G]
    extra: dict = field(default_factory=dict)


def tiny(seed=1, G=2, B=1, N=256, heads=2, d=64, W=64, p=0.25):
    """Tiny case: fp32, 2 heads (MHA), d=64, N=256, W=64, gate Bernoulli(p)
    per token per head group."""
    rng = np.random.default_rng(seed)
    Q = _normal(rng, (B, N, heads, d), dtype="f32")
    K = _normal(rng, (B, N, heads, d), dtype="f32")
    V = _normal(rng, (B, N, heads, d), dtype="f32")
    gate = (rng.random((B, N, G)) < p).astype(np.uint8)
    return Workload("tiny", "f32", W, Q, K, V, gate)


def router_bias(r, p):
    """Bias that makes P(H.r + bias > 0) = p for H ~ N(0, I): the logit is
    normal with standard deviation |r|, so bias = |r| * Phi^-1(p)."""
    norm = float(np.sqrt((np.asarray(r, dtype=np.float64) ** 2).sum(axis=0)).mean())
    return np.float32(norm * statistics.NormalDist().inv_cdf(p))


def layer(seed=2, B=1, N=4096, hidden=2048, heads=16, d=128, W=1024, p=0.13, G=1):
    """One layer's prefill: H ~ N(0,1), r ~ N(0, 1/hidden), bias set for a
    full-branch fraction p, bf16 Q/K/V ~ N(0,1), MHA."""
    rng = np.random.default_rng(seed)
    Q = _normal(rng, (B, N, heads, d))
    K = _normal(rng, (B, N, heads, d))
    V = _normal(rng, (B, N, heads, d))
    H = _normal(rng, (B, N, hidden))
    r = _normal(rng, (hidden, G), std=hidden ** -0.5)
    bias = np.full(G, router_bias(r, p), dtype=np.float32)
    return Workload("layer", "bf16", W, Q, K, V, None, H, r, bias)


def long_prefill(seed=3, B=1, N=32768, Hq=16, Hkv=4, d=128, W=1024, p=0.13,
                 gate_mode="bernoulli", G=1, with_router=False, hidden=2048):
    """Long prefill: bf16 GQA Q/K/V ~ N(0,1).  gate_mode "bernoulli" draws an
    i.i.d. Bernoulli(p) gate, "zeros"/"ones" give the pure-window and
    pure-full bounds.  with_router=True instead draws router inputs H, r and
    a bias for density p (the logits are then i.i.d. across tokens, so the
    gate bits are i.i.d. Bernoulli(p) as well)."""
    rng = np.random.default_rng(seed)
    Q = _normal(rng, (B, N, Hq, d))
    K = _normal(rng, (B, N, Hkv, d))
    V = _normal(rng, (B, N, Hkv, d))
    w = Workload("long", "bf16", W, Q, K, V)
    if with_router:
        w.H = _normal(rng, (B, N, hidden))
        w.r = _normal(rng, (hidden, G), std=hidden ** -0.5)
        w.bias = np.full(G, router_bias(w.r, p), dtype=np.float32)
    elif gate_mode == "bernoulli":
        w.gate = (rng.random((B, N, G)) < p).astype(np.uint8)
    elif gate_mode == "zeros":
        w.gate = np.zeros((B, N, G), np.uint8)
    elif gate_mode == "ones":
        w.gate = np.ones((B, N, G), np.uint8)
    else:
        raise ValueError(gate_mode)
    return w


def structured_gate(rng, N, p, run_lo=64, run_hi=512):
    """Alternating runs starting with an 'off' run: on-runs of U{run_lo..run_hi}
    tokens, off-runs of U{round(run_lo(1-p)/p)..round(run_hi(1-p)/p)} tokens,
    so the expected on-fraction is p.  Truncated at N."""
    g = np.zeros(N, np.uint8)
    off_lo = int(round(run_lo * (1 - p) / p))
    off_hi = int(round(run_hi * (1 - p) / p))
    pos, on = 0, False
    while pos < N:
        n = int(rng.integers(run_lo, run_hi + 1)) if on else int(rng.integers(off_lo, off_hi + 1))
        if on:
            g[pos : pos + n] = 1
        pos += n
        on = not on
    return g


def structured(p, seed=None, B=1, N=32768, heads=16, d=128, W=1024, G=1):
    """Structured routing: bf16 MHA Q/K/V ~ N(0,1); gate in contiguous runs
    of 64-512 tokens at density p (seed 4 for p=0.30, 40 for p=0.05)."""
    if seed is None:
        seed = 4 if p >= 0.2 else 40
    rng = np.random.default_rng(seed)
    Q = _normal(rng, (B, N, heads, d))
    K = _normal(rng, (B, N, heads, d))
    V = _normal(rng, (B, N, heads, d))
    gate = np.stack([np.stack([structured_gate(rng, N, p) for _ in range(G)], -1) for _ in range(B)])
    return Workload("structured", "bf16", W, Q, K, V, gate)


def decode_cache(seed=5, B=64, Lmax=32768, Hq=16, Hkv=4, d=128, W=1024, p=0.13,
                 G=1, cache_len=None, gate=None, device="cpu"):
    """Routed decode inputs as torch bf16 tensors on `device` (the cache is
    2 GiB per tensor at full size, so it is drawn where it will live):
    q [B,Hq,d], Kc/Vc [B,Lmax,Hkv,d] ~ N(0,1); gate [B,G] i.i.d. Bernoulli(p)
    (numpy draw, uint8); cache_len int32 [B] (default Lmax everywhere)."""
    import torch

    gen = torch.Generator(device=device).manual_seed(seed)
    bf = torch.bfloat16
    q = torch.randn(B, Hq, d, generator=gen, device=device, dtype=torch.float32).to(bf)
    Kc = torch.empty(B, Lmax, Hkv, d, dtype=bf, device=device)
    Vc = torch.empty(B, Lmax, Hkv, d, dtype=bf, device=device)
    for t in (Kc, Vc):
        for b in range(B):
            t[b] = torch.randn(Lmax, Hkv, d, generator=gen, device=device, dtype=torch.float32).to(bf)
    rng = np.random.default_rng(seed)
    if gate is None:
        gate = (rng.random((B, G)) < p).astype(np.uint8)
    if cache_len is None:
        cache_len = np.full(B, Lmax, np.int32)
    return {"q": q, "Kc": Kc, "Vc": Vc, "gate": np.asarray(gate, np.uint8),
            "cache_len": np.asarray(cache_len, np.int32), "W": W}

"""GPU parity of the router gradient through the straight-through gate
(swiattn_router_backward) against the float64 CPU reference.

Inputs are seeded and synthetic on both sides: dO and the two branch
outputs ~ N(0,1), router logits z ~ N(0, 2^2) in float32, H ~ N(0,1),
r ~ N(0, 1/hidden).  Tolerances follow from float32 summation: a sum of n
products carries an error of at most about n * 2^-24 of the sum of their
magnitudes (the kernels add at most 32 products per lane plus a 6-level
wave tree for dz, and 32 tokens per split plus 1024 split sums for dr), and
dH is rounded once to its storage type (2^-8 relative for bf16)."""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_router_amd import synth
from tests.gpu_util import TORCH_DTYPE, dev, ensure_built, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    yield
    torch.cuda.empty_cache()


def swa():
    import sliding_window_attention_router_amd as m

    return m


def _inputs(seed, B, N, Hq, d, hidden, G, dtype):
    rng = np.random.default_rng(seed)
    rnd = (lambda s, sc=1.0: synth.round_bf16((rng.standard_normal(s, dtype=np.float32) * sc).astype(np.float32))) \
        if dtype == "bf16" else (lambda s, sc=1.0: (rng.standard_normal(s, dtype=np.float32) * sc).astype(np.float32))
    dO, Of, Os = rnd((B, N, Hq, d)), rnd((B, N, Hq, d)), rnd((B, N, Hq, d))
    H = rnd((B, N, hidden))
    r = rnd((hidden, G), hidden ** -0.5)
    z = (rng.standard_normal((B, N, G), dtype=np.float32) * 2.0).astype(np.float32)
    z.reshape(-1)[:3] = [0.0, 30.0, -30.0]  # the sigmoid's centre and tails
    return dO, Of, Os, z, H, r


def _magnitudes(dO, Of, Os, z, G):
    """m[b,t,g] = sigmoid'(z) * sum |dO (O_full - O_swa)| over the group."""
    B, N, Hq, d = dO.shape
    a = np.abs(np.asarray(dO, np.float64) * (np.asarray(Of, np.float64) - np.asarray(Os, np.float64)))
    s = a.sum(axis=3).reshape(B, N, G, Hq // G).sum(axis=3)
    u = np.exp(-np.abs(np.asarray(z, np.float64)))
    return s * u / ((1.0 + u) * (1.0 + u))


def _check(out, ref, m, H, r, dtype, rows=None):
    dz, dH, dr, dbias = (host(t) for t in out)
    ref_dz, ref_dH = ref["dz"], ref["dH"]
    if rows is not None:
        dz_s, dH_s = dz[:, rows], dH[:, rows]
    else:
        dz_s, dH_s = dz, dH
    ez = np.abs(dz_s - ref_dz)
    assert np.all(ez <= 1e-5 * m + 1e-30), f"dz: worst {np.max(ez / (m + 1e-30)):.3e} of magnitude"
    rl = 2.0 ** -8 if dtype == "bf16" else 1e-6
    hm = (np.abs(ref_dz) + m) @ np.abs(np.asarray(r, np.float64)).T
    eh = np.abs(dH_s - ref_dH)
    assert np.all(eh <= rl * np.abs(ref_dH) + 2e-5 * hm + 1e-30), \
        f"dH: worst {np.max(eh / (rl * np.abs(ref_dH) + 2e-5 * hm + 1e-30)):.3e} of bound"
    return dz, dH, dr, dbias


CASES = [
    # B, N,    Hq, d,   hidden, G, dtype
    (1, 1000, 16, 128, 2048, 1, "bf16"),
    (2, 333, 8, 64, 256, 2, "bf16"),     # two groups, ragged N (not a split multiple)
    (1, 1, 4, 128, 64, 4, "bf16"),       # one token, one head per group
    (3, 130, 12, 64, 96, 3, "f32"),      # float32, three groups of four heads
    (1, 517, 2, 64, 2056, 1, "f32"),     # hidden past one column block
    (1, 300, 16, 64, 128, 1, "bf16"),    # 2 x 64 pieces of 8 elements per group: loads issued together
    (2, 77, 16, 128, 64, 1, "f32"),      # 4 x 64 pieces per group, float32
]


@pytest.mark.parametrize("B,N,Hq,d,hidden,G,dtype", CASES)
def test_router_backward(B, N, Hq, d, hidden, G, dtype):
    say(f"router backward B={B} N={N} Hq={Hq} d={d} hidden={hidden} G={G} {dtype}")
    dO, Of, Os, z, H, r = _inputs(N + hidden + G, B, N, Hq, d, hidden, G, dtype)
    td = TORCH_DTYPE[dtype]
    out = swa().router_backward(dev(dO, td), dev(Of, td), dev(Os, td), dev(z), dev(H, td), dev(r, td))
    torch.cuda.synchronize()
    ref = oracle.router_backward(dO, Of, Os, z, H, r)
    m = _magnitudes(dO, Of, Os, z, G)
    dz, dH, dr, dbias = _check(out, ref, m, H, r, dtype)
    Hd = np.abs(np.asarray(H, np.float64))
    tol_r = 1e-4 * np.einsum("btk,btg->kg", Hd, np.abs(ref["dz"]) + m) + 1e-30
    tol_b = 1e-4 * (np.abs(ref["dz"]) + m).sum(axis=(0, 1)) + 1e-30
    er = np.abs(dr - ref["dr"])
    eb = np.abs(dbias - ref["dbias"])
    say(f"  dr worst {np.max(er / tol_r):.3e} of bound, dbias worst {np.max(eb / tol_b):.3e} of bound")
    assert np.all(er <= tol_r) and np.all(eb <= tol_b)


def test_router_backward_identical_branches_give_zero():
    B, N, Hq, d, hidden, G = 1, 200, 4, 64, 64, 2
    dO, Of, _, z, H, r = _inputs(61, B, N, Hq, d, hidden, G, "bf16")
    bf = torch.bfloat16
    Ofg = dev(Of, bf)
    dz, dH, dr, dbias = swa().router_backward(dev(dO, bf), Ofg, Ofg, dev(z), dev(H, bf), dev(r, bf))
    torch.cuda.synchronize()
    for t in (dz, dH, dr, dbias):
        assert torch.count_nonzero(t).item() == 0


def test_router_backward_32k_layer():
    """The layer's size: N=32768, 16 heads, d=128, hidden 2048, one gate
    group, bf16; sampled tokens for dz and dH, every token for dr and dbias;
    two runs bitwise equal."""
    B, N, Hq, d, hidden, G = 1, 32768, 16, 128, 2048, 1
    say("router backward N=32768 Hq=16 d=128 hidden=2048 G=1 bf16")
    dO, Of, Os, z, H, r = _inputs(62, B, N, Hq, d, hidden, G, "bf16")
    bf = torch.bfloat16
    args = (dev(dO, bf), dev(Of, bf), dev(Os, bf), dev(z), dev(H, bf), dev(r, bf))
    out1 = swa().router_backward(*args)
    out2 = swa().router_backward(*args)
    torch.cuda.synchronize()
    for a, b in zip(out1, out2):
        assert torch.equal(a, b), "two runs differ"
    rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N),
                                     np.random.default_rng(63).choice(N, 512, replace=False)]))
    ref_rows = oracle.router_backward(dO[:, rows], Of[:, rows], Os[:, rows], z[:, rows], H[:, rows], r)
    m_rows = _magnitudes(dO[:, rows], Of[:, rows], Os[:, rows], z[:, rows], G)
    _check(out1, ref_rows, m_rows, H, r, "bf16", rows=rows)
    ref = oracle.router_backward(dO, Of, Os, z, H, r)
    m = _magnitudes(dO, Of, Os, z, G)
    dr, dbias = host(out1[2]), host(out1[3])
    Hd = np.abs(np.asarray(H, np.float64))
    tol_r = 1e-4 * np.einsum("btk,btg->kg", Hd, np.abs(ref["dz"]) + m) + 1e-30
    tol_b = 1e-4 * (np.abs(ref["dz"]) + m).sum(axis=(0, 1)) + 1e-30
    er = np.abs(dr - ref["dr"])
    eb = np.abs(dbias - ref["dbias"])
    say(f"  dr worst {np.max(er / tol_r):.3e} of bound, dbias worst {np.max(eb / tol_b):.3e} of bound")
    assert np.all(er <= tol_r) and np.all(eb <= tol_b)

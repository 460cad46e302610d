"""GPU parity of the both-branch prefill that returns both branch outputs
(swiattn_prefill_branches) against the float64 oracle, and the router's
gradient fed from that one pass.

O_FULL and O_SWA of every row are held to the output tolerance (bf16 2e-2,
float32 1e-4); the gated output and the distance must equal those of the
plain both-branch call bitwise (the same kernels and order)."""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_router_amd import synth
from tests.gpu_util import TOL, TORCH_DTYPE, dev, ensure_built, host, max_abs, say
from tests.test_gpu_router_grad import _check, _magnitudes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    yield
    torch.cuda.empty_cache()


def swa():
    import sliding_window_attention_router_amd as m

    return m


def _qkv(seed, B, N, Hq, Hkv, d, dtype):
    rng = np.random.default_rng(seed)
    mk = (lambda s: synth.round_bf16(rng.standard_normal(s, dtype=np.float32))) if dtype == "bf16" \
        else (lambda s: rng.standard_normal(s, dtype=np.float32))
    return mk((B, N, Hq, d)), mk((B, N, Hkv, d)), mk((B, N, Hkv, d))


CASES = [
    # B, N,   Hq, Hkv, G, d,  W,   A,  dtype
    (1, 1000, 8, 2, 1, 128, 200, 0, "bf16"),
    (2, 777, 4, 4, 2, 64, 100, 0, "bf16"),
    (1, 600, 8, 1, 4, 128, 64, 40, "bf16"),   # anchors: rows i < W + A have O_FULL = O_SWA
    (1, 300, 4, 2, 2, 64, 50, 0, "f32"),
    (1, 200, 4, 2, 1, 128, 400, 0, "bf16"),   # W > N: both branches identical
]


@pytest.mark.parametrize("B,N,Hq,Hkv,G,d,W,A,dtype", CASES)
def test_prefill_branches(B, N, Hq, Hkv, G, d, W, A, dtype):
    say(f"branches B={B} N={N} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} A={A} {dtype}")
    Q, K, V = _qkv(N + d + A, B, N, Hq, Hkv, d, dtype)
    gate = (np.random.default_rng(N).random((B, N, G)) < 0.3).astype(np.uint8)
    td = TORCH_DTYPE[dtype]
    args = (dev(Q, td), dev(K, td), dev(V, td), dev(gate), W)
    O, diff, Of, Os = swa().prefill_branches(*args, anchors=A)
    O2, diff2 = swa().prefill(*args, both_branch=True, anchors=A)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(diff, diff2)
    ref = oracle.prefill(Q, K, V, gate, W, both_branch=True, anchors=A)
    ef, es = max_abs(host(Of), ref["O_full"]), max_abs(host(Os), ref["O_swa"])
    say(f"  O_FULL max-abs {ef:.3e}, O_SWA max-abs {es:.3e}")
    assert ef <= TOL[dtype] and es <= TOL[dtype]
    # the gated output is one of the two branch outputs, bit for bit
    sel = np.stack([gate[:, :, h * G // Hq] for h in range(Hq)], axis=2).astype(bool)[..., None]
    assert np.array_equal(host(O), np.where(sel, host(Of), host(Os)))


def test_router_gradient_from_one_branches_pass():
    """Router -> branches pass -> router gradient, against the oracle's chain
    (the branch outputs of one pass replace the two extra prefills)."""
    B, N, Hq, Hkv, G, d, W, hidden = 1, 1500, 8, 2, 1, 64, 200, 256
    w = synth.long_prefill(seed=53, B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, W=W, p=0.3, G=G, with_router=True,
                           hidden=hidden)
    bf = torch.bfloat16
    gate, _, _, z = swa().route(dev(w.H, bf), dev(w.r, bf), dev(w.bias), want_z=True)
    _, _, Of, Os = swa().prefill_branches(dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), gate, W)
    dO = synth.round_bf16(np.random.default_rng(54).standard_normal(w.Q.shape, dtype=np.float32))
    dz, dH, dr, dbias = swa().router_backward(dev(dO, bf), Of, Os, z, dev(w.H, bf), dev(w.r, bf))
    torch.cuda.synchronize()
    rz = oracle.route(w.H, w.r, w.bias)
    rp = oracle.prefill(w.Q, w.K, w.V, rz["gate"], W, both_branch=True)
    # the oracle takes the GPU's branch outputs rounded to bf16 as stored, so
    # that the check isolates the gradient; the branch outputs themselves are
    # checked against rp above their own tolerance
    assert max_abs(host(Of), rp["O_full"]) <= TOL["bf16"] and max_abs(host(Os), rp["O_swa"]) <= TOL["bf16"]
    ref = oracle.router_backward(dO, host(Of), host(Os), host(z), w.H, w.r)
    m = _magnitudes(dO, host(Of), host(Os), host(z), G)
    dz_, dH_, dr_, dbias_ = _check((dz, dH, dr, dbias), ref, m, w.H, w.r, "bf16")
    Hd = np.abs(np.asarray(w.H, np.float64))
    tol_r = 1e-4 * np.einsum("btk,btg->kg", Hd, np.abs(ref["dz"]) + m) + 1e-30
    tol_b = 1e-4 * (np.abs(ref["dz"]) + m).sum(axis=(0, 1)) + 1e-30
    er, eb = np.abs(dr_ - ref["dr"]), np.abs(dbias_ - ref["dbias"])
    say(f"router gradient from one branches pass: dr worst {np.max(er / tol_r):.3e} of bound, "
        f"dbias worst {np.max(eb / tol_b):.3e} of bound")
    assert np.all(er <= tol_r) and np.all(eb <= tol_b)

"""GPU parity of the attention backward of the hard-gated prefill
(swiattn_prefill_backward) against the float64 CPU reference.

Q, K, V and dO are seeded and synthetic (the same stored values on both
sides); O is the library's forward output, as in a forward -> backward
pipeline (the reference forms its own).  Tolerance: max-abs error at most
2^-6 of the largest reference magnitude of that gradient for bf16 (outputs
rounded to bf16, O rounded to bf16 in the forward) and 1e-4 of it for
float32."""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_router_amd import synth
from tests.gpu_util import TORCH_DTYPE, dev, ensure_built, host, max_abs, say

pytestmark = pytest.mark.gpu

REL = {"bf16": 2.0 ** -6, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    yield
    torch.cuda.empty_cache()


def swa():
    import sliding_window_attention_router_amd as m

    return m


def _inputs(seed, B, N, Hq, Hkv, d, dtype):
    rng = np.random.default_rng(seed)
    mk = (lambda s: synth.round_bf16(rng.standard_normal(s, dtype=np.float32))) if dtype == "bf16" \
        else (lambda s: rng.standard_normal(s, dtype=np.float32))
    return mk((B, N, Hq, d)), mk((B, N, Hkv, d)), mk((B, N, Hkv, d)), mk((B, N, Hq, d))


CASES = [
    # B, N,   Hq, Hkv, G, d,  W,   p,   dtype
    (1, 300, 4, 2, 1, 128, 64, 0.3, "bf16"),     # GQA 2:1, ragged
    (2, 200, 4, 4, 2, 64, 50, 0.4, "bf16"),      # MHA, two gate groups, d=64
    (1, 257, 8, 2, 4, 128, 100, 0.5, "bf16"),    # gate groups inside a KV group
    (1, 150, 4, 2, 1, 128, 400, 0.5, "bf16"),    # W > N
    (1, 120, 4, 1, 1, 64, 1, 0.0, "bf16"),       # W = 1: dQ = dK = 0
    (1, 200, 4, 2, 2, 64, 30, 1.0, "bf16"),      # gate all ones
    (1, 220, 4, 2, 1, 128, 40, 0.3, "f32"),      # float32
    # several gathered tiles per head for dQ (about 460 routed rows) and many
    # window and gathered tiles per key block for dK, dV; ragged N
    (1, 1531, 8, 2, 2, 128, 200, 0.3, "bf16"),
    (2, 777, 4, 4, 1, 64, 97, 0.5, "bf16"),
    # W a multiple of the 64-row tile: row tiles whose rows all see a key
    # block's 64 keys border tiles that do not, on both sides
    (1, 705, 4, 2, 1, 128, 128, 0.2, "bf16"),
    (1, 650, 4, 4, 2, 64, 192, 0.0, "bf16"),
]


@pytest.mark.parametrize("B,N,Hq,Hkv,G,d,W,p,dtype", CASES)
def test_prefill_backward(B, N, Hq, Hkv, G, d, W, p, dtype):
    say(f"backward B={B} N={N} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} p={p} {dtype}")
    Q, K, V, dO = _inputs(N * 5 + d, B, N, Hq, Hkv, d, dtype)
    gate = (np.random.default_rng(N + W).random((B, N, G)) < p).astype(np.uint8)
    td = TORCH_DTYPE[dtype]
    Qg, Kg, Vg, dOg, gg = dev(Q, td), dev(K, td), dev(V, td), dev(dO, td), dev(gate)
    O, _ = swa().prefill(Qg, Kg, Vg, gg, W)
    dQ, dK, dV = swa().prefill_backward(Qg, Kg, Vg, O, dOg, gg, W)
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(Q, K, V, gate, W, dO)
    zb = zero_gradient_bounds(Q, K, V, dO, scale=d ** -0.5) if W == 1 else None
    for name, got in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        r = ref[name]
        g = host(got)
        err = max_abs(g, r)
        if np.abs(r).max() < 1e-12:
            # the exact gradient is zero: element-wise rounding bound
            bnd = zb[name]
            share = np.abs(g - r) / bnd
            say(f"  {name} exact zero: max-abs {err:.3e}, largest share of its element bound "
                f"{share.max():.3f} (largest bound {bnd.max():.3e})")
            assert np.all(np.abs(g - r) <= bnd)
            continue
        bound = REL[dtype] * max(float(np.abs(r).max()), 1e-30)
        say(f"  {name} max-abs {err:.3e} (bound {bound:.3e})")
        assert err <= bound


def zero_gradient_bounds(Q, K, V, dO, scale):
    """Element-wise bounds on the float32 rounding left in dQ and dK when
    the exact gradient is zero (W = 1: each row attends to itself alone, so
    P = 1 and dS = dP - D = <dO_i, v_i> - <dO_i, O_i> with O_i = v_i).

    The two dot products are summed in different orders by the kernels:
      D  (row pass)  each half-wave lane g in {0, 1} runs a float32 fma chain
                     over channels 16 ks + 8 g + e (ks = 0 .. d/16-1,
                     e = 0 .. 7), then the two halves are added;
      dP (products)  the matrix core adds 16 exact bf16 products per k-step
                     into a float32 accumulator, d/16 k-steps.
    First-order rounding analysis (terms of order u^2 are dropped): each
    rounded addition errs by at most u = 2^-24 of its result, so
    |fl(D) - D| <= u (sum of |partial sums| of the chain, both halves, plus
    |D|), and a k-step errs by at most u (|new accumulator| + sum of |its 16
    products|): one rounding of the step's 16-term sum of exact products and
    one of its addition to the accumulator.  Their sum bounds |dP - D|; dS
    is rounded to bf16 (factor 1 + 2^-8), dQ_i = scale dS_i k_i and
    dK_i = scale sum_h dS_ih q_ih (one term per head), each rounded to the
    output type (1 + 2^-8)."""
    Q, K, V, dO = (np.asarray(x, np.float64) for x in (Q, K, V, dO))
    B, N, Hq, d = Q.shape
    HK = Hq // K.shape[2]
    Vq = np.repeat(V, HK, axis=2)
    t = dO * Vq  # exact products of the stored values, [B,N,Hq,d]
    u = 2.0 ** -24
    sD = np.abs(t.sum(axis=3))
    for g in (0, 1):
        order = [16 * ks + 8 * g + e for ks in range(d // 16) for e in range(8)]
        sD = sD + np.abs(np.cumsum(t[..., order], axis=3)).sum(axis=3)
    steps = t.reshape(B, N, Hq, d // 16, 16)
    acc = np.cumsum(steps.sum(axis=4), axis=3)
    sP = np.abs(acc).sum(axis=3) + np.abs(t).sum(axis=3)
    ds = u * (sD + sP) * (1 + 2.0 ** -8)  # [B,N,Hq]
    out = 1 + 2.0 ** -8
    dQ = scale * ds[..., None] * np.abs(np.repeat(K, HK, axis=2)) * out
    dK = (scale * ds[..., None] * np.abs(Q)).reshape(B, N, K.shape[2], HK, d).sum(axis=3) * out
    return {"dQ": dQ + 1e-30, "dK": dK + 1e-30}


def test_prefill_backward_32k_layer():
    """N=32768, GQA 16/4, d=128, W=1024, gate Bernoulli(0.13): two runs
    bitwise equal; per KV head the dK rows sum to 0 and the dV rows sum to
    the dO rows of its query heads (softmax rows sum to one); sampled dQ
    rows and sampled dK, dV keys against the reference."""
    say("backward N=32768 GQA 16/4 W=1024 gate Bernoulli(0.13)")
    W = 1024
    w = synth.long_prefill(seed=3)
    bf = torch.bfloat16
    rng = np.random.default_rng(91)
    dO = synth.round_bf16(rng.standard_normal(w.Q.shape, dtype=np.float32))
    Qg, Kg, Vg, dOg, gg = dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), dev(dO, bf), dev(w.gate)
    O, _ = swa().prefill(Qg, Kg, Vg, gg, W)
    g1 = swa().prefill_backward(Qg, Kg, Vg, O, dOg, gg, W)
    g2 = swa().prefill_backward(Qg, Kg, Vg, O, dOg, gg, W)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b), "two runs differ"
    dQ, dK, dV = (host(t) for t in g1)
    assert np.all(np.isfinite(dQ)) and np.all(np.isfinite(dK)) and np.all(np.isfinite(dV))
    Hq, Hkv = w.Q.shape[2], w.K.shape[2]
    sum_dO = dO.astype(np.float64).reshape(1, -1, Hkv, Hq // Hkv, 128).sum(axis=(1, 3))  # [1,Hkv,d]
    scale_v = np.abs(dO).astype(np.float64).reshape(1, -1, Hkv, Hq // Hkv, 128).sum(axis=(1, 3))
    ev = np.abs(dV.sum(axis=1) - sum_dO)
    say(f"  sum dV - sum dO: worst {np.max(ev / scale_v):.3e} of sum |dO|")
    assert np.all(ev <= 2.0 ** -6 * scale_v)
    sk = np.abs(dK.sum(axis=1))
    mk = np.abs(dK).sum(axis=1)
    say(f"  |sum dK|: worst {np.max(sk / mk):.3e} of sum |dK|")
    assert np.all(sk <= 2.0 ** -5 * mk)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(W - 4, W + 4), np.arange(32760, 32768),
                                     rng.choice(np.flatnonzero(w.gate[0, :, 0]), 24, replace=False),
                                     rng.choice(np.flatnonzero(w.gate[0, :, 0] == 0), 24, replace=False)]))
    ref = oracle.prefill_backward_rows(w.Q, w.K, w.V, w.gate, W, dO, rows)
    err = max_abs(dQ[:, rows], ref)
    bound = REL["bf16"] * float(np.abs(ref).max())
    say(f"  {rows.size} sampled dQ rows x 16 heads: max-abs {err:.3e} (bound {bound:.3e})")
    assert err <= bound
    # sampled keys of every KV head: the first key block (every gate=1 row
    # of the sequence sees keys 0..70), block and window edges, the middle,
    # the last window and the end
    N = w.Q.shape[1]
    keys = np.array([0, 1, 63, 64, 70, W - 1, W, 1100, 5000, N // 2, N // 2 + 1, N - 1500, N - W - 40,
                     N - W - 1, N - W, N - W + 5, N - 65, N - 2, N - 1])
    refk = oracle.prefill_backward_keys(w.Q, w.K, w.V, w.gate, W, dO, keys)
    for name, got in (("dK", dK), ("dV", dV)):
        r = refk[name]
        err = max_abs(got[:, keys], r)
        bound = REL["bf16"] * float(np.abs(r).max())
        say(f"  {keys.size} sampled {name} keys x {Hkv} KV heads: max-abs {err:.3e} (bound {bound:.3e})")
        assert err <= bound


@pytest.mark.parametrize("Hq,Hkv,G,d,W,p", [
    (16, 4, 1, 128, 1024, 0.13),   # the long-prefill heads at a quarter of its length
    (16, 16, 2, 64, 256, 0.3),     # MHA, two gate groups, d=64
])
def test_prefill_backward_8k_sampled(Hq, Hkv, G, d, W, p):
    """N=8192: the dQ grid holds 64 row tiles per head of each kind (gathered
    gate=1 rows, heaviest first, then the window rows), dK/dV 128 key blocks
    per KV head, so every grid runs in several waves of workgroups.  Two runs
    bitwise equal; sampled dQ rows (start, window edge, end, routed and
    unrouted) and sampled dK, dV keys of every KV head against the
    reference."""
    N, B = 8192, 1
    say(f"backward N={N} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} p={p}")
    rng = np.random.default_rng(93)
    w = synth.long_prefill(seed=94, N=N, Hq=Hq, Hkv=Hkv, d=d, W=W, p=p)
    gate = (rng.random((B, N, G)) < p).astype(np.uint8) if G > 1 else w.gate
    dO = synth.round_bf16(rng.standard_normal(w.Q.shape, dtype=np.float32))
    bf = torch.bfloat16
    Qg, Kg, Vg, dOg, gg = dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), dev(dO, bf), dev(gate)
    O, _ = swa().prefill(Qg, Kg, Vg, gg, W)
    g1 = swa().prefill_backward(Qg, Kg, Vg, O, dOg, gg, W)
    g2 = swa().prefill_backward(Qg, Kg, Vg, O, dOg, gg, W)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b), "two runs differ"
    dQ, dK, dV = (host(x) for x in g1)
    assert np.all(np.isfinite(dQ)) and np.all(np.isfinite(dK)) and np.all(np.isfinite(dV))
    routed = np.flatnonzero(gate[0, :, 0])
    unrouted = np.flatnonzero(gate[0, :, 0] == 0)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(W - 3, W + 3), np.arange(N - 4, N),
                                     rng.choice(routed, 24, replace=False),
                                     rng.choice(unrouted, 24, replace=False)]))
    ref = oracle.prefill_backward_rows(w.Q, w.K, w.V, gate, W, dO, rows)
    err = max_abs(dQ[:, rows], ref)
    bound = REL["bf16"] * float(np.abs(ref).max())
    say(f"  {rows.size} sampled dQ rows x {Hq} heads: max-abs {err:.3e} (bound {bound:.3e})")
    assert err <= bound
    keys = np.array([0, 1, 64, W - 1, W, N // 3, N // 2, N - W - 1, N - W, N - 65, N - 1])
    refk = oracle.prefill_backward_keys(w.Q, w.K, w.V, gate, W, dO, keys)
    for name, got in (("dK", dK), ("dV", dV)):
        r = refk[name]
        err = max_abs(got[:, keys], r)
        bound = REL["bf16"] * float(np.abs(r).max())
        say(f"  {keys.size} sampled {name} keys x {Hkv} KV heads: max-abs {err:.3e} (bound {bound:.3e})")
        assert err <= bound


"""GPU parity of the global-anchor variant of the window branch (every window
query also sees the first A keys; weimeta SWA glossary, pitfall 1, fix 2)
against the float64 CPU reference, through the anchored C ABI entry points."""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_router_amd import synth
from tests.gpu_util import TOL, TORCH_DTYPE, dev, diff_tolerance, ensure_built, host, max_abs, say

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


def _gpu(Q, K, V, gate, W, A, dtype, both=False):
    td = TORCH_DTYPE[dtype]
    O, diff = swa().prefill(dev(Q, td), dev(K, td), dev(V, td), dev(gate), W, both_branch=both,
                            anchors=A)
    torch.cuda.synchronize()
    return host(O), (host(diff) if diff is not None else None)


ANCHOR_CASES = [
    # B, N,   Hq, Hkv, G, d,  W,   A,   p,   dtype
    (1, 1000, 8, 2, 1, 128, 200, 256, 0.2, "bf16"),   # A a block multiple, GQA 4:1, ragged tail
    (1, 1000, 8, 2, 1, 128, 200, 100, 0.2, "bf16"),   # A inside a block
    (2, 777, 4, 4, 2, 64, 100, 37, 0.3, "bf16"),      # MHA, two gate groups, d=64
    (1, 530, 8, 1, 4, 128, 64, 300, 0.5, "bf16"),     # A > W; gate groups inside a KV group
    (1, 300, 2, 2, 2, 128, 512, 64, 0.5, "bf16"),     # W > N: anchors inside the window
    (1, 400, 4, 2, 1, 128, 50, 1, 0.4, "bf16"),       # one anchor
    (1, 350, 4, 2, 1, 128, 100, 1000, 0.0, "bf16"),   # A > N: every row sees [0, i]
    (1, 2100, 16, 4, 1, 64, 256, 256, 0.2, "bf16"),   # many window tiles and far chunks
    (1, 400, 4, 2, 2, 128, 70, 90, 0.4, "f32"),       # float32 path (one workgroup per tile)
    (1, 300, 4, 4, 1, 64, 40, 200, 0.3, "f32"),       # float32, d=64, anchor blocks overlap windows
]


@pytest.mark.parametrize("B,N,Hq,Hkv,G,d,W,A,p,dtype", ANCHOR_CASES)
def test_prefill_anchored(B, N, Hq, Hkv, G, d, W, A, p, dtype):
    say(f"anchored prefill B={B} N={N} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} A={A} p={p} {dtype}")
    Q, K, V = _qkv(N * 3 + A, B, N, Hq, Hkv, d, dtype)
    gate = (np.random.default_rng(N + A).random((B, N, G)) < p).astype(np.uint8)
    O, _ = _gpu(Q, K, V, gate, W, A, dtype)
    ref = oracle.prefill(Q, K, V, gate, W, anchors=A)["O"]
    err = max_abs(O, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= TOL[dtype]


def test_anchors_covering_everything_is_causal():
    """W + A >= N: the window branch with anchors is full causal attention,
    so gate 0 and gate 1 give the same rows (within the tolerance)."""
    B, N, Hq, Hkv, G, d, W, A = 1, 500, 4, 2, 1, 128, 200, 300
    Q, K, V = _qkv(41, B, N, Hq, Hkv, d, "bf16")
    O0, _ = _gpu(Q, K, V, np.zeros((B, N, G), np.uint8), W, A, "bf16")
    O1, _ = _gpu(Q, K, V, np.ones((B, N, G), np.uint8), W, A, "bf16")
    ref = oracle.prefill(Q, K, V, np.ones((B, N, G), np.uint8), W)["O"]
    assert max_abs(O0, ref) <= TOL["bf16"] and max_abs(O1, ref) <= TOL["bf16"]


@pytest.mark.parametrize("B,N,Hq,Hkv,G,d,W,A,dtype", [
    (1, 900, 8, 2, 2, 128, 128, 256, "bf16"),
    (2, 600, 4, 4, 1, 64, 100, 70, "bf16"),
    (1, 400, 4, 2, 1, 128, 60, 100, "f32"),
])
def test_prefill_anchored_both_branch(B, N, Hq, Hkv, G, d, W, A, dtype):
    say(f"anchored both-branch B={B} N={N} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} A={A} {dtype}")
    Q, K, V = _qkv(43 + N, B, N, Hq, Hkv, d, dtype)
    rng = np.random.default_rng(44)
    gate = np.stack([synth.structured_gate(rng, N, 0.3, 16, 64) for _ in range(B * G)], -1)
    gate = gate.reshape(N, B, G).transpose(1, 0, 2).copy()
    O, diff = _gpu(Q, K, V, gate, W, A, dtype, both=True)
    ref = oracle.prefill(Q, K, V, gate, W, both_branch=True, anchors=A)
    err = max_abs(O, ref["O"])
    derr = np.abs(diff - ref["diff"])
    tol = diff_tolerance(ref["diff"], Hq * d, TOL[dtype])
    say(f"  O max-abs {err:.3e}; diff max-abs {derr.max():.3e}")
    assert err <= TOL[dtype]
    assert np.all(derr <= tol)
    # rows i < W + A see [0, i] in both branches: distance exactly 0
    assert np.all(diff[:, : W + A] == 0.0)


def test_prefill_anchored_deterministic_and_zero_anchors_match_plain():
    B, N, Hq, Hkv, G, d, W = 1, 3000, 8, 2, 1, 128, 500
    Q, K, V = _qkv(45, B, N, Hq, Hkv, d, "bf16")
    gate = (np.random.default_rng(46).random((B, N, G)) < 0.2).astype(np.uint8)
    bf = torch.bfloat16
    Qg, Kg, Vg, gg = dev(Q, bf), dev(K, bf), dev(V, bf), dev(gate)
    a1, _ = swa().prefill(Qg, Kg, Vg, gg, W, anchors=256)
    a2, _ = swa().prefill(Qg, Kg, Vg, gg, W, anchors=256)
    p0, _ = swa().prefill(Qg, Kg, Vg, gg, W)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2), "two anchored runs differ"
    # rows that see no anchors (i < W) are the plain window rows, bit for bit
    assert torch.equal(a1[:, :W], p0[:, :W])


# ---------------------------------------------------------------- decode
DECODE_ANCHOR_CASES = [
    # B, Lmax, Hq, Hkv, G, d, W, A, lens, dtype
    (5, 700, 8, 2, 2, 128, 100, 256, [700, 1, 99, 300, 357], "bf16"),
    (3, 513, 8, 1, 4, 128, 64, 100, [513, 200, 64], "bf16"),   # window and full heads in one KV pair
    (4, 300, 4, 4, 1, 64, 50, 30, [300, 3, 81, 257], "bf16"),
    (2, 260, 2, 1, 1, 128, 40, 77, [260, 117], "f32"),
    # 400 ragged pairs, several shares per pair
    (100, 2048, 8, 4, 2, 64, 300, 256, [int(x) for x in np.random.default_rng(47).integers(1, 2049, 100)],
     "bf16"),
]


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,G,d,W,A,lens,dtype", DECODE_ANCHOR_CASES)
def test_decode_anchored(B, Lmax, Hq, Hkv, G, d, W, A, lens, dtype):
    say(f"anchored decode B={B} Lmax={Lmax} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} A={A} {dtype}")
    rng = np.random.default_rng(Lmax + A)
    mk = (lambda s: synth.round_bf16(rng.standard_normal(s, dtype=np.float32))) if dtype == "bf16" \
        else (lambda s: rng.standard_normal(s, dtype=np.float32))
    q, Kc, Vc = mk((B, Hq, d)), mk((B, Lmax, Hkv, d)), mk((B, Lmax, Hkv, d))
    gate = (rng.random((B, G)) < 0.5).astype(np.uint8)
    gate[0, :] = 0
    lens = np.array(lens, np.int32)
    td = TORCH_DTYPE[dtype]
    o = swa().decode(dev(q, td), dev(Kc, td), dev(Vc, td), dev(lens), dev(gate), W, anchors=A)
    torch.cuda.synchronize()
    ref = oracle.decode(q, Kc, Vc, lens, gate, W, anchors=A)["o"]
    err = max_abs(host(o), ref)
    say(f"  max-abs {err:.3e}")
    assert err <= TOL[dtype]


def test_decode_anchored_matches_prefill_last_row():
    B, N, Hq, Hkv, G, d, W, A = 1, 1500, 8, 2, 1, 128, 300, 256
    Q, K, V = _qkv(48, B, N, Hq, Hkv, d, "bf16")
    gate = np.zeros((B, N, G), np.uint8)
    O, _ = _gpu(Q, K, V, gate, W, A, "bf16")
    bf = torch.bfloat16
    o = swa().decode(dev(Q[:, -1], bf), dev(K, bf), dev(V, bf), dev(np.array([N], np.int32)),
                     dev(gate[:, -1]), W, anchors=A)
    torch.cuda.synchronize()
    assert max_abs(host(o), O[:, -1]) <= 2 * TOL["bf16"]
    ref = oracle.decode(Q[:, -1], K, V, np.array([N]), gate[:, -1], W, anchors=A)["o"]
    assert max_abs(host(o), ref) <= TOL["bf16"]


# ---------------------------------------------------------------- full size
N32K, W1K, A256 = 32768, 1024, 256


def test_long_prefill_32k_anchored():
    say("anchored long prefill N=32768 GQA 16/4 W=1024 A=256 gate Bernoulli(0.13)")
    w = synth.long_prefill(seed=3)
    bf = torch.bfloat16
    Q, K, V = dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf)
    O, _ = swa().prefill(Q, K, V, dev(w.gate), W1K, anchors=A256)
    O2, _ = swa().prefill(Q, K, V, dev(w.gate), W1K, anchors=A256)
    torch.cuda.synchronize()
    assert torch.equal(O, O2), "two runs differ"
    Oh = host(O)
    assert np.all(np.abs(Oh) <= np.abs(w.V).max() + 1e-2)
    rng = np.random.default_rng(49)
    routed = np.flatnonzero(w.gate[0, :, 0])
    plain = np.flatnonzero(w.gate[0, :, 0] == 0)
    rows = set(range(0, 32)) | set(range(W1K - 16, W1K + 16)) | set(range(W1K + A256 - 16, W1K + A256 + 16))
    rows |= set(range(N32K - 16, N32K))
    rows |= set(rng.choice(routed, 64, replace=False).tolist()) | set(rng.choice(plain, 64, replace=False).tolist())
    rows = np.array(sorted(rows))
    ref = oracle.prefill(np.asarray(w.Q, np.float64), np.asarray(w.K, np.float64),
                         np.asarray(w.V, np.float64), w.gate, W1K, rows=rows, anchors=A256)["O"]
    err = max_abs(Oh[:, rows], ref)
    say(f"  {rows.size} sampled rows x 16 heads: max-abs {err:.3e}")
    assert err <= TOL["bf16"]


def test_decode_64x32k_anchored():
    say("anchored decode: 64 sequences x 32768 cache, GQA 16/4, W=1024, A=256, gate Bernoulli(0.13)")
    d = synth.decode_cache(seed=5, device="cuda")
    lens = dev(d["cache_len"])
    gate = dev(d["gate"])
    o = swa().decode(d["q"], d["Kc"], d["Vc"], lens, gate, W1K, anchors=A256)
    o2 = swa().decode(d["q"], d["Kc"], d["Vc"], lens, gate, W1K, anchors=A256)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "two runs differ"
    oh = host(o)
    qh = host(d["q"])
    errs = []
    for b in range(d["q"].shape[0]):
        L = int(d["cache_len"][b])
        full = bool(d["gate"][b, 0])
        # the keys this sequence reads: all L, or the anchors and the last W
        keep = np.arange(L) if full else np.union1d(np.arange(min(A256, max(0, L - W1K))),
                                                   np.arange(max(0, L - W1K), L))
        Kb = host(d["Kc"][b:b + 1, :L])[:, keep]
        Vb = host(d["Vc"][b:b + 1, :L])[:, keep]
        # on the gathered keys the set is [0, n-1]: full attention over them
        ref = oracle.decode(qh[b:b + 1], Kb, Vb, np.array([keep.size]), np.ones((1, 1), np.uint8), W1K)["o"]
        errs.append(max_abs(oh[b:b + 1], ref))
    say(f"  full sequences {int(d['gate'].sum())}; max-abs over all 64 sequences {max(errs):.3e}")
    assert max(errs) <= TOL["bf16"]
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_step_anchored(dtype):
    """Serving step with anchors: route the new tokens, append their K/V at
    each sequence's length (empty, short, long and full caches), decode
    with the first A keys in every window head's key set."""
    B, Lmax, Hq, Hkv, G, d, W, A, hidden = 6, 700, 8, 2, 2, 128, 100, 256, 128
    rng = np.random.default_rng(71)
    rnd = (lambda *sh: synth.round_bf16(rng.standard_normal(sh, dtype=np.float32))) if dtype == "bf16" \
        else (lambda *sh: rng.standard_normal(sh, dtype=np.float32))
    Kc, Vc = rnd(B, Lmax, Hkv, d), rnd(B, Lmax, Hkv, d)
    q, k, v = rnd(B, Hq, d), rnd(B, Hkv, d), rnd(B, Hkv, d)
    Hn = rnd(B, hidden)
    r = (rnd(hidden, G) / np.sqrt(hidden)).astype(np.float32)
    if dtype == "bf16":
        r = synth.round_bf16(r)
    bias = np.array([-0.3, 0.2], np.float32)
    L0 = np.array([0, 5, 300, 457, 699, 700], np.int32)
    td = TORCH_DTYPE[dtype]
    Kg, Vg, Lg = dev(Kc, td), dev(Vc, td), dev(L0)
    o, gate = swa().decode_step(dev(Hn, td), dev(r, td), dev(bias), dev(q, td), dev(k, td), dev(v, td),
                                Kg, Vg, Lg, W, anchors=A)
    torch.cuda.synchronize()
    ref = oracle.decode_step(Hn, r, bias, q, k, v, Kc, Vc, L0, W, anchors=A)
    near = np.abs(ref["z"]) < 1e-5
    g = gate.cpu().numpy()
    assert np.array_equal(g[~near], ref["gate"][~near])
    assert np.array_equal(Lg.cpu().numpy(), ref["cache_len"])
    ok = ~near.any(axis=1)
    err = max_abs(host(o)[ok], ref["o"][ok])
    say(f"anchored decode step {dtype}: o max-abs {err:.3e}, gates {g.tolist()}")
    assert err <= TOL[dtype]

"""GPU parity of the HIP library against the float64 CPU reference.

Every test calls the C ABI through the thin binding, on seeded inputs that
are fed unchanged (same stored bf16/fp32 values) to the reference."""
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


def swa():
    import sliding_window_attention_router_amd as m

    return m


def _qkv(seed, B, N, Hq, Hkv, d, dtype):
    rng = np.random.default_rng(seed)
    mk = (lambda s: synth.round_bf16(rng.standard_normal(s, dtype=np.float32))) if dtype == "bf16" \
        else (lambda s: rng.standard_normal(s, dtype=np.float32))
    return mk((B, N, Hq, d)), mk((B, N, Hkv, d)), mk((B, N, Hkv, d))


def _gpu_prefill(Q, K, V, gate, W, dtype, both=False):
    td = TORCH_DTYPE[dtype]
    O, diff = swa().prefill(dev(Q, td), dev(K, td), dev(V, td), dev(gate), W, both_branch=both)
    torch.cuda.synchronize()
    return host(O), (host(diff) if diff is not None else None)


# ---------------------------------------------------------------- router
def test_route_layer_bf16():
    w = synth.layer()
    say(f"route layer: H {w.H.shape}")
    gate, idx, cnt, z = swa().route(dev(w.H, torch.bfloat16), dev(w.r, torch.bfloat16),
                                     dev(w.bias), want_z=True)
    torch.cuda.synchronize()
    ref = oracle.route(w.H, w.r, w.bias)
    g_gpu = gate.cpu().numpy()
    far = ~ref["near"]
    assert np.array_equal(g_gpu[far], ref["gate"][far])
    assert max_abs(host(z), ref["z"]) < 1e-3
    idx_ref, cnt_ref = oracle.compact(g_gpu)
    c = cnt.cpu().numpy()
    assert np.array_equal(c, cnt_ref)
    ih = idx.cpu().numpy()
    for b in range(ih.shape[0]):
        for g in range(ih.shape[1]):
            assert np.array_equal(ih[b, g, : c[b, g]], idx_ref[b, g, : c[b, g]])
    dens = g_gpu.mean()
    say(f"route layer: density {dens:.4f}, near-threshold tokens {int(ref['near'].sum())}")
    assert 0.09 < dens < 0.17


def test_route_f32_groups_unaligned_hidden():
    rng = np.random.default_rng(21)
    H = rng.standard_normal((2, 777, 100), dtype=np.float32)
    r = (rng.standard_normal((100, 3), dtype=np.float32) * 0.1).astype(np.float32)
    bias = np.array([0.0, -0.3, 0.4], np.float32)
    gate, idx, cnt, z = swa().route(dev(H), dev(r), dev(bias), want_z=True)
    torch.cuda.synchronize()
    ref = oracle.route(H, r, bias)
    far = ~ref["near"]
    assert np.array_equal(gate.cpu().numpy()[far], ref["gate"][far])
    assert max_abs(host(z), ref["z"]) < 1e-4


@pytest.mark.parametrize("B,N,G,p", [(2, 1000, 3, 0.2), (1, 1, 1, 1.0), (1, 31, 2, 0.0),
                                     (3, 33, 1, 1.0), (1, 32768, 1, 0.13), (1, 40000, 2, 0.5)])
def test_compaction_given_gate(B, N, G, p):
    rng = np.random.default_rng(N + G)
    gate = (rng.random((B, N, G)) < p).astype(np.uint8)
    _, idx, cnt, _ = swa().route(None, gate=dev(gate))
    torch.cuda.synchronize()
    idx_ref, cnt_ref = oracle.compact(gate)
    c = cnt.cpu().numpy()
    assert np.array_equal(c, cnt_ref)
    ih = idx.cpu().numpy()
    for b in range(B):
        for g in range(G):
            assert np.array_equal(ih[b, g, : c[b, g]], idx_ref[b, g, : c[b, g]])


# ---------------------------------------------------------------- prefill
@pytest.mark.parametrize("G", [2, 1])
def test_prefill_tiny_f32(G):
    w = synth.tiny(G=G)
    O, _ = _gpu_prefill(w.Q, w.K, w.V, w.gate, w.W, "f32")
    ref = oracle.prefill(w.Q, w.K, w.V, w.gate, w.W)["O"]
    err = max_abs(O, ref)
    say(f"tiny f32 G={G}: max-abs {err:.3e}")
    assert err <= TOL["f32"]


PREFILL_CASES = [
    # B, N,   Hq, Hkv, G, d,  W,   p,   dtype
    (1, 1000, 8, 2, 1, 128, 200, 0.2, "bf16"),   # GQA 4:1, ragged tail
    (2, 777, 4, 4, 2, 64, 100, 0.3, "bf16"),     # MHA, two gate groups, d=64
    (1, 530, 8, 1, 4, 128, 64, 0.5, "bf16"),     # gate groups inside one KV group
    (1, 300, 2, 2, 2, 128, 512, 0.5, "bf16"),    # W > N
    (1, 129, 4, 2, 1, 128, 64, 0.5, "bf16"),     # N just past a tile
    (1, 5, 2, 1, 1, 64, 3, 0.5, "bf16"),         # N smaller than a block
    (1, 400, 4, 2, 2, 128, 70, 0.4, "f32"),      # fp32 path, GQA
    (1, 2100, 16, 4, 1, 64, 256, 0.2, "bf16"),   # d=64 GQA 4:1, many window blocks and far chunks
    (2, 1500, 8, 2, 1, 128, 300, 0.3, "bf16"),   # two sequences: per-sequence K/V copy offsets
]


@pytest.mark.parametrize("B,N,Hq,Hkv,G,d,W,p,dtype", PREFILL_CASES)
def test_prefill_hard_gate(B, N, Hq, Hkv, G, d, W, p, dtype):
    say(f"prefill case B={B} N={N} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} p={p} {dtype}")
    Q, K, V = _qkv(N * 7 + d, B, N, Hq, Hkv, d, dtype)
    gate = (np.random.default_rng(N).random((B, N, G)) < p).astype(np.uint8)
    O, _ = _gpu_prefill(Q, K, V, gate, W, dtype)
    ref = oracle.prefill(Q, K, V, gate, W)["O"]
    err = max_abs(O, ref)
    say(f"  max-abs {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("mode", ["zeros", "ones"])
def test_prefill_gate_bounds(mode):
    B, N, Hq, Hkv, G, d, W = 1, 700, 8, 2, 1, 128, 128
    Q, K, V = _qkv(3, B, N, Hq, Hkv, d, "bf16")
    gate = np.full((B, N, G), 1 if mode == "ones" else 0, np.uint8)
    O, _ = _gpu_prefill(Q, K, V, gate, W, "bf16")
    ref = oracle.prefill(Q, K, V, gate, W)["O"]
    err = max_abs(O, ref)
    say(f"gate all-{mode}: max-abs {err:.3e}")
    assert err <= TOL["bf16"]


def test_prefill_window_one_is_v_exactly():
    B, N, Hq, Hkv, G, d = 1, 300, 4, 2, 1, 128
    Q, K, V = _qkv(4, B, N, Hq, Hkv, d, "bf16")
    gate = np.zeros((B, N, G), np.uint8)
    O, _ = _gpu_prefill(Q, K, V, gate, 1, "bf16")
    for h in range(Hq):
        assert np.array_equal(O[:, :, h], V[:, :, h // 2].astype(np.float64))


def test_prefill_window_covering_sequence_is_gate_independent():
    B, N, Hq, Hkv, G, d = 1, 250, 4, 1, 1, 128
    Q, K, V = _qkv(5, B, N, Hq, Hkv, d, "bf16")
    g0 = np.zeros((B, N, G), np.uint8)
    g1 = np.ones((B, N, G), np.uint8)
    O0, _ = _gpu_prefill(Q, K, V, g0, N, "bf16")
    O1, _ = _gpu_prefill(Q, K, V, g1, N, "bf16")
    assert max_abs(O0, O1) <= 2 * TOL["bf16"] and max_abs(O0, oracle.prefill(Q, K, V, g0, N)["O"]) <= TOL["bf16"]


@pytest.mark.parametrize("Hq,Hkv,G,W", [(4, 4, 1, 128), (8, 2, 2, 100)])
def test_prefill_both_branch(Hq, Hkv, G, W):
    B, N, d = 1, 600, 128
    Q, K, V = _qkv(6, B, N, Hq, Hkv, d, "bf16")
    rng = np.random.default_rng(7)
    gate = np.stack([synth.structured_gate(rng, N, 0.3, 16, 64) for _ in range(G)], -1)[None]
    O, diff = _gpu_prefill(Q, K, V, gate, W, "bf16", both=True)
    ref = oracle.prefill(Q, K, V, gate, W, both_branch=True)
    err = max_abs(O, ref["O"])
    derr = np.abs(diff - ref["diff"])
    tol = diff_tolerance(ref["diff"], Hq * d, TOL["bf16"])
    say(f"both-branch: O max-abs {err:.3e}; diff max-abs {derr.max():.3e} "
        f"(max rel {np.max(derr / np.maximum(ref['diff'], 1e-30)):.3e})")
    assert err <= TOL["bf16"]
    assert np.all(derr <= tol)
    assert np.all(diff[:, :W] == 0.0)  # identical key sets before the window fills


BOTH_CASES = [
    # B, N, Hq, Hkv, G, d, W, dtype
    (2, 300, 4, 2, 2, 64, 50, "f32"),      # float32 path; window output stored exactly
    (2, 700, 8, 1, 4, 64, 64, "bf16"),     # gate groups inside a KV group (2 heads per unit)
    (1, 600, 4, 2, 1, 128, 1000, "bf16"),  # W > N: no row has far keys, diff all 0
    (1, 1000, 8, 4, 2, 128, 333, "bf16"),  # ragged N and W
]


@pytest.mark.parametrize("B,N,Hq,Hkv,G,d,W,dtype", BOTH_CASES)
def test_prefill_both_branch_shapes(B, N, Hq, Hkv, G, d, W, dtype):
    Q, K, V = _qkv(13, B, N, Hq, Hkv, d, dtype)
    gate = (np.random.default_rng(14).random((B, N, G)) < 0.3).astype(np.uint8)
    O, diff = _gpu_prefill(Q, K, V, gate, W, dtype, both=True)
    ref = oracle.prefill(Q, K, V, gate, W, both_branch=True)
    err = max_abs(O, ref["O"])
    derr = np.abs(diff - ref["diff"])
    tol = diff_tolerance(ref["diff"], Hq * d, TOL[dtype])
    say(f"both-branch {dtype} B={B} N={N} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W}: O max-abs {err:.3e}; "
        f"diff max-abs {derr.max():.3e}")
    assert err <= TOL[dtype]
    assert np.all(derr <= tol)
    assert np.all(diff[:, :min(W, N)] == 0.0)


@pytest.mark.parametrize("N,W", [(1, 1), (2, 1), (65, 64), (64, 64)])
def test_prefill_both_branch_degenerate(N, W):
    """Single tokens, a window of one key (row i's far part is [0, i-1]), and
    a sequence that is one key longer than the window."""
    B, Hq, Hkv, G, d = 1, 4, 2, 2, 64
    Q, K, V = _qkv(17, B, N, Hq, Hkv, d, "bf16")
    gate = (np.arange(N * G).reshape(1, N, G) % 3 == 0).astype(np.uint8)
    O, diff = _gpu_prefill(Q, K, V, gate, W, "bf16", both=True)
    ref = oracle.prefill(Q, K, V, gate, W, both_branch=True)
    assert max_abs(O, ref["O"]) <= TOL["bf16"]
    assert np.all(np.abs(diff - ref["diff"]) <= diff_tolerance(ref["diff"], Hq * d, TOL["bf16"]))
    assert np.all(diff[:, :min(W, N)] == 0.0)
    if N > W:
        assert np.all(diff[:, W:] > 0.0)  # the far keys change the full-branch output


def test_decode_step_one_slot_cache():
    """Lmax = 1: the first token fills the cache, a second step finds it full."""
    B, Lmax, Hq, Hkv, G, d, W, hidden = 2, 1, 4, 2, 1, 128, 1, 64
    rng = np.random.default_rng(61)
    rnd = lambda *sh: synth.round_bf16(rng.standard_normal(sh, dtype=np.float32))
    Kc, Vc = np.zeros((B, Lmax, Hkv, d), np.float32), np.zeros((B, Lmax, Hkv, d), np.float32)
    q, k, v, Hn = rnd(B, Hq, d), rnd(B, Hkv, d), rnd(B, Hkv, d), rnd(B, hidden)
    r = synth.round_bf16(rnd(hidden, G) / 8.0)
    bias = np.zeros(G, np.float32)
    bf = torch.bfloat16
    Kg, Vg, Lg = dev(Kc, bf), dev(Vc, bf), dev(np.zeros(B, np.int32))
    o, _ = swa().decode_step(dev(Hn, bf), dev(r, bf), dev(bias), dev(q, bf), dev(k, bf), dev(v, bf),
                             Kg, Vg, Lg, W)
    ref = oracle.decode_step(Hn, r, bias, q, k, v, Kc, Vc, np.zeros(B, np.int32), W)
    assert np.array_equal(Lg.cpu().numpy(), [1, 1])
    assert max_abs(host(o), ref["o"]) <= TOL["bf16"]
    # the cache is full now: nothing is appended, the output is the decode over it
    k2, v2 = rnd(B, Hkv, d), rnd(B, Hkv, d)
    o2, _ = swa().decode_step(dev(Hn, bf), dev(r, bf), dev(bias), dev(q, bf), dev(k2, bf), dev(v2, bf),
                              Kg, Vg, Lg, W)
    assert np.array_equal(Lg.cpu().numpy(), [1, 1])
    assert np.array_equal(host(Kg), ref["Kc"]) and np.array_equal(host(Vg), ref["Vc"])
    assert max_abs(host(o2), ref["o"]) <= TOL["bf16"]


def test_prefill_both_branch_deterministic():
    B, N, Hq, Hkv, G, d, W = 1, 900, 8, 2, 1, 128, 128
    Q, K, V = _qkv(15, B, N, Hq, Hkv, d, "bf16")
    gate = (np.random.default_rng(16).random((B, N, G)) < 0.2).astype(np.uint8)
    a, da = _gpu_prefill(Q, K, V, gate, W, "bf16", both=True)
    b, db = _gpu_prefill(Q, K, V, gate, W, "bf16", both=True)
    assert np.array_equal(a, b) and np.array_equal(da, db)


# ---------------------------------------------------------------- regulariser
@pytest.mark.parametrize("B,N,G", [(2, 1000, 3), (1, 1, 1), (1, 32768, 1), (3, 777, 2)])
def test_regularizer(B, N, G):
    rng = np.random.default_rng(31 + N)
    z = rng.normal(0.0, 4.0, (B, N, G)).astype(np.float32)
    z.reshape(-1)[:6] = [0.0, 800.0, -800.0, 50.0, -50.0, -100.0][: z.size]
    nll = rng.uniform(0.0, 8.0, (B, N)).astype(np.float32)
    diff = (rng.random((B, N)) < 0.5) * rng.exponential(0.05, (B, N))
    diff = diff.astype(np.float32)
    loss = host(swa().regularizer(dev(z), dev(nll), dev(diff)))
    ref = oracle.regularizer(z, nll, diff)
    err = np.abs(loss - ref)
    say(f"regularizer B={B} N={N} G={G}: max rel {np.max(err / np.maximum(ref, 1e-30)):.2e}")
    # float32: a few roundings of the weight and of softplus; denormal
    # softplus values (z below about -87) keep an absolute bound
    assert np.all(err <= 2e-6 * ref + 1e-40)
    # other hyperparameters are passed through
    loss2 = host(swa().regularizer(dev(z), dev(nll), dev(diff), gamma_base=2e-3, eps=0.5, alpha=10.0))
    ref2 = oracle.regularizer(z, nll, diff, gamma_base=2e-3, eps=0.5, alpha=10.0)
    assert np.all(np.abs(loss2 - ref2) <= 2e-6 * ref2 + 1e-40)


def test_regularizer_after_both_branch_layer():
    """Router logits -> both-branch prefill distance -> regulariser, against
    the same chain in the oracle (synthetic NLL)."""
    B, N, Hq, Hkv, G, d, W, hidden = 1, 1500, 8, 2, 1, 64, 200, 256
    w = synth.long_prefill(seed=33, B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, W=W, p=0.3, G=G, with_router=True,
                           hidden=hidden)
    bf = torch.bfloat16
    gate, idx, cnt, z = swa().route(dev(w.H, bf), dev(w.r, bf), dev(w.bias), want_z=True)
    O, diff = swa().prefill(dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), gate, W, both_branch=True)
    nll = np.random.default_rng(34).uniform(0.0, 6.0, (B, N)).astype(np.float32)
    loss = host(swa().regularizer(z, dev(nll), diff))
    # the oracle chain runs on its own router output (the distance does not
    # depend on the gate)
    rz = oracle.route(w.H, w.r, w.bias)
    rp = oracle.prefill(w.Q, w.K, w.V, rz["gate"], W, both_branch=True)
    ref = oracle.regularizer(rz["z"], nll, rp["diff"])
    # the distance is within diff_tolerance of the oracle's, so the weight's
    # relative error is at most alpha * tol / (eps + NLL + alpha * diff); the
    # logits are within 1e-3 (float32 accumulation), and softplus changes by
    # at most that much relatively (d log softplus(z) / dz = sigmoid(z) /
    # softplus(z) <= 1)
    tol_d = diff_tolerance(rp["diff"], Hq * d, TOL["bf16"])
    den = 0.1 + nll + 100.0 * rp["diff"]
    # rows before the window fills have distance exactly 0 on both sides
    tol_d[:, :W] = 0.0
    assert np.all(host(diff)[:, :W] == 0.0)
    rel = (100.0 * tol_d / den)[..., None] + 2e-3
    err = np.abs(loss - ref)
    say(f"regulariser after both-branch: max rel {np.max(err / ref):.2e} (bound {rel.max():.2e})")
    assert np.all(err <= rel * ref + 1e-30)


def test_prefill_deterministic():
    B, N, Hq, Hkv, G, d, W = 1, 900, 8, 2, 1, 128, 128
    Q, K, V = _qkv(8, B, N, Hq, Hkv, d, "bf16")
    gate = (np.random.default_rng(9).random((B, N, G)) < 0.2).astype(np.uint8)
    a, _ = _gpu_prefill(Q, K, V, gate, W, "bf16")
    b, _ = _gpu_prefill(Q, K, V, gate, W, "bf16")
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- decode
DECODE_CASES = [
    # B, Lmax, Hq, Hkv, G, d, W, lens, dtype
    (5, 700, 8, 2, 2, 128, 100, [700, 1, 99, 100, 350], "bf16"),
    (3, 513, 8, 1, 4, 128, 64, [513, 200, 64], "bf16"),   # gate groups inside a KV group
    (4, 300, 4, 4, 1, 64, 50, [300, 3, 51, 257], "bf16"),
    (2, 260, 2, 1, 1, 128, 40, [260, 17], "f32"),
    # more blocks' worth of workgroups than blocks: some key-block shares are empty
    (40, 200, 4, 2, 1, 128, 32, [int(x) for x in np.random.default_rng(11).integers(1, 61, 40)], "bf16"),
    # 400 (sequence, KV head) pairs, ragged: pairs cut across several shares
    (100, 2048, 8, 4, 2, 64, 300, [int(x) for x in np.random.default_rng(12).integers(1, 2049, 100)], "bf16"),
    # fewer blocks than workgroups and a full 4096-key sequence: its pairs are
    # cut into 64 one-block pieces each, more than one merge batch
    (2, 4096, 4, 2, 1, 128, 256, [4096, 3000], "bf16"),
    (1, 2600, 2, 1, 1, 64, 100, [2600], "f32"),
]


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,G,d,W,lens,dtype", DECODE_CASES)
def test_decode(B, Lmax, Hq, Hkv, G, d, W, lens, dtype):
    say(f"decode case B={B} Lmax={Lmax} Hq={Hq} Hkv={Hkv} G={G} d={d} W={W} {dtype}")
    rng = np.random.default_rng(Lmax)
    mk = (lambda s: synth.round_bf16(rng.standard_normal(s, dtype=np.float32))) if dtype == "bf16" \
        else (lambda s: rng.standard_normal(s, dtype=np.float32))
    q, Kc, Vc = mk((B, Hq, d)), mk((B, Lmax, Hkv, d)), mk((B, Lmax, Hkv, d))
    gate = (rng.random((B, G)) < 0.5).astype(np.uint8)
    gate[0, :] = 1
    lens = np.array(lens, np.int32)
    td = TORCH_DTYPE[dtype]
    o = swa().decode(dev(q, td), dev(Kc, td), dev(Vc, td), dev(lens), dev(gate), W)
    torch.cuda.synchronize()
    ref = oracle.decode(q, Kc, Vc, lens, gate, W)["o"]
    err = max_abs(host(o), ref)
    say(f"  max-abs {err:.3e}")
    assert err <= TOL[dtype]


STEP_CASES = [
    # B, Lmax, Hq, Hkv, G, d, W, hidden, lens (before the step), dtype
    (6, 300, 8, 2, 2, 128, 64, 128, [0, 1, 150, 299, 300, 64], "bf16"),
    (3, 200, 4, 4, 1, 64, 30, 96, [199, 17, 0], "f32"),
]


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,G,d,W,hidden,lens,dtype", STEP_CASES)
def test_decode_step(B, Lmax, Hq, Hkv, G, d, W, hidden, lens, dtype):
    rng = np.random.default_rng(51 + B)
    rnd = (lambda *sh: synth.round_bf16(rng.standard_normal(sh, dtype=np.float32))) if dtype == "bf16" \
        else (lambda *sh: rng.standard_normal(sh, dtype=np.float32))
    Kc, Vc = rnd(B, Lmax, Hkv, d), rnd(B, Lmax, Hkv, d)
    q, k, v = rnd(B, Hq, d), rnd(B, Hkv, d), rnd(B, Hkv, d)
    Hn = rnd(B, hidden)
    r = (rnd(hidden, G) / np.sqrt(hidden)).astype(np.float32)
    if dtype == "bf16":
        r = synth.round_bf16(r)
    bias = np.zeros(G, np.float32)
    L0 = np.array(lens, np.int32)
    td = TORCH_DTYPE[dtype]
    Kg, Vg, Lg = dev(Kc, td), dev(Vc, td), dev(L0)
    o, gate = swa().decode_step(dev(Hn, td), dev(r, td), dev(bias), dev(q, td), dev(k, td), dev(v, td),
                                Kg, Vg, Lg, W)
    ref = oracle.decode_step(Hn, r, bias, q, k, v, Kc, Vc, L0, W)
    near = np.abs(ref["z"]) < 1e-5
    g = gate.cpu().numpy()
    assert np.array_equal(g[~near], ref["gate"][~near])
    assert np.array_equal(Lg.cpu().numpy(), ref["cache_len"])
    assert np.array_equal(host(Kg), ref["Kc"]) and np.array_equal(host(Vg), ref["Vc"])
    ok = ~near.any(axis=1)
    err = max_abs(host(o)[ok], ref["o"][ok])
    say(f"decode step {dtype} B={B} lens={lens}: o max-abs {err:.3e}, near-threshold sequences {int((~ok).sum())}")
    assert err <= TOL[dtype]


def test_decode_step_serves_a_sequence():
    """Token-by-token serving from an empty cache reproduces the prefill rows
    of the whole sequence (gates from the router on each token)."""
    B, N, Hq, Hkv, G, d, W, hidden = 3, 80, 8, 2, 1, 128, 24, 64
    w = synth.long_prefill(seed=52, B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, W=W, p=0.3, G=G, with_router=True,
                           hidden=hidden)
    rz = oracle.route(w.H, w.r, w.bias)
    assert not rz["near"].any()  # no token within 1e-5 of the threshold for this seed
    ref = oracle.prefill(w.Q, w.K, w.V, rz["gate"], W)["O"]
    bf = torch.bfloat16
    Kc = torch.zeros((B, N, Hkv, d), dtype=bf, device="cuda")
    Vc = torch.zeros_like(Kc)
    L = torch.zeros(B, dtype=torch.int32, device="cuda")
    H, Q, K, V = dev(w.H, bf), dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf)
    r, bias = dev(w.r, bf), dev(w.bias)
    outs, gates = [], []
    for t in range(N):
        o, g = swa().decode_step(H[:, t].contiguous(), r, bias, Q[:, t].contiguous(), K[:, t].contiguous(),
                                 V[:, t].contiguous(), Kc, Vc, L, W)
        outs.append(host(o))
        gates.append(g.cpu().numpy())
    O = np.stack(outs, 1)
    assert np.array_equal(np.stack(gates, 1), rz["gate"])
    assert np.array_equal(L.cpu().numpy(), np.full(B, N))
    assert np.array_equal(host(Kc), w.K) and np.array_equal(host(Vc), w.V)
    err = max_abs(O, ref)
    say(f"served {N} tokens x {B} sequences: max-abs vs prefill rows {err:.3e}")
    assert err <= TOL["bf16"]


def test_decode_matches_prefill_last_row():
    B, N, Hq, Hkv, G, d, W = 1, 640, 8, 2, 1, 128, 96
    Q, K, V = _qkv(10, B, N, Hq, Hkv, d, "bf16")
    for g in (0, 1):
        gate = np.full((B, N, G), g, np.uint8)
        O, _ = _gpu_prefill(Q, K, V, gate, W, "bf16")
        o = swa().decode(dev(Q[:, -1], torch.bfloat16), dev(K, torch.bfloat16), dev(V, torch.bfloat16),
                         dev(np.array([N], np.int32)), dev(gate[:, -1]), W)
        torch.cuda.synchronize()
        assert max_abs(host(o), O[:, -1]) <= 2 * TOL["bf16"]

"""Checks that pin the CPU reference to facts fixed by the pages and by
mathematics.  Each check raises AssertionError on a mismatch; the oracle pin
tests call them on the reference as written, and the mutation tests call them
on copies with a planted mistake to show that the mistake is caught.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle.swiattn_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_w4_table():
    rows = []
    with open(os.path.join(GOLDEN, "swa_mask_w4.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(c) for c in line])
    return np.array(rows, dtype=bool)


def check_w4_key_ranges():
    """The window key set of each of the 7 rows equals the printed table."""
    table = load_w4_table()
    for i in range(7):
        lo, hi = ref.swa_key_range(i, 4)
        got = np.array([lo <= j <= hi for j in range(7)])
        assert np.array_equal(got, table[i]), (i, got, table[i])


def check_w4_attention_weights():
    """With q = 0 every attended key gets the same weight, and V = identity
    makes the output row equal to the weight vector: the attended set and the
    normalisation both show up in the output of the full prefill path."""
    table = load_w4_table()
    N = 7
    Q = np.zeros((1, N, 1, N))
    K = np.random.default_rng(0).standard_normal((1, N, 1, N))
    V = np.eye(N)[None, :, None, :]
    out = ref.prefill(Q, K, V, np.zeros((1, N, 1), np.uint8), W=4)["O"][0, :, 0, :]
    expect = table / table.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-15)


def check_full_branch_causal():
    """Gate all ones with q = 0, V = identity gives the uniform lower triangle
    (the full branch sees every key up to and including itself)."""
    N = 9
    Q = np.zeros((1, N, 1, N))
    K = np.random.default_rng(1).standard_normal((1, N, 1, N))
    V = np.eye(N)[None, :, None, :]
    out = ref.prefill(Q, K, V, np.ones((1, N, 1), np.uint8), W=3)["O"][0, :, 0, :]
    tri = np.tril(np.ones((N, N)))
    np.testing.assert_allclose(out, tri / tri.sum(axis=1, keepdims=True), rtol=0, atol=1e-15)


def _rand_qkv(seed, B, N, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, N, Hq, d)), rng.standard_normal((B, N, Hkv, d)),
            rng.standard_normal((B, N, Hkv, d)))


def check_window_covering_all_equals_full():
    """W >= N: the window mask is the whole lower triangle, so both branches
    coincide and the output does not depend on the gate."""
    Q, K, V = _rand_qkv(2, 1, 40, 4, 2, 8)
    gate = (np.random.default_rng(3).random((1, 40, 2)) < 0.5).astype(np.uint8)
    for W in (40, 57):
        a = ref.prefill(Q, K, V, np.zeros_like(gate), W=W)["O"]
        b = ref.prefill(Q, K, V, np.ones_like(gate), W=W)["O"]
        c = ref.prefill(Q, K, V, gate, W=W, both_branch=True)
        assert np.array_equal(a, b)
        assert np.array_equal(a, c["O"])
        assert np.all(c["diff"] == 0.0)


def check_window_one_returns_v():
    """W = 1: each row attends only to itself, so the output is its own value
    row of the KV head the query head maps to."""
    Q, K, V = _rand_qkv(4, 2, 33, 4, 2, 8)
    out = ref.prefill(Q, K, V, np.zeros((2, 33, 1), np.uint8), W=1)["O"]
    for h in range(4):
        assert np.array_equal(out[:, :, h], V[:, :, h // 2])


def _torch_sdpa(Q, K, V, mask):
    """torch CPU scaled_dot_product_attention in float64 with a boolean mask
    [N,N] (True = attend); K/V heads are repeated for grouped queries."""
    Hq, Hkv = Q.shape[2], K.shape[2]
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)
    k = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    v = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask))
    return o.permute(0, 2, 1, 3).numpy()


def check_gate_extremes_against_sdpa():
    """Gate all ones = causal attention, all zeros = band attention, each
    against torch's own scaled_dot_product_attention in float64."""
    B, N, Hq, Hkv, d, W = 2, 96, 4, 2, 16, 20
    Q, K, V = _rand_qkv(5, B, N, Hq, Hkv, d)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    causal = j <= i
    band = causal & (j > i - W)
    ones = ref.prefill(Q, K, V, np.ones((B, N, 1), np.uint8), W=W)["O"]
    zeros = ref.prefill(Q, K, V, np.zeros((B, N, 1), np.uint8), W=W)["O"]
    np.testing.assert_allclose(ones, _torch_sdpa(Q, K, V, causal), rtol=0, atol=1e-12)
    np.testing.assert_allclose(zeros, _torch_sdpa(Q, K, V, band), rtol=0, atol=1e-12)
    # a mixed gate selects per token and per head group
    gate = (np.random.default_rng(6).random((B, N, 2)) < 0.4).astype(np.uint8)
    mixed = ref.prefill(Q, K, V, gate, W=W)["O"]
    full_ref, band_ref = _torch_sdpa(Q, K, V, causal), _torch_sdpa(Q, K, V, band)
    for h in range(Hq):
        sel = gate[:, :, h // 2].astype(bool)[..., None]
        np.testing.assert_allclose(mixed[:, :, h], np.where(sel, full_ref[:, :, h], band_ref[:, :, h]),
                                   rtol=0, atol=1e-12)


def check_rows_before_window_have_no_discrepancy():
    """Rows i < W see the same keys in both branches: discrepancy exactly 0;
    later rows differ."""
    Q, K, V = _rand_qkv(7, 1, 64, 2, 2, 8)
    out = ref.prefill(Q, K, V, np.zeros((1, 64, 1), np.uint8), W=16, both_branch=True)
    assert np.all(out["diff"][:, :16] == 0.0)
    assert np.all(out["diff"][:, 16:] > 0.0)


def check_decode_equals_last_prefill_row():
    """Decoding at cache length L reproduces prefill row L-1 of the same
    sequence (shared cache, same key sets); entries beyond L are ignored."""
    B, Lmax, Hq, Hkv, d, W = 3, 50, 4, 2, 8, 12
    Q, K, V = _rand_qkv(8, B, Lmax, Hq, Hkv, d)
    lens = np.array([50, 31, 5])
    gate = np.array([[1], [0], [0]], np.uint8)
    Kj, Vj = K.copy(), V.copy()
    for b in range(B):
        Kj[b, lens[b]:] = 1e3  # junk beyond the cache length
        Vj[b, lens[b]:] = -1e3
    q = np.stack([Q[b, lens[b] - 1] for b in range(B)])
    dec = ref.decode(q, Kj, Vj, lens, gate, W)["o"]
    for b in range(B):
        L = lens[b]
        g = np.broadcast_to(gate[b], (1, L, 1)).astype(np.uint8)
        pre = ref.prefill(Q[b:b + 1, :L], K[b:b + 1, :L], V[b:b + 1, :L], g, W)["O"][0, L - 1]
        np.testing.assert_allclose(dec[b], pre, rtol=0, atol=1e-13)


def brute_force(Q, K, V, gate, W, scale, A=0, o=0):
    """Independent pure-Python evaluation: explicit loops, math.exp.  The
    window branch's keys are chosen by a membership test at position
    p = i - o (o = the layer's window offset): j <= p, and either among the
    W newest up to p or among the first A of the sequence.  A row with no
    key gets output 0."""
    B, N, Hq, d = Q.shape
    Hkv, G = K.shape[2], gate.shape[2]
    Of = np.zeros(Q.shape)
    Os = np.zeros(Q.shape)
    for b in range(B):
        for h in range(Hq):
            kv = h * Hkv // Hq
            for i in range(N):
                for which, out in (("full", Of), ("swa", Os)):
                    p = i if which == "full" else i - o
                    keys = [j for j in range(N)
                            if j <= p and (which == "full" or p - j < W or j < A)]
                    if not keys:
                        out[b, i, h, :] = 0.0
                        continue
                    s = [scale * sum(Q[b, i, h, c] * K[b, j, kv, c] for c in range(d)) for j in keys]
                    mx = max(s)
                    w = [math.exp(x - mx) for x in s]
                    tot = sum(w)
                    for c in range(d):
                        out[b, i, h, c] = sum(wj * V[b, j, kv, c] for wj, j in zip(w, keys)) / tot
    sel = np.stack([gate[:, :, h * G // Hq] for h in range(Hq)], axis=2).astype(bool)[..., None]
    O = np.where(sel, Of, Os)
    diff = ((Of - Os) ** 2).sum(axis=(2, 3))
    return O, diff


def check_brute_force_tiny():
    B, N, Hq, Hkv, d, W = 1, 11, 4, 2, 3, 4
    Q, K, V = _rand_qkv(9, B, N, Hq, Hkv, d)
    gate = (np.random.default_rng(10).random((B, N, 2)) < 0.5).astype(np.uint8)
    scale = 0.7
    O_bf, diff_bf = brute_force(Q, K, V, gate, W, scale)
    out = ref.prefill(Q, K, V, gate, W, scale=scale, both_branch=True)
    np.testing.assert_allclose(out["O"], O_bf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["diff"], diff_bf, rtol=1e-12, atol=1e-14)
    # the default scale is 1/sqrt(d)
    dflt = ref.prefill(Q, K, V, gate, W)["O"]
    O_bf2, _ = brute_force(Q, K, V, gate, W, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(dflt, O_bf2, rtol=0, atol=1e-12)


def check_anchors_brute_force():
    """Global anchors ([Glossary] pitfall 1, fix 2): every query also sees the
    first A keys, each key once.  Against the membership-test brute force,
    for anchors inside, overlapping and beyond the window."""
    B, N, Hq, Hkv, d, W = 1, 13, 4, 2, 3, 4
    Q, K, V = _rand_qkv(31, B, N, Hq, Hkv, d)
    gate = (np.random.default_rng(32).random((B, N, 2)) < 0.5).astype(np.uint8)
    for A in (1, 3, 6, 20):
        O_bf, diff_bf = brute_force(Q, K, V, gate, W, 0.9, A=A)
        out = ref.prefill(Q, K, V, gate, W, scale=0.9, both_branch=True, anchors=A)
        np.testing.assert_allclose(out["O"], O_bf, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out["diff"], diff_bf, rtol=1e-12, atol=1e-14)
        hard = ref.prefill(Q, K, V, gate, W, scale=0.9, anchors=A)["O"]
        np.testing.assert_allclose(hard, O_bf, rtol=0, atol=1e-12)


def check_anchors_closed_form():
    """W = 1 with A anchors and q = 0: row i >= A averages the anchors and
    itself, (v_0 + ... + v_{A-1} + v_i) / (A + 1); row i < A averages
    v_0..v_i (its anchors end where its window starts)."""
    N, A = 10, 3
    Q = np.zeros((1, N, 1, N))
    K = np.random.default_rng(33).standard_normal((1, N, 1, N))
    V = np.eye(N)[None, :, None, :]
    out = ref.prefill(Q, K, V, np.zeros((1, N, 1), np.uint8), W=1, anchors=A)["O"][0, :, 0]
    expect = np.zeros((N, N))
    for i in range(N):
        if i >= A:
            expect[i, :A] = 1.0 / (A + 1)
            expect[i, i] = 1.0 / (A + 1)
        else:
            expect[i, : i + 1] = 1.0 / (i + 1)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-15)


def check_anchors_against_sdpa_and_cover():
    """Gate all zeros with anchors equals torch's float64 attention under the
    mask causal & (band | first A keys); W + A >= N turns the window branch
    into full causal attention (diff 0 everywhere); rows i < W + A have the
    full key set in both branches (diff exactly 0), later rows do not."""
    B, N, Hq, Hkv, d, W, A = 1, 80, 4, 2, 8, 16, 8
    Q, K, V = _rand_qkv(34, B, N, Hq, Hkv, d)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    mask = (j <= i) & ((j > i - W) | (j < A))
    zeros = ref.prefill(Q, K, V, np.zeros((B, N, 1), np.uint8), W=W, anchors=A)["O"]
    np.testing.assert_allclose(zeros, _torch_sdpa(Q, K, V, mask), rtol=0, atol=1e-12)
    out = ref.prefill(Q, K, V, np.zeros((B, N, 1), np.uint8), W=W, both_branch=True, anchors=A)
    assert np.all(out["diff"][:, : W + A] == 0.0)
    assert np.all(out["diff"][:, W + A:] > 0.0)
    cover = ref.prefill(Q, K, V, np.zeros((B, N, 1), np.uint8), W=50, both_branch=True, anchors=30)
    assert np.all(cover["diff"] == 0.0)
    np.testing.assert_allclose(cover["O"], _torch_sdpa(Q, K, V, j <= i), rtol=0, atol=1e-12)


def check_anchored_decode_equals_last_prefill_row():
    """Decode with anchors at cache length L reproduces anchored prefill row
    L-1 (the anchors are the first A entries of the same linear cache)."""
    B, Lmax, Hq, Hkv, d, W, A = 3, 60, 4, 2, 8, 12, 5
    Q, K, V = _rand_qkv(35, B, Lmax, Hq, Hkv, d)
    lens = np.array([60, 16, 7])
    gate = np.array([[0], [0], [1]], np.uint8)
    q = np.stack([Q[b, lens[b] - 1] for b in range(B)])
    dec = ref.decode(q, K, V, lens, gate, W, anchors=A)["o"]
    for b in range(B):
        L = lens[b]
        g = np.broadcast_to(gate[b], (1, L, 1)).astype(np.uint8)
        pre = ref.prefill(Q[b:b + 1, :L], K[b:b + 1, :L], V[b:b + 1, :L], g, W, anchors=A)["O"][0, L - 1]
        np.testing.assert_allclose(dec[b], pre, rtol=0, atol=1e-13)
    # a window sequence past W + A differs from its anchor-free decode
    plain = ref.decode(q, K, V, lens, gate, W)["o"]
    assert not np.allclose(dec[0], plain[0])


def load_offset_table():
    layers, offsets = [], None
    with open(os.path.join(GOLDEN, "window_offsets.txt"), encoding="utf-8") as f:
        for line in f:
            parts = line.split("#", 1)[0].split()
            if not parts:
                continue
            if parts[0] == "layers":
                layers.append((int(parts[1]), float(parts[2]), float(parts[3])))
            elif parts[0] == "offsets":
                offsets = [float(x) for x in parts[1:]]
    return layers, offsets


def _distances(i, W, o, N):
    lo, hi = ref.offset_window_key_range(i, W, o)
    return sorted(i - j for j in range(N) if lo <= j <= hi)


def check_offset_layer_windows_match_page():
    """The page's layer windows [0, W], [W/2, 3W/2], [W, 2W] are distance
    ranges behind the query: the key set of a layer with offset o = lower * W
    is the W distances lower*W .. upper*W - 1 (a window holds W keys, so the
    printed upper end is where the next window starts).  The offsets 0, W/4,
    W/2, 3W/4 together reach every distance below 7W/4."""
    layers, offsets = load_offset_table()
    W, N = 16, 200
    i = N - 1
    for _, lo, hi in layers:
        o = int(lo * W)
        assert _distances(i, W, o, N) == list(range(int(lo * W), int(hi * W)))
    reach = set()
    for f in offsets:
        reach |= set(_distances(i, W, int(f * W), N))
    assert reach == set(range(int((offsets[-1] + 1) * W)))


def check_offset_brute_force():
    """Offset windows (with and without anchors) against the membership-test
    brute force, both branches and the distance; offsets inside the window,
    equal to it, beyond it and beyond the sequence (every window empty)."""
    B, N, Hq, Hkv, d, W = 1, 13, 4, 2, 3, 4
    Q, K, V = _rand_qkv(36, B, N, Hq, Hkv, d)
    gate = (np.random.default_rng(37).random((B, N, 2)) < 0.5).astype(np.uint8)
    for o, A in ((1, 0), (2, 0), (4, 0), (6, 0), (20, 0), (3, 2), (5, 3)):
        O_bf, diff_bf = brute_force(Q, K, V, gate, W, 0.9, A=A, o=o)
        out = ref.prefill(Q, K, V, gate, W, scale=0.9, both_branch=True, anchors=A, offset=o)
        np.testing.assert_allclose(out["O"], O_bf, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out["diff"], diff_bf, rtol=1e-12, atol=1e-14)
        hard = ref.prefill(Q, K, V, gate, W, scale=0.9, anchors=A, offset=o)["O"]
        np.testing.assert_allclose(hard, O_bf, rtol=0, atol=1e-12)


def check_offset_against_sdpa():
    """Gate all zeros with offset o equals torch's float64 attention under
    the mask i-o-W < j <= i-o on rows i >= o; rows i < o are exactly 0;
    offset 0 is the plain window; with W + o >= N every row i >= o sees the
    prefix [0, i-o]; gate all ones does not depend on the offset."""
    B, N, Hq, Hkv, d, W = 1, 90, 4, 2, 8, 16
    Q, K, V = _rand_qkv(38, B, N, Hq, Hkv, d)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    zeros = np.zeros((B, N, 1), np.uint8)
    for o, Wl in ((5, W), (16, W), (23, W), (0, W), (40, 60)):
        out = ref.prefill(Q, K, V, zeros, W=Wl, offset=o)["O"]
        mask = (j <= i - o) & (j > i - o - Wl)
        live = np.arange(N) >= o
        np.testing.assert_allclose(out[:, live], _torch_sdpa(Q, K, V, mask)[:, live], rtol=0, atol=1e-12)
        assert np.all(out[:, ~live] == 0.0)
        if Wl + o >= N:
            np.testing.assert_allclose(out[:, live], _torch_sdpa(Q, K, V, j <= i - o)[:, live], rtol=0,
                                       atol=1e-12)
    plain = ref.prefill(Q, K, V, zeros, W=W)["O"]
    np.testing.assert_allclose(ref.prefill(Q, K, V, zeros, W=W, offset=0)["O"], plain, rtol=0, atol=0)
    ones = np.ones((B, N, 1), np.uint8)
    full = _torch_sdpa(Q, K, V, j <= i)
    for o in (0, 7, 30):
        np.testing.assert_allclose(ref.prefill(Q, K, V, ones, W=W, offset=o)["O"], full, rtol=0, atol=1e-12)


def check_offset_closed_forms():
    """W = 1, offset 2: row i returns v_{i-2} exactly and rows 0, 1 return 0;
    q = 0 with V = identity gives weight 1/W on the W keys at distances
    o .. o+W-1 (the window of the page's table shifted back by o)."""
    N = 9
    Q, K, V = _rand_qkv(39, 1, N, 2, 1, 4)
    out = ref.prefill(Q, K, V, np.zeros((1, N, 1), np.uint8), W=1, offset=2)["O"][0]
    for h in range(2):
        assert np.all(out[:2, h] == 0.0)
        assert np.array_equal(out[2:, h], V[0, :-2, 0])
    table = load_w4_table()
    Nt, o = 7 + 3, 3
    Qz = np.zeros((1, Nt, 1, Nt))
    Kz = np.random.default_rng(40).standard_normal((1, Nt, 1, Nt))
    Vi = np.eye(Nt)[None, :, None, :]
    got = ref.prefill(Qz, Kz, Vi, np.zeros((1, Nt, 1), np.uint8), W=4, offset=o)["O"][0, :, 0, :]
    assert np.all(got[:o] == 0.0)
    expect = table / table.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(got[o:, :7], expect, rtol=0, atol=1e-15)
    assert np.all(got[o:, 7:] == 0.0)


def check_offset_decode_equals_last_prefill_row():
    """Decode with a window offset at cache length L reproduces the offset
    prefill row L-1, also for L <= o (output 0) and with anchors."""
    B, Lmax, Hq, Hkv, d, W = 4, 60, 4, 2, 8, 12
    Q, K, V = _rand_qkv(41, B, Lmax, Hq, Hkv, d)
    lens = np.array([60, 16, 5, 30])
    gate = np.array([[0], [0], [0], [1]], np.uint8)
    q = np.stack([Q[b, lens[b] - 1] for b in range(B)])
    for o, A in ((6, 0), (6, 4), (20, 0)):
        dec = ref.decode(q, K, V, lens, gate, W, anchors=A, offset=o)["o"]
        for b in range(B):
            L = lens[b]
            g = np.broadcast_to(gate[b], (1, L, 1)).astype(np.uint8)
            pre = ref.prefill(Q[b:b + 1, :L], K[b:b + 1, :L], V[b:b + 1, :L], g, W, anchors=A,
                              offset=o)["O"][0, L - 1]
            np.testing.assert_allclose(dec[b], pre, rtol=0, atol=1e-13)
        assert np.all(dec[2] == 0.0) == (lens[2] <= o)


def check_convex_hull():
    """Softmax weights are non-negative and sum to one: every output channel
    lies between the smallest and largest attended value."""
    Q, K, V = _rand_qkv(11, 1, 80, 2, 1, 8)
    gate = (np.random.default_rng(12).random((1, 80, 1)) < 0.3).astype(np.uint8)
    W = 10
    O = ref.prefill(Q * 3, K, V, gate, W)["O"]
    for i in range(80):
        lo = 0 if gate[0, i, 0] else max(0, i - W + 1)
        vs = V[0, lo:i + 1, 0]
        for h in range(2):
            assert np.all(O[0, i, h] >= vs.min(axis=0) - 1e-12)
            assert np.all(O[0, i, h] <= vs.max(axis=0) + 1e-12)


def check_router_closed_form():
    """One-hot hidden states make each logit c * r[k, g] + bias exactly; the
    gate is 1 exactly when the logit is positive (sigmoid above one half),
    a logit of exactly 0 routes to the window branch."""
    hidden, G = 8, 2
    r = np.arange(hidden * G, dtype=np.float64).reshape(hidden, G) / 4.0 - 1.5
    bias = np.array([0.25, -0.5])
    ks = [0, 3, 5, 7, 2, 6]
    cs = [1.0, -2.0, 0.5, 3.0, -1.0, 2.0]
    H = np.zeros((1, len(ks), hidden))
    for t, (k, c) in enumerate(zip(ks, cs)):
        H[0, t, k] = c
    out = ref.route(H, r, bias)
    expect = np.array([[c * r[k, g] + bias[g] for g in range(G)] for k, c in zip(ks, cs)])
    np.testing.assert_array_equal(out["z"][0], expect)
    np.testing.assert_array_equal(out["gate"][0], (expect > 0).astype(np.uint8))
    # a logit of exactly zero: strict threshold -> 0; just above -> 1
    Hz = np.array([[[1.0], [1.0]]])
    z0 = ref.route(Hz, np.array([[0.5]]), np.array([-0.5]))
    z1 = ref.route(Hz, np.array([[0.5]]), np.array([-0.4999]))
    assert z0["gate"][0, 0, 0] == 0 and z0["near"][0, 0, 0]
    assert z1["gate"][0, 0, 0] == 1 and not z1["near"][0, 0, 0]


def check_compact():
    gate = (np.random.default_rng(13).random((2, 300, 3)) < 0.2).astype(np.uint8)
    gate[1, :, 2] = 0
    gate[0, :, 1] = 1
    idx, cnt = ref.compact(gate)
    for b in range(2):
        for g in range(3):
            pos = [i for i in range(300) if gate[b, i, g]]
            assert cnt[b, g] == len(pos)
            assert list(idx[b, g, : len(pos)]) == pos
            assert np.all(idx[b, g, len(pos):] == -1)


def check_regularizer_hand_values():
    """[SwiAttn] section 2, adaptive regulariser: values worked by hand with
    gamma_base = 1e-3, eps = 0.1, alpha = 100.
      z = 0, NLL = 0.9, d = 0:      gamma = 1e-3 / 1.0 = 1e-3, softplus(0) = ln 2
      z = 0, NLL = 0, d = 0.009:    alpha*d = 0.9, the same gamma and value
      z = ln(e - 1), NLL = 1.9:     softplus = ln e = 1, gamma = 1e-3 / 2
      z = 50:                       softplus(50) = 50 + ln(1 + e^-50) = 50 to double precision
      z = -50:                      softplus(-50) = ln(1 + e^-50) = e^-50 (1 - e^-50/2 ...)
      z = 800:                      softplus(800) = 800 (no overflow)"""
    z = np.array([0.0, 0.0, math.log(math.e - 1.0), 50.0, -50.0, 800.0])
    nll = np.array([0.9, 0.0, 1.9, 0.9, 0.9, 0.9])
    d = np.array([0.0, 0.009, 0.0, 0.0, 0.0, 0.0])
    L = ref.regularizer(z[None, :, None], nll[None], d[None])[0, :, 0]
    want = [1e-3 * math.log(2.0), 1e-3 * math.log(2.0), 5e-4, 1e-3 * 50.0,
            1e-3 * math.exp(-50.0), 1e-3 * 800.0]
    for got, w in zip(L, want):
        assert abs(got - w) <= 1e-12 * abs(w), (got, w)


def check_regularizer_ratios():
    """gamma is inversely proportional to eps + NLL + alpha*d, so
    L(d) / L(0) = (eps + NLL) / (eps + NLL + alpha d) for any logit, L scales
    with gamma_base, and every gate group of a token shares one gamma."""
    rng = np.random.default_rng(21)
    z = rng.normal(0.0, 3.0, (2, 40, 3))
    nll = rng.uniform(0.0, 5.0, (2, 40))
    d = rng.uniform(0.0, 0.2, (2, 40))
    L = ref.regularizer(z, nll, d)
    L0 = ref.regularizer(z, nll, np.zeros_like(d))
    assert np.allclose(L / L0, ((0.1 + nll) / (0.1 + nll + 100.0 * d))[..., None], rtol=1e-12, atol=0)
    assert np.allclose(ref.regularizer(z, nll, d, gamma_base=3e-3), 3.0 * L, rtol=1e-12, atol=0)
    # ratio across groups of one token = ratio of the softplus values
    sp = np.log1p(np.exp(z[..., 1])) / np.log1p(np.exp(z[..., 0]))
    assert np.allclose(L[..., 1] / L[..., 0], sp, rtol=1e-12, atol=0)


def check_decode_step_rebuilds_prefill():
    """Serving a sequence token by token from an empty cache (route the new
    token's hidden state, append its key and value, decode) reproduces the
    prefill rows of the whole sequence with the gates the router gives each
    token; the cache then holds exactly the sequence's keys and values."""
    rng = np.random.default_rng(41)
    B, N, Hq, Hkv, d, W, hidden, G = 2, 24, 4, 2, 8, 5, 16, 1
    Q, K, V = _rand_qkv(42, B, N, Hq, Hkv, d)
    H = rng.standard_normal((B, N, hidden))
    r = rng.standard_normal((hidden, G)) / 4.0
    bias = np.array([0.0])
    gates = ref.route(H, r, bias)["gate"]
    assert 0 < gates.sum() < B * N  # both branches occur
    pre = ref.prefill(Q, K, V, gates, W)["O"]
    Kc = np.full((B, N, Hkv, d), 7.0)
    Vc = np.full((B, N, Hkv, d), -7.0)
    L = np.zeros(B, np.int64)
    for t in range(N):
        st = ref.decode_step(H[:, t], r, bias, Q[:, t], K[:, t], V[:, t], Kc, Vc, L, W)
        Kc, Vc, L = st["Kc"], st["Vc"], st["cache_len"]
        assert np.array_equal(L, np.full(B, t + 1))
        assert np.array_equal(st["gate"], gates[:, t])
        np.testing.assert_allclose(st["o"], pre[:, t], rtol=0, atol=1e-13)
    assert np.array_equal(Kc, K) and np.array_equal(Vc, V)


def check_decode_step_ragged_and_full():
    """Each sequence appends at its own length; a full cache is left as it is
    and decodes over its Lmax keys (the same as decode() on it)."""
    rng = np.random.default_rng(43)
    B, Lmax, Hq, Hkv, d, W, hidden, G = 3, 10, 2, 1, 4, 3, 6, 2
    Kc = rng.standard_normal((B, Lmax, Hkv, d))
    Vc = rng.standard_normal((B, Lmax, Hkv, d))
    L0 = np.array([3, Lmax, 0])
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, d))
    v = rng.standard_normal((B, Hkv, d))
    Hn = rng.standard_normal((B, hidden))
    r = rng.standard_normal((hidden, G))
    bias = np.zeros(G)
    st = ref.decode_step(Hn, r, bias, q, k, v, Kc, Vc, L0, W)
    assert list(st["cache_len"]) == [4, Lmax, 1]
    assert np.array_equal(st["Kc"][0, 3], k[0]) and np.array_equal(st["Vc"][2, 0], v[2])
    assert np.array_equal(st["Kc"][1], Kc[1]) and np.array_equal(st["Vc"][1], Vc[1])
    mask = np.ones((B, Lmax), bool)
    mask[0, 3] = mask[2, 0] = False
    assert np.array_equal(st["Kc"][mask], Kc[mask])
    want = ref.decode(q[1:2], Kc[1:2], Vc[1:2], [Lmax], st["gate"][1:2], W)["o"]
    np.testing.assert_allclose(st["o"][1:2], want, rtol=0, atol=0)


def _router_grad_case(seed, B=2, N=5, Hq=4, d=3, G=2, hidden=6):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((B, N, hidden))
    r = rng.standard_normal((hidden, G)) * 0.5
    bias = rng.standard_normal(G) * 0.3
    Of = rng.standard_normal((B, N, Hq, d))
    Os = rng.standard_normal((B, N, Hq, d))
    dO = rng.standard_normal((B, N, Hq, d))
    return H, r, bias, Of, Os, dO


def _soft_surrogate(H, r, bias, Of, Os, dO):
    """Sum of dO times the output with the soft gate in place of the hard one
    (the function whose gradient the straight-through estimator returns)."""
    B, N, Hq, d = Of.shape
    G = r.shape[1]
    soft = 1.0 / (1.0 + np.exp(-(H @ r + bias)))                # [B,N,G]
    sh = np.repeat(soft, Hq // G, axis=2)[..., None]            # heads in group order
    return float((dO * (sh * Of + (1.0 - sh) * Os)).sum())


def check_router_backward_finite_differences():
    """Central differences (h = 1e-6) of the soft surrogate with respect to
    every entry of H, r and bias match dH, dr and dbias."""
    H, r, bias, Of, Os, dO = _router_grad_case(51)
    z = H @ r + bias
    g = ref.router_backward(dO, Of, Os, z, H, r)
    eps = 1e-6
    for name, arr, want in (("H", H, g["dH"]), ("r", r, g["dr"]), ("bias", bias, g["dbias"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            a1, a2 = arr.copy(), arr.copy()
            a1[i] += eps
            a2[i] -= eps
            args = {"H": H, "r": r, "bias": bias}
            args[name] = a1
            f1 = _soft_surrogate(args["H"], args["r"], args["bias"], Of, Os, dO)
            args[name] = a2
            f2 = _soft_surrogate(args["H"], args["r"], args["bias"], Of, Os, dO)
            num[i] = (f1 - f2) / (2 * eps)
        np.testing.assert_allclose(want, num, rtol=1e-6, atol=1e-8, err_msg=name)


def check_router_backward_against_autograd():
    """torch float64 autograd of the soft surrogate gives the same dz, dH,
    dr and dbias (a library routine, independent of the formula)."""
    H, r, bias, Of, Os, dO = _router_grad_case(52, B=1, N=7, Hq=6, d=4, G=3, hidden=5)
    Ht = torch.tensor(H, requires_grad=True)
    rt = torch.tensor(r, requires_grad=True)
    bt = torch.tensor(bias, requires_grad=True)
    zt = Ht @ rt + bt
    zt.retain_grad()
    soft = torch.sigmoid(zt).repeat_interleave(2, dim=2)[..., None]
    loss = (torch.tensor(dO) * (soft * torch.tensor(Of) + (1 - soft) * torch.tensor(Os))).sum()
    loss.backward()
    g = ref.router_backward(dO, Of, Os, (H @ r + bias), H, r)
    np.testing.assert_allclose(g["dz"], zt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dH"], Ht.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dr"], rt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dbias"], bt.grad.numpy(), rtol=1e-12, atol=1e-14)


def check_router_backward_special_cases():
    """Identical branches give zero gradients; dO = O_FULL - O_SWA gives
    dz = soft(1-soft) * (the group's squared branch distance) >= 0; at
    z = 0 the factor is exactly 1/4; one hot r picks H's column."""
    H, r, bias, Of, Os, dO = _router_grad_case(53, B=1, N=4, Hq=2, d=3, G=1, hidden=3)
    z = H @ r + bias
    zero = ref.router_backward(dO, Of, Of, z, H, r)
    for k in ("dz", "dH", "dr", "dbias"):
        assert np.all(zero[k] == 0.0), k
    g = ref.router_backward(Of - Os, Of, Os, np.zeros_like(z), H, r)
    dist = ((Of - Os) ** 2).sum(axis=(2, 3))[..., None]
    np.testing.assert_allclose(g["dz"], 0.25 * dist, rtol=1e-14)
    r1 = np.zeros((3, 1))
    r1[1, 0] = 1.0
    g1 = ref.router_backward(dO, Of, Os, z, H, r1)
    np.testing.assert_allclose(g1["dH"][..., 1], g1["dz"][..., 0], rtol=0, atol=0)
    assert np.all(g1["dH"][..., [0, 2]] == 0.0)
    np.testing.assert_allclose(g1["dr"][:, 0], (H * g1["dz"]).sum(axis=(0, 1)), rtol=1e-14)


def check_prefill_backward_finite_differences():
    """Central differences (h = 1e-6) of L = sum(dO * O) through the forward
    reference prefill() give dQ, dK, dV, for a mixed gate, GQA and two gate
    groups (the forward is pinned on its own)."""
    rng = np.random.default_rng(81)
    B, N, Hq, Hkv, d, W = 1, 7, 4, 2, 3, 3
    Q, K, V = (rng.standard_normal(s) for s in ((B, N, Hq, d), (B, N, Hkv, d), (B, N, Hkv, d)))
    dO = rng.standard_normal((B, N, Hq, d))
    gate = (rng.random((B, N, 2)) < 0.5).astype(np.uint8)
    g = ref.prefill_backward(Q, K, V, gate, W, dO, scale=0.8)
    eps = 1e-6

    def loss(q, k, v):
        return float((dO * ref.prefill(q, k, v, gate, W, scale=0.8)["O"]).sum())
    for name, arr in (("dQ", Q), ("dK", K), ("dV", V)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            args1 = [Q, K, V]
            args2 = [Q, K, V]
            pos = {"dQ": 0, "dK": 1, "dV": 2}[name]
            args1[pos], args2[pos] = a1, a2
            num[idx] = (loss(*args1) - loss(*args2)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)


def check_prefill_backward_against_autograd():
    """torch float64 autograd through scaled_dot_product_attention with the
    per-row masks of the gate (a library routine) gives dQ, dK, dV."""
    rng = np.random.default_rng(82)
    B, N, Hq, Hkv, d, W = 2, 40, 4, 2, 8, 9
    Q, K, V = (rng.standard_normal(s) for s in ((B, N, Hq, d), (B, N, Hkv, d), (B, N, Hkv, d)))
    dO = rng.standard_normal((B, N, Hq, d))
    gate = (rng.random((B, N, 1)) < 0.3).astype(np.uint8)
    g = ref.prefill_backward(Q, K, V, gate, W, dO)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    qt = torch.tensor(Q, requires_grad=True)
    kt = torch.tensor(K, requires_grad=True)
    vt = torch.tensor(V, requires_grad=True)
    outs = []
    for b in range(B):
        sig = gate[b, :, 0].astype(bool)[:, None]
        mask = torch.from_numpy(np.where(sig, j <= i, (j <= i) & (j > i - W)))
        q = qt[b].permute(1, 0, 2)
        k = kt[b].permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        v = vt[b].permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask).permute(1, 0, 2))
    loss = (torch.stack(outs) * torch.tensor(dO)).sum()
    loss.backward()
    np.testing.assert_allclose(g["dQ"], qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dK"], kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dV"], vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def check_prefill_backward_special_cases():
    """W = 1 (each row sees only itself): dV = dO summed over the query heads
    of the KV head, dQ = dK = 0 (a one-key softmax does not depend on the
    score).  Gate all ones equals the W >= N result."""
    rng = np.random.default_rng(83)
    B, N, Hq, Hkv, d = 1, 9, 4, 2, 5
    Q, K, V = (rng.standard_normal(s) for s in ((B, N, Hq, d), (B, N, Hkv, d), (B, N, Hkv, d)))
    dO = rng.standard_normal((B, N, Hq, d))
    g = ref.prefill_backward(Q, K, V, np.zeros((B, N, 1), np.uint8), 1, dO)
    np.testing.assert_allclose(g["dV"], dO.reshape(B, N, Hkv, Hq // Hkv, d).sum(axis=3), rtol=1e-14, atol=1e-14)
    assert np.all(np.abs(g["dQ"]) < 1e-14) and np.all(np.abs(g["dK"]) < 1e-14)
    a = ref.prefill_backward(Q, K, V, np.ones((B, N, 1), np.uint8), 3, dO)
    c = ref.prefill_backward(Q, K, V, np.zeros((B, N, 1), np.uint8), N, dO)
    for k in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(a[k], c[k], rtol=1e-13, atol=1e-13)


def check_prefill_backward_rows_matches_full():
    """The per-row dQ evaluation equals the rows of the full backward."""
    rng = np.random.default_rng(84)
    B, N, Hq, Hkv, d, W = 2, 30, 4, 2, 6, 7
    Q, K, V = (rng.standard_normal(s) for s in ((B, N, Hq, d), (B, N, Hkv, d), (B, N, Hkv, d)))
    dO = rng.standard_normal((B, N, Hq, d))
    gate = (rng.random((B, N, 2)) < 0.4).astype(np.uint8)
    full = ref.prefill_backward(Q, K, V, gate, W, dO)["dQ"]
    rows = np.array([0, 1, 6, 7, 8, 29])
    np.testing.assert_allclose(ref.prefill_backward_rows(Q, K, V, gate, W, dO, rows), full[:, rows],
                               rtol=1e-12, atol=1e-13)


def check_prefill_backward_keys_matches_full():
    """The per-key dK, dV evaluation equals the rows of the full backward
    (keys at both ends and at the window edge; one KV head alone too)."""
    rng = np.random.default_rng(85)
    B, N, Hq, Hkv, d, W = 2, 40, 4, 2, 6, 7
    Q, K, V = (rng.standard_normal(s) for s in ((B, N, Hq, d), (B, N, Hkv, d), (B, N, Hkv, d)))
    dO = rng.standard_normal((B, N, Hq, d))
    gate = (rng.random((B, N, 2)) < 0.4).astype(np.uint8)
    full = ref.prefill_backward(Q, K, V, gate, W, dO)
    keys = np.array([0, 1, 6, 7, 20, 33, 39])
    got = ref.prefill_backward_keys(Q, K, V, gate, W, dO, keys)
    for k in ("dK", "dV"):
        np.testing.assert_allclose(got[k], full[k][:, keys], rtol=1e-12, atol=1e-13)
    one = ref.prefill_backward_keys(Q, K, V, gate, W, dO, keys, kv_heads=[1])
    np.testing.assert_allclose(one["dK"][:, :, 0], full["dK"][:, keys, 1], rtol=1e-12, atol=1e-13)


ALL_PINS = [
    check_w4_key_ranges,
    check_w4_attention_weights,
    check_full_branch_causal,
    check_window_covering_all_equals_full,
    check_window_one_returns_v,
    check_gate_extremes_against_sdpa,
    check_rows_before_window_have_no_discrepancy,
    check_decode_equals_last_prefill_row,
    check_brute_force_tiny,
    check_convex_hull,
    check_router_closed_form,
    check_compact,
    check_regularizer_hand_values,
    check_regularizer_ratios,
    check_decode_step_rebuilds_prefill,
    check_decode_step_ragged_and_full,
    check_anchors_brute_force,
    check_anchors_closed_form,
    check_anchors_against_sdpa_and_cover,
    check_anchored_decode_equals_last_prefill_row,
    check_offset_layer_windows_match_page,
    check_offset_brute_force,
    check_offset_against_sdpa,
    check_offset_closed_forms,
    check_offset_decode_equals_last_prefill_row,
    check_router_backward_finite_differences,
    check_router_backward_against_autograd,
    check_router_backward_special_cases,
    check_prefill_backward_finite_differences,
    check_prefill_backward_against_autograd,
    check_prefill_backward_special_cases,
    check_prefill_backward_rows_matches_full,
    check_prefill_backward_keys_matches_full,
]

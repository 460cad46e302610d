"""SwiAttn routed dual-branch attention: plain CPU reference in float64.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
check of the package entry file and the CPU-baseline leg of the benchmark
may import or call this module.  The HIP library never routes through it,
and this module imports nothing from the HIP package (it shares no code,
tables or helpers with it).

Sources (cited by page title and section):
  [SwiAttn]  paper-daily report on SwiAttn (Peking University),
             section 2 "方法详解" (router, hard gate with STE, the two branches
             and their gated combination, shared KV cache in decode, adaptive
             regulariser).
  [Glossary] weimeta glossary "滑窗注意力 Sliding Window Attention 是什么？",
             section "详细解释" (the SWA key set), the W=4 visualisation table,
             and the FAQ entry on W equal to the context length.

Every floating-point step runs in float64 on the values the caller passes
(bf16 or fp32 values decoded exactly).  Readings taken where the pages leave
a step open are marked "Reading:" in the docstrings.

Pins: every function below is checked by the CPU tests against something
other than itself (the printed W=4 table, W>=N equals causal attention,
W=1 returns V, all-ones / all-zeros gates against torch's CPU
scaled_dot_product_attention in float64, a pure-Python brute force on tiny
inputs, closed forms for the router, decode equal to the last prefill row,
hand-computed values and exact ratios for the regulariser).
No function here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "route",
    "compact",
    "swa_key_range",
    "anchor_key_range",
    "offset_window_key_range",
    "full_key_range",
    "attend_rows",
    "prefill",
    "decode",
    "softplus",
    "regularizer",
    "decode_step",
    "router_backward",
    "prefill_backward",
    "prefill_backward_rows",
    "prefill_backward_keys",
]

NEAR_THRESHOLD = 1e-5


# ---------------------------------------------------------------------------
# Router  ([SwiAttn] section 2, router paragraph)
# ---------------------------------------------------------------------------
def route(H, r, bias):
    """Per-token router: a linear map of the hidden state, a sigmoid, then a
    hard threshold at 0.5.

    [SwiAttn] section 2: the soft gate is sigmoid(R(H)) with R linear; the
    forward value of the straight-through estimator is the 0/1 indicator of
    soft gate > 0.5 (the sigmoid term and its stop-gradient copy cancel in
    value, so the forward value is the indicator itself).

    Reading: R(H) = H.r + bias with r of shape [hidden, G] (one logit per
    gate group).  The threshold is strict, so a logit of exactly 0 routes to
    the window branch.

    H [B,N,hidden], r [hidden,G], bias [G]  ->  dict with
      z    float64 [B,N,G]  router logits
      soft float64 [B,N,G]  sigmoid(z)
      gate uint8   [B,N,G]  1 = full branch, 0 = window branch
      near bool    [B,N,G]  |z| < 1e-5 (either decision is acceptable there)
    """
    Hd = np.asarray(H, dtype=np.float64)
    rd = np.asarray(r, dtype=np.float64)
    bd = np.asarray(bias, dtype=np.float64)
    z = Hd @ rd + bd  # [B,N,G]
    with np.errstate(over="ignore"):
        soft = 1.0 / (1.0 + np.exp(-z))
    gate = (soft > 0.5).astype(np.uint8)
    near = np.abs(z) < NEAR_THRESHOLD
    return {"z": z, "soft": soft, "gate": gate, "near": near}


def compact(gate):
    """Ascending positions of the tokens routed to the full branch.

    gate uint8 [B,N,G]  ->  idx int32 [B,G,N] (first cnt entries valid, the
    rest -1), cnt int32 [B,G].

    Reading: the pages fix no order; ascending position is the one order that
    is unique given the gate.
    """
    g = np.asarray(gate)
    B, N, G = g.shape
    idx = np.full((B, G, N), -1, dtype=np.int32)
    cnt = np.zeros((B, G), dtype=np.int32)
    for b in range(B):
        for k in range(G):
            pos = np.flatnonzero(g[b, :, k] != 0)
            idx[b, k, : pos.size] = pos
            cnt[b, k] = pos.size
    return idx, cnt


# ---------------------------------------------------------------------------
# Key sets of the two branches
# ---------------------------------------------------------------------------
def swa_key_range(i, W):
    """Window branch key set of query position i: the W most recent keys,
    self included, clipped at position 0 -> inclusive [max(0, i-W+1), i].

    [Glossary] section "详细解释" and the W=4 table (row t4 drops t0)."""
    return max(0, i - W + 1), i


def anchor_key_range(i, W, A):
    """Global anchors of the window branch: the first A keys of the sequence,
    which every query sees in addition to its window, minus the keys its
    window already holds -> inclusive [0, min(A, i-W+1) - 1] (empty, hi < lo,
    when A = 0 or the window reaches position 0).

    [Glossary] section "SWA 落地的四个常见坑", pitfall 1, fix (2): the keys
    of the first 256 tokens are listed on their own, every query also
    attends to them, and they take no part in the sliding.
    Reading: an anchor is a key like any other in the window branch's
    softmax (one key set, window union anchors); anchors are causal like the
    window (the window starts at or before i, so the anchors end before it);
    the full branch already sees them."""
    lo, _ = swa_key_range(i, W)
    return 0, min(A, lo) - 1


def offset_window_key_range(i, W, offset):
    """Window branch key set of query position i in a layer whose window is
    offset by `offset` >= 0 positions: the W keys at distances offset ..
    offset+W-1 behind the query, i.e. the plain window of the query `offset`
    positions earlier -> inclusive [max(0, i-offset-W+1), i-offset]; empty
    (hi < lo) when i < offset.

    [Glossary] section "两个核心工程参数（W 和步长 S）详解": the stride S is
    the offset between the windows of different layers (no offset, or half a
    window between neighbouring layers; offsets 0, W/4, W/2, 3W/4 in turn
    reach past W); pitfall 2, fix (2): the windows of layers 0, 1, 2 are
    [0, W], [W/2, 3W/2], [W, 2W].
    Reading: those intervals are distances behind the query, W keys each
    (the glossary's window holds W keys); the query itself is in the set
    only for offset 0; a row with no key in its window has window output 0
    (an empty attention sum)."""
    return swa_key_range(i - offset, W)


def full_key_range(i):
    """Full branch key set of query position i: every key up to and including
    i -> inclusive [0, i].

    Reading: causal.  [Glossary] FAQ on W equal to the context length states
    that the window mask then becomes the whole lower triangle, identical to
    full attention, so full attention here is the causal one."""
    return 0, i


# ---------------------------------------------------------------------------
# Softmax attention over an explicit key interval per row
# ---------------------------------------------------------------------------
def attend_rows(q, K, V, lo, hi, scale, lo2=None, hi2=None):
    """Softmax attention of each query row over its own inclusive key interval
    (and, if given, a second interval disjoint from it: one key set, their
    union).

    q [R,d], K [L,d], V [L,dv], lo/hi int [R]  ->
      O   float64 [R,dv]  sum_j p_j v_j / sum_j p_j,  p_j = exp(s_j - max s)
      lse float64 [R]     log sum_j exp(s_j)
    with s_j = scale * <q, k_j> for lo <= j <= hi (or lo2 <= j <= hi2; an
    interval with hi < lo is empty).  A row whose key set is empty attends
    to nothing: O = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lo = np.asarray(lo, dtype=np.int64)
    hi = np.asarray(hi, dtype=np.int64)
    R = q.shape[0]
    two = lo2 is not None
    if two:
        lo2 = np.broadcast_to(np.asarray(lo2, dtype=np.int64), (R,))
        hi2 = np.broadcast_to(np.asarray(hi2, dtype=np.int64), (R,))
    O = np.empty((R, V.shape[1]), dtype=np.float64)
    lse = np.empty(R, dtype=np.float64)
    if R == 0:
        return O, lse
    # a row whose key set is empty attends to nothing: output 0, lse -inf
    live = hi >= lo
    if two:
        live |= hi2 >= lo2
    O[~live] = 0.0
    lse[~live] = -np.inf
    # rows are independent: evaluate the live ones in batches that bound memory
    top = np.maximum(hi, hi2) if two else hi
    order = np.flatnonzero(live)[np.argsort(top[live], kind="stable")]
    R = order.size
    if R == 0:
        return O, lse
    n = max(1, (1 << 24) // (int(top[live].max()) + 1))  # score elements per batch
    start = 0
    while start < R:
        sel = order[start : start + n]
        live1 = hi[sel] >= lo[sel]
        kmin, kmax = np.iinfo(np.int64).max, 0
        if live1.any():
            kmin = int(lo[sel][live1].min())
            kmax = int(hi[sel][live1].max()) + 1
        if two:
            live2 = hi2[sel] >= lo2[sel]
            if live2.any():
                kmin = min(kmin, int(lo2[sel][live2].min()))
                kmax = max(kmax, int(hi2[sel][live2].max()) + 1)
        j = np.arange(kmin, kmax)
        s = scale * (q[sel] @ K[kmin:kmax].T)
        mask = (j[None, :] >= lo[sel, None]) & (j[None, :] <= hi[sel, None])
        if two:
            mask |= (j[None, :] >= lo2[sel, None]) & (j[None, :] <= hi2[sel, None])
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        O[sel] = (p @ V[kmin:kmax]) / l
        lse[sel] = m[:, 0] + np.log(l[:, 0])
        start += sel.size
    return O, lse


def _head_maps(Hq, Hkv, G):
    if Hq % Hkv or Hq % G:
        raise ValueError("Hq must be a multiple of Hkv and of G")
    # Reading: consecutive grouping of query heads onto KV heads and gate groups
    return Hq // Hkv, Hq // G


# ---------------------------------------------------------------------------
# Prefill: both branches on shared Q/K/V, gated combination
# ---------------------------------------------------------------------------
def prefill(Q, K, V, gate, W, scale=None, both_branch=False, rows=None, anchors=0, offset=0):
    """Dual-branch attention forward over a prefix.

    [SwiAttn] section 2, dual-branch paragraph: both branches use the same Q,
    K, V; the output is O = sigma * O_FULL + (1 - sigma) * O_SWA.  With the
    hard gate sigma in {0,1} this is a per-token selection.
    [SwiAttn] section 2, regulariser paragraph: the per-token branch
    discrepancy is the squared L2 norm of O_FULL - O_SWA.

    Reading: the discrepancy of token i sums the squares over every query head
    and every channel of the attention output (no output projection is named).

    Q [B,N,Hq,d], K/V [B,N,Hkv,d], gate [B,N,G] (0/1)
    rows: optional sorted token positions to evaluate (default all N)
    anchors: A >= 0 global anchor keys added to the window branch
             (anchor_key_range); 0 is plain SWA
    offset:  o >= 0 window offset of the layer (offset_window_key_range):
             the window branch of query i takes the window and anchors of
             query i - o; 0 is plain SWA
    ->  dict
      O     float64 [B,R,Hq,d]
      lse   float64 [B,R,Hq]      natural-log normaliser of the chosen branch
      diff  float64 [B,R]         only when both_branch
      O_full, O_swa float64 [B,R,Hq,d]  only when both_branch
    """
    Q = np.asarray(Q)
    K = np.asarray(K)
    V = np.asarray(V)
    gate = np.asarray(gate)
    B, N, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = gate.shape[2]
    hk, hg = _head_maps(Hq, Hkv, G)
    if scale is None:
        scale = 1.0 / np.sqrt(d)  # Reading: the pages fix no softmax scale
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    dv = V.shape[3]
    O = np.empty((B, R, Hq, dv))
    lse = np.empty((B, R, Hq))
    if both_branch:
        Of = np.empty((B, R, Hq, dv))
        Os = np.empty((B, R, Hq, dv))
    sw = np.array([offset_window_key_range(int(i), W, offset) for i in rows],
                  dtype=np.int64).reshape(R, 2)
    an = np.array([anchor_key_range(int(i) - offset, W, anchors) for i in rows],
                  dtype=np.int64).reshape(R, 2)
    fu = np.array([full_key_range(int(i)) for i in rows], dtype=np.int64).reshape(R, 2)
    none = np.array([0, -1], dtype=np.int64)  # no second interval
    for b in range(B):
        for h in range(Hq):
            kv, g = h // hk, h // hg
            qh = Q[b, rows, h, :]
            sig = gate[b, rows, g] != 0
            if both_branch:
                o_f, l_f = attend_rows(qh, K[b, :, kv], V[b, :, kv], fu[:, 0], fu[:, 1], scale)
                o_s, l_s = attend_rows(qh, K[b, :, kv], V[b, :, kv], sw[:, 0], sw[:, 1], scale,
                                       an[:, 0], an[:, 1])
                Of[b, :, h], Os[b, :, h] = o_f, o_s
                O[b, :, h] = np.where(sig[:, None], o_f, o_s)
                lse[b, :, h] = np.where(sig, l_f, l_s)
            else:
                lo = np.where(sig, fu[:, 0], sw[:, 0])
                hi = np.where(sig, fu[:, 1], sw[:, 1])
                lo2 = np.where(sig, none[0], an[:, 0])
                hi2 = np.where(sig, none[1], an[:, 1])
                O[b, :, h], lse[b, :, h] = attend_rows(qh, K[b, :, kv], V[b, :, kv], lo, hi, scale,
                                                       lo2, hi2)
    out = {"O": O, "lse": lse}
    if both_branch:
        out["O_full"], out["O_swa"] = Of, Os
        out["diff"] = ((Of - Os) ** 2).sum(axis=(2, 3))
    return out


# ---------------------------------------------------------------------------
# Decode: one new query per sequence against the shared KV cache
# ---------------------------------------------------------------------------
def decode(q, Kc, Vc, cache_len, gate, W, scale=None, anchors=0, offset=0):
    """One decode step per sequence, both branches reading one KV cache.

    [SwiAttn] section 2: in decode the two branches share the KV cache.
    Reading: the cache of sequence b already holds the new token, so the
    query sits at position L-1 with L = cache_len[b]; the full branch reads
    keys [0, L-1] and the window branch the last min(W, L) of them.  The cache
    is linear (no ring buffer), since any later token may route full.

    q [B,Hq,d], Kc/Vc [B,Lmax,Hkv,d], cache_len int [B] (1 <= L <= Lmax),
    gate [B,G]  ->  dict  o float64 [B,Hq,d], lse float64 [B,Hq]
    anchors: A >= 0 global anchor keys of the window branch (anchor_key_range
    at position L-1); the anchors stay in the linear cache like every key.
    offset: o >= 0 window offset of the layer (offset_window_key_range): a
    window head takes the window and anchors of position L-1-o (none when
    L-1 < o: output 0).
    """
    q = np.asarray(q)
    gate = np.asarray(gate)
    B, Hq, d = q.shape
    Hkv = Kc.shape[2]
    G = gate.shape[1]
    hk, hg = _head_maps(Hq, Hkv, G)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, Hq, Vc.shape[3]))
    lse = np.empty((B, Hq))
    for b in range(B):
        i = int(cache_len[b]) - 1
        for h in range(Hq):
            kv, g = h // hk, h // hg
            if gate[b, g]:
                (lo, hi), (lo2, hi2) = full_key_range(i), (0, -1)
            else:
                (lo, hi) = offset_window_key_range(i, W, offset)
                (lo2, hi2) = anchor_key_range(i - offset, W, anchors)
            ob, lb = attend_rows(q[b, h][None, :], np.asarray(Kc[b, : i + 1, kv]),
                                 np.asarray(Vc[b, : i + 1, kv]), [lo], [hi], scale, [lo2], [hi2])
            o[b, h], lse[b, h] = ob[0], lb[0]
    return {"o": o, "lse": lse}


# ---------------------------------------------------------------------------
# Serving decode step  ([SwiAttn] section 2: router per token, shared cache)
# ---------------------------------------------------------------------------
def decode_step(Hn, r, bias, q, k, v, Kc, Vc, cache_len, W, scale=None, anchors=0):
    """One serving step: route the new tokens, append their keys and values
    to the shared cache, then decode.

    [SwiAttn] section 2: the router decides per token, from its hidden state,
    which branch it takes, and in decode both branches read one KV cache, so
    the new token's key and value are appended whatever the gate says.

    Hn [B,hidden] hidden states of the new tokens, r [hidden,G], bias [G];
    q [B,Hq,d]; k, v [B,Hkv,d] the new tokens' keys and values;
    Kc, Vc [B,Lmax,Hkv,d] and cache_len [B] the cache before the step (not
    modified: copies are returned).
    Returns dict gate [B,G], z [B,G], Kc, Vc, cache_len (after the step),
    o [B,Hq,d], lse [B,Hq].

    Reading: the new token of sequence b goes to position cache_len[b] and
    the length grows by one; the query then sits at that position, as in
    decode().  A sequence whose cache is already full (cache_len = Lmax) is
    not appended and decodes over the cache as it stands.
    """
    Hn = np.asarray(Hn)
    rt = route(Hn[:, None, :], r, bias)
    gate = rt["gate"][:, 0, :]
    Kc = np.array(Kc, copy=True)
    Vc = np.array(Vc, copy=True)
    L = np.array(cache_len, dtype=np.int64, copy=True)
    Lmax = Kc.shape[1]
    for b in range(L.shape[0]):
        if L[b] < Lmax:
            Kc[b, L[b]] = k[b]
            Vc[b, L[b]] = v[b]
            L[b] += 1
    out = decode(q, Kc, Vc, L, gate, W, scale, anchors)
    return {"gate": gate, "z": rt["z"][:, 0, :], "Kc": Kc, "Vc": Vc, "cache_len": L,
            "o": out["o"], "lse": out["lse"]}


# ---------------------------------------------------------------------------
# Adaptive regulariser  ([SwiAttn] section 2, adaptive regulariser paragraph)
# ---------------------------------------------------------------------------
def softplus(x):
    """log(1 + e^x), evaluated as max(x, 0) + log1p(e^-|x|) (no overflow)."""
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def regularizer(z, nll, diff, gamma_base=1e-3, eps=0.1, alpha=100.0):
    """Per-token adaptive regulariser of one layer.

    [SwiAttn] section 2, adaptive regulariser paragraph: the loss of token t
    is gamma_t * softplus(R(h_t)) with the weight
    gamma_t = gamma_base / (eps + NLL(t) + alpha * ||o_FULL - o_SWA||^2),
    and the hyperparameters gamma_base = 1e-3, eps = 0.1, alpha = 100.

    z     [B,N,G]  router logits R(h_t) (the values route() thresholds)
    nll   [B,N]    the token's negative log-likelihood (an input here)
    diff  [B,N]    ||o_FULL - o_SWA||^2 of the token (prefill's both-branch
                   output: summed over heads and channels)
    Returns L [B,N,G] float64.

    Reading: with G > 1 gate groups (the pages have one router per token)
    every group's logit is weighted by the token's gamma, which uses the
    distance summed over all heads.  The pages' loss is this value per token
    and layer; how it is reduced over tokens and layers is not part of it.
    """
    z = np.asarray(z, np.float64)
    gamma = gamma_base / (eps + np.asarray(nll, np.float64) + alpha * np.asarray(diff, np.float64))
    return gamma[..., None] * softplus(z)


# ---------------------------------------------------------------------------
# Router gradient through the straight-through gate  ([SwiAttn] section 2,
# router and dual-branch paragraphs)
# ---------------------------------------------------------------------------
def router_backward(dO, O_full, O_swa, z, H, r):
    """Gradient of the loss with respect to the router's logits, hidden
    states, weight and bias, given the gradient dO of the layer output.

    [SwiAttn] section 2: the hard gate is sigma = 1(soft > 0.5) + soft -
    sg(soft) with soft = sigmoid(z), so its value is the 0/1 indicator and
    its derivative is d soft / dz = soft * (1 - soft); the output is
    O = sigma * O_FULL + (1 - sigma) * O_SWA, so dL/dsigma is the inner
    product of dO with O_FULL - O_SWA over the heads the gate multiplies
    and their channels.  With z = H.r + bias (route()):
      dz[b,t,g]  = soft(1 - soft) * sum_{h in g} sum_c dO (O_FULL - O_SWA)
      dH[b,t,k]  = sum_g dz[b,t,g] r[k,g]
      dr[k,g]    = sum_{b,t} H[b,t,k] dz[b,t,g]
      dbias[g]   = sum_{b,t} dz[b,t,g]
    Only the router's path is covered: the gradients that reach Q, K, V
    through O_FULL and O_SWA are not part of this function.

    dO, O_full, O_swa [B,N,Hq,d]; z [B,N,G]; H [B,N,hidden]; r [hidden,G]
    ->  dict dz [B,N,G], dH [B,N,hidden], dr [hidden,G], dbias [G]  (float64)
    Reading: query head h belongs to gate group h // (Hq/G), as everywhere.
    """
    dO = np.asarray(dO, np.float64)
    diff = np.asarray(O_full, np.float64) - np.asarray(O_swa, np.float64)
    z = np.asarray(z, np.float64)
    H = np.asarray(H, np.float64)
    r = np.asarray(r, np.float64)
    B, N, Hq, d = dO.shape
    G = z.shape[2]
    if Hq % G:
        raise ValueError("Hq must be a multiple of G")
    hg = Hq // G
    per_head = (dO * diff).sum(axis=3)                          # [B,N,Hq]
    s = per_head.reshape(B, N, G, hg).sum(axis=3)               # [B,N,G]
    # soft * (1 - soft) written as e^-|z| / (1 + e^-|z|)^2 (the same
    # function): in the tails 1 - soft cancels to a few significant digits
    u = np.exp(-np.abs(z))
    dz = s * (u / ((1.0 + u) * (1.0 + u)))
    dH = dz @ r.T                                               # [B,N,hidden]
    dr = np.einsum("btk,btg->kg", H, dz)
    dbias = dz.sum(axis=(0, 1))
    return {"dz": dz, "dH": dH, "dr": dr, "dbias": dbias}


# ---------------------------------------------------------------------------
# Attention backward of the hard-gated layer  ([SwiAttn] section 2: the
# gated output O = sigma * O_FULL + (1 - sigma) * O_SWA with a 0/1 forward
# gate, so each row's output is one softmax attention over its own key set)
# ---------------------------------------------------------------------------
def prefill_backward_rows(Q, K, V, gate, W, dO, rows, scale=None):
    """dQ of prefill_backward for the given token positions only (row i's
    dQ depends on row i alone): dQ [B,R,Hq,d] float64.  The same steps
    per row, over row i's own key set."""
    Q = np.asarray(Q)
    K = np.asarray(K)
    V = np.asarray(V)
    dO = np.asarray(dO)
    gate = np.asarray(gate)
    B, N, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = gate.shape[2]
    hk, hg = _head_maps(Hq, Hkv, G)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.asarray(rows, np.int64)
    dQ = np.zeros((B, rows.size, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kv, g = h // hk, h // hg
            for r, i in enumerate(rows):
                lo, hi = full_key_range(int(i)) if gate[b, i, g] else swa_key_range(int(i), W)
                k = np.asarray(K[b, lo:hi + 1, kv], np.float64)
                v = np.asarray(V[b, lo:hi + 1, kv], np.float64)
                q = np.asarray(Q[b, i, h], np.float64)
                go = np.asarray(dO[b, i, h], np.float64)
                s = scale * (k @ q)
                p = np.exp(s - s.max())
                p /= p.sum()
                dp = v @ go
                ds = p * (dp - go @ (p @ v))
                dQ[b, r, h] = scale * (ds @ k)
    return dQ


def prefill_backward_keys(Q, K, V, gate, W, dO, keys, kv_heads=None, scale=None):
    """dK, dV of prefill_backward for the given key positions only:
    dK_j = scale * sum_i dS_ij q_i and dV_j = sum_i P_ij dO_i over the rows i
    that see key j (i >= j, and i - j < W or gate 1), summed over the query
    heads of the KV head.  P_ij and D_i = <dO_i, O_i> need row i's whole key
    set; those row quantities are formed for blocks of rows with one masked
    matrix product each (a library matmul; each row masked to its own key
    set) and reused across keys.

    -> dict dK, dV [B,R,len(kv_heads),d] float64 (kv_heads: the KV heads to
    evaluate, all by default)."""
    Q = np.asarray(Q)
    K = np.asarray(K)
    V = np.asarray(V)
    dO = np.asarray(dO)
    gate = np.asarray(gate)
    B, N, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = gate.shape[2]
    hk, hg = _head_maps(Hq, Hkv, G)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    keys = np.asarray(keys, np.int64)
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    dK = np.zeros((B, keys.size, len(kv_heads), d))
    dV = np.zeros((B, keys.size, len(kv_heads), d))
    for b in range(B):
        for c, kv in enumerate(kv_heads):
            Kf = np.asarray(K[b, :, kv], np.float64)
            Vf = np.asarray(V[b, :, kv], np.float64)
            for h in range(kv * hk, (kv + 1) * hk):
                g = h // hg
                Qh = np.asarray(Q[b, :, h], np.float64)
                dOh = np.asarray(dO[b, :, h], np.float64)
                # the rows that see each key
                sees = []
                for j in keys:
                    i = np.arange(int(j), N)
                    sees.append(i[(i - j < W) | (gate[b, i, g] != 0)])
                need = np.unique(np.concatenate(sees))
                # log-normaliser and D of every needed row, over its own key set
                lse = np.zeros(N)
                Drow = np.zeros(N)
                for i0 in range(0, need.size, 256):
                    rows = need[i0:i0 + 256]
                    lo = np.array([(full_key_range(int(i)) if gate[b, i, g] else swa_key_range(int(i), W))[0]
                                   for i in rows])
                    a, e = int(lo.min()), int(rows.max()) + 1
                    S = scale * (Qh[rows] @ Kf[a:e].T)
                    cols = np.arange(a, e)
                    S[(cols[None, :] < lo[:, None]) | (cols[None, :] > rows[:, None])] = -np.inf
                    mx = S.max(axis=1, keepdims=True)
                    Pn = np.exp(S - mx)
                    tot = Pn.sum(axis=1, keepdims=True)
                    lse[rows] = (mx + np.log(tot))[:, 0]
                    O = (Pn / tot) @ Vf[a:e]
                    Drow[rows] = (dOh[rows] * O).sum(axis=1)
                for r, j in enumerate(keys):
                    i = sees[r]
                    p = np.exp(scale * (Qh[i] @ Kf[j]) - lse[i])
                    ds = p * (dOh[i] @ Vf[j] - Drow[i])
                    dK[b, r, c] += scale * (ds @ Qh[i])
                    dV[b, r, c] += p @ dOh[i]
    return {"dK": dK, "dV": dV}


def prefill_backward(Q, K, V, gate, W, dO, scale=None):
    """Gradients of L = sum(dO * O) with respect to Q, K, V for the routed
    prefill (hard gate: row i of a head in gate group g attends to [0, i]
    if gate[b,i,g] else [max(0, i-W+1), i]).

    With s_ij = scale * <q_i, k_j> over row i's key set S_i,
    P_ij = exp(s_ij) / sum_{j' in S_i} exp(s_ij'), O_i = sum_j P_ij v_j:
      dV_j = sum_i P_ij dO_i
      dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
      dQ_i = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i
    where sum_j' P_ij' dP_ij' = <dO_i, O_i>.  K and V gradients add over the
    query heads that share a KV head.  The gate's own gradient (through the
    straight-through estimator) is router_backward's.

    Q, dO [B,N,Hq,d]; K, V [B,N,Hkv,d]; gate [B,N,G]
    ->  dict dQ [B,N,Hq,d], dK, dV [B,N,Hkv,d]  (float64)
    Each (b, h) is evaluated with explicit [N, N] matrices: small N only.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    gate = np.asarray(gate)
    B, N, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = gate.shape[2]
    hk, hg = _head_maps(Hq, Hkv, G)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    full_mask = j <= i
    band_mask = full_mask & (j > i - W)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(Hq):
            kv, g = h // hk, h // hg
            sig = gate[b, :, g].astype(bool)[:, None]
            mask = np.where(sig, full_mask, band_mask)
            s = scale * (Q[b, :, h] @ K[b, :, kv].T)
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            P = np.exp(s)
            P /= P.sum(axis=1, keepdims=True)
            O = P @ V[b, :, kv]
            dP = dO[b, :, h] @ V[b, :, kv].T
            Dr = (dO[b, :, h] * O).sum(axis=1, keepdims=True)
            dS = P * (dP - Dr)
            dQ[b, :, h] = scale * (dS @ K[b, :, kv])
            dK[b, :, kv] += scale * (dS.T @ Q[b, :, h])
            dV[b, :, kv] += P.T @ dO[b, :, h]
    return {"dQ": dQ, "dK": dK, "dV": dV}

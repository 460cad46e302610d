"""Plant plausible mistakes in a copy of the CPU reference and show that the
pins catch each one.  Mistakes are planted on the CPU only."""
import numpy as np
import pytest

import oracle.swiattn_ref as ref
from tests import pins

_attend = ref.attend_rows


def _attend_no_scale(q, K, V, lo, hi, scale, lo2=None, hi2=None):
    return _attend(q, K, V, lo, hi, 1.0, lo2, hi2)


def _attend_transposed_kv(q, K, V, lo, hi, scale, lo2=None, hi2=None):
    return _attend(q, V, K, lo, hi, scale, lo2, hi2)


def _attend_unnormalised(q, K, V, lo, hi, scale, lo2=None, hi2=None):
    O, lse = _attend(q, K, V, lo, hi, scale, lo2, hi2)
    n = (np.asarray(hi) - np.asarray(lo) + 1)[:, None]
    return O * n, lse


def _attend_drop_last_key(q, K, V, lo, hi, scale, lo2=None, hi2=None):
    hi = np.asarray(hi)
    lo = np.asarray(lo)
    return _attend(q, K, V, lo, np.maximum(lo, hi - 1), scale, lo2, hi2)


MUTANTS = {
    # the explanatory example on the SWA introduction page counts one key too many
    "window_one_key_too_many": ("swa_key_range", lambda i, W: (max(0, i - W), i)),
    "window_excludes_self": ("swa_key_range", lambda i, W: (max(0, i - W), max(0, i - 1))),
    # reading the glossary's "all N keys" literally (non-causal full branch)
    "full_branch_not_causal": ("full_key_range", lambda i: (0, i + 1)),
    "full_branch_is_window": ("full_key_range", lambda i: (max(0, i - 3), i)),
    "missing_softmax_scale": ("attend_rows", _attend_no_scale),
    "k_and_v_swapped": ("attend_rows", _attend_transposed_kv),
    "unnormalised_weights": ("attend_rows", _attend_unnormalised),
    "drops_newest_key": ("attend_rows", _attend_drop_last_key),
    # anchors not cut at the window start: early rows see future anchor keys
    "anchors_not_causal": ("anchor_key_range", lambda i, W, A: (0, A - 1)),
    # one anchor key too many
    "anchors_one_too_many": ("anchor_key_range",
                             lambda i, W, A: (0, min(A, max(0, i - W + 1)) - (0 if A else 1))),
    # anchors that slide with the window (the A keys before it, not the first A)
    "anchors_slide": ("anchor_key_range",
                      lambda i, W, A: (max(0, i - W + 1 - A), max(0, i - W + 1) - 1)),
    # anchors ignored altogether
    "anchors_ignored": ("anchor_key_range", lambda i, W, A: (0, -1)),
    # window offset ignored (every layer a plain window)
    "offset_ignored": ("offset_window_key_range", lambda i, W, o: ref.swa_key_range(i, W)),
    # window moved forward instead of back (sees keys past the query)
    "offset_forward": ("offset_window_key_range", lambda i, W, o: ref.swa_key_range(i + o, W)),
    # one position too far back
    "offset_one_too_far": ("offset_window_key_range", lambda i, W, o: ref.swa_key_range(i - o - 1, W)),
    # the shifted window's start with the keys up to the query kept
    "offset_runs_to_query": ("offset_window_key_range", lambda i, W, o: (max(0, i - o - W + 1), i)),
    # the shift applied as a window of W + o keys ending at the query
    "offset_widens_window": ("offset_window_key_range", lambda i, W, o: ref.swa_key_range(i, W + o)),
}


def _run_all_pins():
    failures = 0
    for check in pins.ALL_PINS:
        try:
            check()
        except (AssertionError, IndexError, ValueError):
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    assert _run_all_pins() > 0, f"no pin caught the planted mistake {name}"


def test_router_mutants_caught(monkeypatch):
    real = ref.route

    def sign_flip(H, r, bias):
        out = real(H, r, bias)
        out["gate"] = (out["soft"] < 0.5).astype(np.uint8)
        return out

    def non_strict(H, r, bias):
        out = real(H, r, bias)
        out["gate"] = (out["soft"] >= 0.5).astype(np.uint8)
        return out

    for m in (sign_flip, non_strict):
        monkeypatch.setattr(ref, "route", m)
        with pytest.raises(AssertionError):
            pins.check_router_closed_form()


def test_regularizer_mutants_caught(monkeypatch):
    def alpha_on_nll(z, nll, diff, gamma_base=1e-3, eps=0.1, alpha=100.0):
        g = gamma_base / (eps + alpha * np.asarray(nll) + np.asarray(diff))
        return g[..., None] * ref.softplus(z)

    def no_eps(z, nll, diff, gamma_base=1e-3, eps=0.1, alpha=100.0):
        g = gamma_base / (np.asarray(nll) + alpha * np.asarray(diff))
        return g[..., None] * ref.softplus(z)

    def sigmoid_not_softplus(z, nll, diff, gamma_base=1e-3, eps=0.1, alpha=100.0):
        g = gamma_base / (eps + np.asarray(nll) + alpha * np.asarray(diff))
        return g[..., None] / (1.0 + np.exp(-np.asarray(z, np.float64)))

    def gamma_multiplies(z, nll, diff, gamma_base=1e-3, eps=0.1, alpha=100.0):
        g = gamma_base * (eps + np.asarray(nll) + alpha * np.asarray(diff))
        return g[..., None] * ref.softplus(z)

    def naive_softplus(x):
        with np.errstate(over="ignore"):
            return np.log(1.0 + np.exp(np.asarray(x, np.float64)))

    for m in (alpha_on_nll, no_eps, sigmoid_not_softplus, gamma_multiplies):
        monkeypatch.setattr(ref, "regularizer", m)
        assert _run_all_pins() > 0, m.__name__
    monkeypatch.undo()
    monkeypatch.setattr(ref, "softplus", naive_softplus)
    assert _run_all_pins() > 0, "naive softplus"


def test_decode_step_mutants_caught(monkeypatch):
    real_decode, real_route = ref.decode, ref.route

    def step_with(append_at, grow, route_row=0):
        def step(Hn, r, bias, q, k, v, Kc, Vc, cache_len, W, scale=None):
            Hn = np.asarray(Hn)
            rt = real_route(np.roll(Hn, route_row, axis=0)[:, None, :], r, bias)
            gate = rt["gate"][:, 0, :]
            Kc, Vc = np.array(Kc, copy=True), np.array(Vc, copy=True)
            L = np.array(cache_len, dtype=np.int64, copy=True)
            for b in range(L.shape[0]):
                if L[b] < Kc.shape[1]:
                    p = min(max(append_at(L[b]), 0), Kc.shape[1] - 1)
                    Kc[b, p], Vc[b, p] = k[b], v[b]
                    L[b] += grow
            Ld = np.maximum(L, 1)
            out = real_decode(q, Kc, Vc, Ld, gate, W, scale)
            return {"gate": gate, "z": rt["z"][:, 0, :], "Kc": Kc, "Vc": Vc, "cache_len": L,
                    "o": out["o"], "lse": out["lse"]}
        return step

    mutants = {
        "append_one_past": step_with(lambda L: L + 1, 1),
        "append_over_last": step_with(lambda L: L - 1, 1),
        "no_length_growth": step_with(lambda L: L, 0),
        "routes_other_token": step_with(lambda L: L, 1, route_row=1),
    }
    for name, m in mutants.items():
        monkeypatch.setattr(ref, "decode_step", m)
        assert _run_all_pins() > 0, name


def test_router_backward_mutants_caught(monkeypatch):
    """Plausible mistakes in the router gradient, each caught by a pin."""
    good = ref.router_backward

    def make(kind):
        def mutant(dO, O_full, O_swa, z, H, r):
            dO = np.asarray(dO, np.float64)
            diff = np.asarray(O_full, np.float64) - np.asarray(O_swa, np.float64)
            if kind == "flipped_difference":
                diff = -diff
            z = np.asarray(z, np.float64)
            B, N, Hq, d = dO.shape
            G = z.shape[2]
            per_head = (dO * diff).sum(axis=3)
            if kind == "heads_interleaved":  # head h in group h % G
                s = per_head.reshape(B, N, Hq // G, G).sum(axis=2)
            else:
                s = per_head.reshape(B, N, G, Hq // G).sum(axis=3)
            soft = 1.0 / (1.0 + np.exp(-z))
            if kind == "no_sigmoid_derivative":
                dz = s
            elif kind == "sigmoid_not_derivative":
                dz = s * soft
            else:
                dz = s * soft * (1.0 - soft)
            out = good(dO, O_full, O_swa, z, H, r)
            out["dz"] = dz
            out["dH"] = dz @ np.asarray(r, np.float64).T
            out["dr"] = np.einsum("btk,btg->kg", np.asarray(H, np.float64), dz)
            out["dbias"] = dz.mean(axis=(0, 1)) if kind == "bias_mean" else dz.sum(axis=(0, 1))
            return out
        return mutant

    checks = [pins.check_router_backward_finite_differences, pins.check_router_backward_against_autograd,
              pins.check_router_backward_special_cases]
    for kind in ("flipped_difference", "heads_interleaved", "no_sigmoid_derivative",
                 "sigmoid_not_derivative", "bias_mean"):
        monkeypatch.setattr(ref, "router_backward", make(kind))
        caught = 0
        for c in checks:
            try:
                c()
            except AssertionError:
                caught += 1
        assert caught > 0, kind
    monkeypatch.setattr(ref, "router_backward", good)
    for c in checks:
        c()


def test_prefill_backward_mutants_caught(monkeypatch):
    """Plausible mistakes in the attention backward, each caught by a pin."""
    good = ref.prefill_backward

    def make(kind):
        def mutant(Q, K, V, gate, W, dO, scale=None):
            Q = np.asarray(Q, np.float64)
            K = np.asarray(K, np.float64)
            V = np.asarray(V, np.float64)
            dO = np.asarray(dO, np.float64)
            B, N, Hq, d = Q.shape
            Hkv, G = K.shape[2], np.asarray(gate).shape[2]
            if scale is None:
                scale = 1.0 / np.sqrt(d)
            i = np.arange(N)[:, None]
            j = np.arange(N)[None, :]
            dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
            for b in range(B):
                for h in range(Hq):
                    kv, g = h // (Hq // Hkv), h // (Hq // G)
                    sig = np.asarray(gate)[b, :, g].astype(bool)[:, None]
                    mask = np.where(sig, j <= i, (j <= i) & (j > i - W))
                    s = np.where(mask, scale * (Q[b, :, h] @ K[b, :, kv].T), -np.inf)
                    P = np.exp(s - s.max(axis=1, keepdims=True))
                    P /= P.sum(axis=1, keepdims=True)
                    dP = dO[b, :, h] @ V[b, :, kv].T
                    Dr = (dO[b, :, h] * (P @ V[b, :, kv])).sum(axis=1, keepdims=True)
                    dS = P * dP if kind == "no_row_term" else P * (dP - Dr)
                    sq = 1.0 if kind == "dq_unscaled" else scale
                    dQ[b, :, h] = sq * (dS @ K[b, :, kv])
                    if kind == "kv_overwritten":
                        dK[b, :, kv] = scale * (dS.T @ Q[b, :, h])
                        dV[b, :, kv] = P.T @ dO[b, :, h]
                    else:
                        dK[b, :, kv] += scale * (dS.T @ Q[b, :, h])
                        dV[b, :, kv] += (P.T if kind != "dv_untransposed" else P) @ dO[b, :, h]
            return {"dQ": dQ, "dK": dK, "dV": dV}
        return mutant

    checks = [pins.check_prefill_backward_finite_differences, pins.check_prefill_backward_against_autograd,
              pins.check_prefill_backward_special_cases]
    for kind in ("no_row_term", "dq_unscaled", "kv_overwritten", "dv_untransposed"):
        monkeypatch.setattr(ref, "prefill_backward", make(kind))
        caught = 0
        for c in checks:
            try:
                c()
            except AssertionError:
                caught += 1
        assert caught > 0, kind
    monkeypatch.setattr(ref, "prefill_backward", good)

"""C ABI checks that need no GPU: the library loads, exports every entry
point declared in include/swiattn.h, sizes workspaces, and rejects invalid
arguments with the documented codes before touching the device."""
import ctypes
import os
import re

import pytest

from sliding_window_attention_router_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "swiattn.h")
OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, TOO_LARGE = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from sliding_window_attention_router_amd import build

        build.build()
    return binding.lib()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swiattn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("swiattn_route", "swiattn_prefill", "swiattn_decode", "swiattn_prefill_workspace_size",
              "swiattn_decode_workspace_size", "swiattn_strerror", "swiattn_prefill_ex", "swiattn_decode_ex",
              "swiattn_regularizer", "swiattn_decode_step", "swiattn_prefill_anchored",
              "swiattn_decode_anchored"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SYMBOLS, f"{name} missing from the binding's table"


def test_strerror_and_version(lib):
    assert binding.strerror(OK) == "ok"
    for c in (INVALID, UNSUPPORTED, WORKSPACE, HIP, TOO_LARGE):
        assert binding.strerror(c) not in ("ok", "unknown error code")
    assert binding.strerror(-99) == "unknown error code"
    assert lib.swiattn_version().decode().count(".") == 2


def test_workspace_sizes(lib):
    # valid shapes give a positive size; invalid ones give 0
    assert lib.swiattn_prefill_workspace_size(1, 32768, 16, 4, 1, 128, 1024, BF16, 0) > 0
    # both-branch mode runs the hard-gate stages over every row (a larger
    # far schedule) and adds the per-(head, token) distances
    hard = lib.swiattn_prefill_workspace_size(1, 32768, 16, 16, 1, 128, 1024, BF16, 0)
    both = lib.swiattn_prefill_workspace_size(1, 32768, 16, 16, 1, 128, 1024, BF16, 1)
    assert both >= hard + 4 * 16 * 32768
    assert lib.swiattn_prefill_workspace_size(0, 10, 2, 2, 1, 64, 4, BF16, 0) == 0
    assert lib.swiattn_prefill_workspace_size(1, 10, 2, 2, 1, 96, 4, BF16, 0) == 0
    assert lib.swiattn_decode_workspace_size(64, 32768, 16, 4, 1, 128, 1024, BF16) > 0
    assert lib.swiattn_decode_workspace_size(64, 32768, 16, 5, 1, 128, 1024, BF16) == 0
    # the size does not depend on the scale or the gate; it grows with N
    a = lib.swiattn_prefill_workspace_size(1, 1000, 8, 2, 1, 128, 100, BF16, 0)
    b = lib.swiattn_prefill_workspace_size(1, 2000, 8, 2, 1, 128, 100, BF16, 0)
    assert 0 < a < b


def _prefill(lib, **kw):
    args = dict(Q=FAKE, K=FAKE, V=FAKE, gate=FAKE, idx=FAKE, cnt=FAKE, O=FAKE, diff=None,
                B=1, N=100, Hq=4, Hkv=2, G=1, d=128, W=16, scale=0.088, dt=BF16, flags=0,
                ws=FAKE, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    a = args
    return lib.swiattn_prefill(a["Q"], a["K"], a["V"], a["gate"], a["idx"], a["cnt"], a["O"], a["diff"],
                               a["B"], a["N"], a["Hq"], a["Hkv"], a["G"], a["d"], a["W"], a["scale"],
                               a["dt"], a["flags"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(W=0), INVALID), (dict(Hq=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(G=3), INVALID), (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=-1.0), INVALID), (dict(dt=7), INVALID),
    (dict(flags=2), INVALID), (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(Hq=64, Hkv=1), UNSUPPORTED),                 # 64 query heads per KV head
    (dict(Hq=12, Hkv=4, G=3), UNSUPPORTED),            # 3 heads per KV head, 4 per gate group
    (dict(Hq=12, Hkv=3, G=3), OK),                     # 4 and 4 nest
    (dict(Q=None), INVALID), (dict(K=None), INVALID), (dict(V=None), INVALID),
    (dict(gate=None), INVALID), (dict(O=None), INVALID), (dict(idx=None), INVALID),
    (dict(cnt=None), INVALID), (dict(flags=1, diff=None), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
])
def test_prefill_rejects_invalid_arguments(lib, kw, code):
    if code == OK:
        # a valid shape: only check that it is accepted by the size query
        assert lib.swiattn_prefill_workspace_size(1, 100, kw["Hq"], kw["Hkv"], kw["G"], 128, 16, BF16, 0) > 0
        return
    assert _prefill(lib, **kw) == code


def _decode(lib, **kw):
    a = dict(q=FAKE, Kc=FAKE, Vc=FAKE, lens=FAKE, gate=FAKE, o=FAKE, B=4, Lmax=100, Hq=4, Hkv=2, G=1,
             d=128, W=16, scale=0.088, dt=BF16, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.swiattn_decode(a["q"], a["Kc"], a["Vc"], a["lens"], a["gate"], a["o"], a["B"], a["Lmax"],
                              a["Hq"], a["Hkv"], a["G"], a["d"], a["W"], a["scale"], a["dt"], a["ws"],
                              a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(Lmax=0), INVALID), (dict(W=0), INVALID), (dict(Hkv=3), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(q=None), INVALID), (dict(lens=None), INVALID),
    (dict(gate=None), INVALID), (dict(o=None), INVALID), (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=8), WORKSPACE), (dict(scale=0.0), INVALID),
])
def test_decode_rejects_invalid_arguments(lib, kw, code):
    assert _decode(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(G=0), dict(gate=None), dict(idx=None),
                                dict(cnt=None), dict(r=None), dict(bias=None), dict(hidden=0), dict(dt=5)])
def test_route_rejects_invalid_arguments(lib, kw):
    a = dict(H=FAKE, r=FAKE, bias=FAKE, gate=FAKE, z=None, idx=FAKE, cnt=FAKE, B=1, N=10, hidden=64, G=1,
             dt=BF16, stream=None)
    a.update(kw)
    rc = lib.swiattn_route(a["H"], a["r"], a["bias"], a["gate"], a["z"], a["idx"], a["cnt"], a["B"], a["N"],
                           a["hidden"], a["G"], a["dt"], a["stream"])
    assert rc == INVALID


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(G=0), dict(z=None), dict(nll=None), dict(diff=None),
                                dict(loss=None), dict(eps=0.0), dict(eps=-1.0), dict(alpha=-1.0),
                                dict(eps=float("nan")), dict(alpha=float("inf")), dict(gamma_base=float("nan"))])
def test_regularizer_rejects_invalid_arguments(lib, kw):
    a = dict(z=FAKE, nll=FAKE, diff=FAKE, loss=FAKE, B=1, N=10, G=1, gamma_base=1e-3, eps=0.1, alpha=100.0,
             stream=None)
    a.update(kw)
    rc = lib.swiattn_regularizer(a["z"], a["nll"], a["diff"], a["loss"], a["B"], a["N"], a["G"],
                                 a["gamma_base"], a["eps"], a["alpha"], a["stream"])
    assert rc == INVALID


@pytest.mark.parametrize("kw,code", [(dict(B=0), INVALID), (dict(hidden=0), INVALID), (dict(Hn=None), INVALID),
                                     (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(cache_len=None), INVALID),
                                     (dict(gate=None), INVALID), (dict(d=96), UNSUPPORTED), (dict(ws=None), WORKSPACE)])
def test_decode_step_rejects_invalid_arguments(lib, kw, code):
    a = dict(Hn=FAKE, r=FAKE, bias=FAKE, q=FAKE, k=FAKE, v=FAKE, Kc=FAKE, Vc=FAKE, cache_len=FAKE, gate=FAKE,
             o=FAKE, B=2, Lmax=100, hidden=64, Hq=4, Hkv=2, G=1, d=128, W=16, scale=0.1, dt=BF16, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    rc = lib.swiattn_decode_step(a["Hn"], a["r"], a["bias"], a["q"], a["k"], a["v"], a["Kc"], a["Vc"],
                                 a["cache_len"], a["gate"], a["o"], a["B"], a["Lmax"], a["hidden"], a["Hq"],
                                 a["Hkv"], a["G"], a["d"], a["W"], a["scale"], a["dt"], a["ws"], a["ws_bytes"],
                                 a["stream"])
    assert rc == code


def _prefill_anchored(lib, anchors, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, gate=FAKE, idx=FAKE, cnt=FAKE, O=FAKE, diff=None,
             B=1, N=100, Hq=4, Hkv=2, G=1, d=128, W=16, scale=0.088, dt=BF16, flags=0,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.swiattn_prefill_anchored(a["Q"], a["K"], a["V"], a["gate"], a["idx"], a["cnt"], a["O"],
                                        a["diff"], a["B"], a["N"], a["Hq"], a["Hkv"], a["G"], a["d"],
                                        a["W"], anchors, a["scale"], a["dt"], a["flags"], a["ws"],
                                        a["ws_bytes"], a["stream"], None)


def _decode_anchored(lib, anchors, **kw):
    a = dict(q=FAKE, Kc=FAKE, Vc=FAKE, lens=FAKE, gate=FAKE, o=FAKE, B=4, Lmax=100, Hq=4, Hkv=2, G=1,
             d=128, W=16, scale=0.088, dt=BF16, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.swiattn_decode_anchored(a["q"], a["Kc"], a["Vc"], a["lens"], a["gate"], a["o"], a["B"],
                                       a["Lmax"], a["Hq"], a["Hkv"], a["G"], a["d"], a["W"], anchors,
                                       a["scale"], a["dt"], a["ws"], a["ws_bytes"], a["stream"], None)


@pytest.mark.parametrize("anchors,kw,code", [
    (-1, {}, INVALID), (-256, {}, INVALID),
    (256, dict(N=0), INVALID), (256, dict(d=96), UNSUPPORTED), (256, dict(Q=None), INVALID),
    (256, dict(ws=None), WORKSPACE), (256, dict(flags=1, diff=None), INVALID),
])
def test_prefill_anchored_rejects_invalid_arguments(lib, anchors, kw, code):
    assert _prefill_anchored(lib, anchors, **kw) == code


@pytest.mark.parametrize("anchors,kw,code", [
    (-1, {}, INVALID), (256, dict(Lmax=0), INVALID), (256, dict(d=32), UNSUPPORTED),
    (256, dict(lens=None), INVALID), (256, dict(ws_bytes=8), WORKSPACE),
])
def test_decode_anchored_rejects_invalid_arguments(lib, anchors, kw, code):
    assert _decode_anchored(lib, anchors, **kw) == code


def _router_backward(lib, **kw):
    a = dict(dO=FAKE, Of=FAKE, Os=FAKE, z=FAKE, H=FAKE, r=FAKE, dz=FAKE, dH=FAKE, dr=FAKE, db=FAKE,
             B=1, N=100, Hq=16, d=128, hidden=2048, G=1, dt=BF16, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.swiattn_router_backward(a["dO"], a["Of"], a["Os"], a["z"], a["H"], a["r"], a["dz"], a["dH"],
                                       a["dr"], a["db"], a["B"], a["N"], a["Hq"], a["d"], a["hidden"], a["G"],
                                       a["dt"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(Hq=0), INVALID), (dict(hidden=0), INVALID),
    (dict(G=0), INVALID), (dict(G=3), INVALID), (dict(dt=9), INVALID), (dict(dO=None), INVALID),
    (dict(z=None), INVALID), (dict(db=None), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(hidden=100), UNSUPPORTED), (dict(Hq=128, G=128), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=64), WORKSPACE),
])
def test_router_backward_rejects_invalid_arguments(lib, kw, code):
    assert _router_backward(lib, **kw) == code


def test_router_backward_workspace_size(lib):
    # one float per (split of 32 tokens, group, hidden unit + bias)
    assert lib.swiattn_router_backward_workspace_size(1, 32768, 2048, 1) == 1024 * 2049 * 4
    assert lib.swiattn_router_backward_workspace_size(2, 33, 8, 2) == 3 * 2 * 9 * 4
    assert lib.swiattn_router_backward_workspace_size(0, 10, 8, 1) == 0


def test_decode_step_anchored_rejects_negative_anchors(lib):
    rc = lib.swiattn_decode_step_anchored(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          4, 100, 64, 4, 2, 1, 128, 16, -1, 0.088, BF16, FAKE, 1 << 40, None)
    assert rc == INVALID
    rc = lib.swiattn_decode_step_anchored(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          4, 100, 64, 4, 2, 1, 96, 16, 8, 0.088, BF16, FAKE, 1 << 40, None)
    assert rc == UNSUPPORTED


def test_prefill_backward_rejects_invalid_arguments(lib):
    def call(**kw):
        a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, gate=FAKE, idx=FAKE, cnt=FAKE, dQ=FAKE, dK=FAKE,
                 dV=FAKE, B=1, N=100, Hq=4, Hkv=2, G=1, d=128, W=16, scale=0.088, dt=BF16, ws=FAKE,
                 ws_bytes=1 << 40, stream=None)
        a.update(kw)
        return lib.swiattn_prefill_backward(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["gate"], a["idx"],
                                            a["cnt"], a["dQ"], a["dK"], a["dV"], a["B"], a["N"], a["Hq"],
                                            a["Hkv"], a["G"], a["d"], a["W"], a["scale"], a["dt"], a["ws"],
                                            a["ws_bytes"], a["stream"])
    for kw, code in ((dict(B=0), INVALID), (dict(N=0), INVALID), (dict(W=0), INVALID),
                     (dict(Hq=6, Hkv=4), INVALID), (dict(scale=0.0), INVALID), (dict(O=None), INVALID),
                     (dict(dO=None), INVALID), (dict(idx=None), INVALID), (dict(dV=None), INVALID),
                     (dict(d=96), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE)):
        assert call(**kw) == code, kw
    # two floats (log-sum-exp, <dO, O>) per (sequence, query head, token)
    assert lib.swiattn_prefill_backward_workspace_size(2, 100, 4) == 2 * 2 * 4 * 100 * 4
    assert lib.swiattn_prefill_backward_workspace_size(0, 100, 4) == 0


def test_decode_noalloc_validates_before_touching_the_device(lib):
    """The allocation-free decode checks its arguments and that the decode
    plan fits its fixed scratch before any HIP call."""
    scratch = lib.swiattn_decode_noalloc_scratch_bytes()
    assert scratch == 16 << 20

    def call(**kw):
        a = dict(B=64, Lmax=32768, Hq=16, Hkv=4, G=1, d=128, W=1024, scale=0.088, dt=BF16, q=FAKE)
        a.update(kw)
        return lib.swiattn_decode_noalloc(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["Lmax"], a["Hq"],
                                          a["Hkv"], a["G"], a["d"], a["W"], a["scale"], a["dt"], None)

    assert call(q=None) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(scale=-1.0) == INVALID
    # 32 query heads per KV head at d=128: 32 MiB of split-K partials
    assert lib.swiattn_decode_workspace_size(64, 32768, 32, 1, 1, 128, 1024, BF16) > scratch
    assert call(Hq=32, Hkv=1) == TOO_LARGE
    # the bench's decode shape fits
    assert lib.swiattn_decode_workspace_size(64, 32768, 16, 4, 1, 128, 1024, BF16) <= scratch


def test_offset_entry_points_validate(lib):
    """Window offsets: negative offsets are rejected, both-branch mode with
    an offset is unsupported (checked before any HIP call)."""
    args = (FAKE,) * 8
    rc = lib.swiattn_prefill_offset(*args, 1, 100, 4, 2, 1, 128, 16, 0, -1, 0.088, BF16, 0, FAKE, 1 << 40,
                                    None, None)
    assert rc == INVALID
    rc = lib.swiattn_prefill_offset(*args, 1, 100, 4, 2, 1, 128, 16, 0, 8, 0.088, BF16, 1, FAKE, 1 << 40,
                                    None, None)
    assert rc == UNSUPPORTED
    rc = lib.swiattn_decode_offset(*(FAKE,) * 6, 2, 100, 4, 2, 1, 128, 16, 0, -3, 0.088, BF16, FAKE,
                                   1 << 40, None, None)
    assert rc == INVALID

"""ctypes binding of libswiattn.so.

Argument marshalling only: shapes and dtypes are checked, torch tensors are
turned into device pointers and the current HIP stream, and every step of
the computation runs in the library's kernels.  Torch provides device memory
and streams, nothing else.  There is no fallback: if the library is missing
or a call fails, a SwiAttnError is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

__all__ = [
    "SwiAttnError",
    "lib",
    "route",
    "regularizer",
    "prefill",
    "prefill_branches",
    "decode",
    "decode_step",
    "decode_noalloc",
    "prefill_workspace_size",
    "decode_workspace_size",
    "strerror",
    "SYMBOLS",
    "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswiattn.so")
FLAG_BOTH_BRANCH = 1
_DTYPES = {torch.bfloat16: 0, torch.float32: 1}

_vp, _i32, _u32, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_float, ctypes.c_size_t
# exported symbol -> (restype, argtypes); mirrors include/swiattn.h
SYMBOLS = {
    "swiattn_route": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]),
    "swiattn_prefill_workspace_size": (_sz, [_i32] * 8 + [_u32]),
    "swiattn_prefill": (_i32, [_vp] * 8 + [_i32] * 7 + [_f32, _i32, _u32, _vp, _sz, _vp]),
    "swiattn_decode_workspace_size": (_sz, [_i32] * 8),
    "swiattn_decode": (_i32, [_vp] * 6 + [_i32] * 7 + [_f32, _i32, _vp, _sz, _vp]),
    "swiattn_prefill_ex": (_i32, [_vp] * 8 + [_i32] * 7 + [_f32, _i32, _u32, _vp, _sz, _vp, _vp]),
    "swiattn_decode_ex": (_i32, [_vp] * 6 + [_i32] * 7 + [_f32, _i32, _vp, _sz, _vp, _vp]),
    "swiattn_regularizer": (_i32, [_vp] * 4 + [_i32] * 3 + [_f32] * 3 + [_vp]),
    "swiattn_decode_step": (_i32, [_vp] * 11 + [_i32] * 8 + [_f32, _i32, _vp, _sz, _vp]),
    "swiattn_prefill_anchored": (_i32, [_vp] * 8 + [_i32] * 8 + [_f32, _i32, _u32, _vp, _sz, _vp, _vp]),
    "swiattn_decode_anchored": (_i32, [_vp] * 6 + [_i32] * 8 + [_f32, _i32, _vp, _sz, _vp, _vp]),
    "swiattn_decode_step_anchored": (_i32, [_vp] * 11 + [_i32] * 9 + [_f32, _i32, _vp, _sz, _vp]),
    "swiattn_prefill_branches": (_i32, [_vp] * 8 + [_i32] * 8 + [_f32, _i32, _vp, _sz, _vp, _vp]),
    "swiattn_prefill_offset": (_i32, [_vp] * 8 + [_i32] * 9 + [_f32, _i32, _u32, _vp, _sz, _vp, _vp]),
    "swiattn_decode_offset": (_i32, [_vp] * 6 + [_i32] * 9 + [_f32, _i32, _vp, _sz, _vp, _vp]),
    "swiattn_router_backward_workspace_size": (_sz, [_i32] * 4),
    "swiattn_prefill_backward_workspace_size": (_sz, [_i32] * 3),
    "swiattn_prefill_backward": (_i32, [_vp] * 11 + [_i32] * 7 + [_f32, _i32, _vp, _sz, _vp]),
    "swiattn_router_backward": (_i32, [_vp] * 10 + [_i32] * 7 + [_vp, _sz, _vp]),
    "swiattn_decode_noalloc": (_i32, [_vp] * 6 + [_i32] * 7 + [_f32, _i32, _vp]),
    "swiattn_decode_noalloc_scratch_bytes": (_sz, []),
    "swiattn_strerror": (ctypes.c_char_p, [_i32]),
    "swiattn_version": (ctypes.c_char_p, []),
}


class SwiAttnError(RuntimeError):
    pass


class _Events(ctypes.Structure):
    _fields_ = [("ev", ctypes.c_void_p * 6)]


def _events(events):
    """List of up to six torch.cuda.Event (or None) -> swiattn_events_t*.
    Each event must have been recorded once so that it exists."""
    if events is None:
        return None
    st = _Events()
    for i, e in enumerate(events):
        if e is not None:
            if not e.cuda_event:
                raise ValueError("record each event once before passing it (torch creates events lazily)")
            st.ev[i] = e.cuda_event
    return ctypes.byref(st)


_lib = None
_lock = threading.Lock()


def lib():
    """Load libswiattn.so (once).  Raises SwiAttnError if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise SwiAttnError(
                    f"{LIB_PATH} is not built; run `python -m sliding_window_attention_router_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SYMBOLS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def strerror(code):
    return lib().swiattn_strerror(int(code)).decode()


def _check(rc, what):
    if rc != 0:
        raise SwiAttnError(f"{what} failed: {strerror(rc)} (code {rc})")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")
    return _DTYPES[t.dtype]


def _need(t, name, shape=None, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def route(H=None, r=None, bias=None, *, gate=None, want_z=False, out=None):
    """Router logits, hard gate and compaction.

    H [B,N,hidden], r [hidden,G] (bf16 or fp32), bias [G] fp32 -> gate.
    Pass H=None and gate=[B,N,G] uint8 to only compact a given gate.
    Returns (gate uint8 [B,N,G], idx int32 [B,G,N], cnt int32 [B,G], z or None).
    out: optional (gate, idx, cnt) tensors to write into.
    """
    L = lib()
    if H is None:
        _need(gate, "gate", dtype=torch.uint8)
        B, N, G = gate.shape
        dev, hidden, code = gate.device, 0, 0
        z = None
    else:
        _need(H, "H")
        code = _dtype_code(H)
        B, N, hidden = H.shape
        dev = H.device
        _need(r, "r", dtype=H.dtype, device=dev)
        if r.dim() != 2 or r.shape[0] != hidden:
            raise ValueError("r must be [hidden, G]")
        G = r.shape[1]
        _need(bias, "bias", shape=(G,), dtype=torch.float32, device=dev)
        gate = out[0] if out is not None else torch.empty((B, N, G), dtype=torch.uint8, device=dev)
        _need(gate, "gate", shape=(B, N, G), dtype=torch.uint8, device=dev)
        z = torch.empty((B, N, G), dtype=torch.float32, device=dev) if want_z else None
    if out is not None:
        idx, cnt = out[1], out[2]
        _need(idx, "idx", shape=(B, G, N), dtype=torch.int32, device=dev)
        _need(cnt, "cnt", shape=(B, G), dtype=torch.int32, device=dev)
    else:
        idx = torch.empty((B, G, N), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, G), dtype=torch.int32, device=dev)
    rc = L.swiattn_route(_p(H), _p(r), _p(bias), _p(gate), _p(z), _p(idx), _p(cnt),
                         B, N, hidden, G, code, _stream(dev))
    _check(rc, "swiattn_route")
    return gate, idx, cnt, z


def regularizer(z, nll, diff, *, gamma_base=1e-3, eps=0.1, alpha=100.0, out=None):
    """Adaptive regulariser per token: gamma_base / (eps + nll + alpha*diff)
    * softplus(z).  z [B,N,G] (router logits), nll [B,N], diff [B,N] (the
    both-branch distance), all float32 on one device.  Returns loss [B,N,G]."""
    _need(z, "z", dtype=torch.float32)
    B, N, G = z.shape
    dev = z.device
    _need(nll, "nll", shape=(B, N), dtype=torch.float32, device=dev)
    _need(diff, "diff", shape=(B, N), dtype=torch.float32, device=dev)
    loss = out if out is not None else torch.empty((B, N, G), dtype=torch.float32, device=dev)
    _need(loss, "loss", shape=(B, N, G), dtype=torch.float32, device=dev)
    rc = lib().swiattn_regularizer(_p(z), _p(nll), _p(diff), _p(loss), B, N, G, float(gamma_base),
                                   float(eps), float(alpha), _stream(dev))
    _check(rc, "swiattn_regularizer")
    return loss


def prefill_backward(Q, K, V, O, dO, gate, W, *, idx=None, cnt=None, scale=None, out=None,
                     workspace=None):
    """Attention backward of the hard-gated prefill: gradients of
    sum(dO * O) w.r.t. Q, K, V.  Q, O, dO [B,N,Hq,d]; K, V [B,N,Hkv,d];
    gate [B,N,G] (idx, cnt from route(); computed here if not given).
    Returns (dQ, dK, dV)."""
    L = lib()
    _need(Q, "Q")
    code = _dtype_code(Q)
    B, N, Hq, d = Q.shape
    dev = Q.device
    _need(K, "K", dtype=Q.dtype, device=dev)
    if K.dim() != 4 or K.shape[0] != B or K.shape[1] != N or K.shape[3] != d:
        raise ValueError("K must be [B,N,Hkv,d]")
    Hkv = K.shape[2]
    _need(V, "V", shape=K.shape, dtype=Q.dtype, device=dev)
    _need(O, "O", shape=Q.shape, dtype=Q.dtype, device=dev)
    _need(dO, "dO", shape=Q.shape, dtype=Q.dtype, device=dev)
    _need(gate, "gate", dtype=torch.uint8, device=dev)
    if gate.dim() != 3 or gate.shape[:2] != (B, N):
        raise ValueError("gate must be [B,N,G]")
    G = gate.shape[2]
    if idx is None or cnt is None:
        _, idx, cnt, _ = route(None, gate=gate)
    _need(idx, "idx", shape=(B, G, N), dtype=torch.int32, device=dev)
    _need(cnt, "cnt", shape=(B, G), dtype=torch.int32, device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = out
    _need(dQ, "dQ", shape=Q.shape, dtype=Q.dtype, device=dev)
    _need(dK, "dK", shape=K.shape, dtype=Q.dtype, device=dev)
    _need(dV, "dV", shape=K.shape, dtype=Q.dtype, device=dev)
    nbytes = int(L.swiattn_prefill_backward_workspace_size(B, N, Hq))
    ws = _workspace(nbytes, dev, workspace)
    rc = L.swiattn_prefill_backward(_p(Q), _p(K), _p(V), _p(O), _p(dO), _p(gate), _p(idx), _p(cnt),
                                    _p(dQ), _p(dK), _p(dV), B, N, Hq, Hkv, G, d, W, float(scale), code,
                                    _p(ws), ws.numel(), _stream(dev))
    _check(rc, "swiattn_prefill_backward")
    return dQ, dK, dV


def router_backward(dO, O_full, O_swa, z, H, r, *, out=None, workspace=None):
    """Router gradient through the straight-through gate.  dO, O_full, O_swa
    [B,N,Hq,d]; z [B,N,G] float32 (router logits); H [B,N,hidden]; r
    [hidden,G] (dO, O_*, H, r in one dtype).  Returns (dz [B,N,G] fp32,
    dH [B,N,hidden] dtype, dr [hidden,G] fp32, dbias [G] fp32); `out` may
    give those four tensors."""
    L = lib()
    _need(dO, "dO")
    code = _dtype_code(dO)
    B, N, Hq, d = dO.shape
    dev = dO.device
    _need(O_full, "O_full", shape=dO.shape, dtype=dO.dtype, device=dev)
    _need(O_swa, "O_swa", shape=dO.shape, dtype=dO.dtype, device=dev)
    _need(z, "z", dtype=torch.float32, device=dev)
    if z.dim() != 3 or z.shape[:2] != (B, N):
        raise ValueError("z must be [B,N,G]")
    G = z.shape[2]
    _need(H, "H", dtype=dO.dtype, device=dev)
    if H.dim() != 3 or H.shape[:2] != (B, N):
        raise ValueError("H must be [B,N,hidden]")
    hidden = H.shape[2]
    _need(r, "r", shape=(hidden, G), dtype=dO.dtype, device=dev)
    if out is None:
        out = (torch.empty((B, N, G), dtype=torch.float32, device=dev),
               torch.empty((B, N, hidden), dtype=dO.dtype, device=dev),
               torch.empty((hidden, G), dtype=torch.float32, device=dev),
               torch.empty((G,), dtype=torch.float32, device=dev))
    dz, dH, dr, dbias = out
    _need(dz, "dz", shape=(B, N, G), dtype=torch.float32, device=dev)
    _need(dH, "dH", shape=(B, N, hidden), dtype=dO.dtype, device=dev)
    _need(dr, "dr", shape=(hidden, G), dtype=torch.float32, device=dev)
    _need(dbias, "dbias", shape=(G,), dtype=torch.float32, device=dev)
    nbytes = int(L.swiattn_router_backward_workspace_size(B, N, hidden, G))
    ws = _workspace(nbytes, dev, workspace)
    rc = L.swiattn_router_backward(_p(dO), _p(O_full), _p(O_swa), _p(z), _p(H), _p(r), _p(dz), _p(dH),
                                   _p(dr), _p(dbias), B, N, Hq, d, hidden, G, code, _p(ws), ws.numel(),
                                   _stream(dev))
    _check(rc, "swiattn_router_backward")
    return dz, dH, dr, dbias


def prefill_workspace_size(B, N, Hq, Hkv, G, d, W, dtype=torch.bfloat16, both_branch=False):
    return int(lib().swiattn_prefill_workspace_size(B, N, Hq, Hkv, G, d, W, _DTYPES[dtype],
                                                    FLAG_BOTH_BRANCH if both_branch else 0))


def decode_workspace_size(B, Lmax, Hq, Hkv, G, d, W, dtype=torch.bfloat16):
    return int(lib().swiattn_decode_workspace_size(B, Lmax, Hq, Hkv, G, d, W, _DTYPES[dtype]))


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        raise SwiAttnError("invalid sizes (workspace size query returned 0)")
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    _need(workspace, "workspace", dtype=torch.uint8, device=device)
    return workspace


def prefill(Q, K, V, gate, W, *, idx=None, cnt=None, scale=None, both_branch=False,
            out=None, diff=None, workspace=None, events=None, anchors=0, offset=0):
    """Dual-branch prefill.  Q [B,N,Hq,d], K/V [B,N,Hkv,d], gate [B,N,G] uint8.
    anchors: global anchor keys of the window branch (swiattn_prefill_anchored);
    offset: window offset of the layer (swiattn_prefill_offset); both 0 calls
    swiattn_prefill_ex.

    In hard-gate mode the compacted positions (idx, cnt) from route() are
    used, or computed here by the library's compaction if not given.
    Returns (O [B,N,Hq,d], diff [B,N] fp32 or None).
    events: optional torch.cuda.Event list recorded at the stage boundaries
    documented for swiattn_prefill_ex.
    """
    L = lib()
    _need(Q, "Q")
    code = _dtype_code(Q)
    B, N, Hq, d = Q.shape
    dev = Q.device
    _need(K, "K", dtype=Q.dtype, device=dev)
    if K.dim() != 4 or K.shape[0] != B or K.shape[1] != N or K.shape[3] != d:
        raise ValueError("K must be [B,N,Hkv,d]")
    Hkv = K.shape[2]
    _need(V, "V", shape=K.shape, dtype=Q.dtype, device=dev)
    _need(gate, "gate", dtype=torch.uint8, device=dev)
    if gate.dim() != 3 or gate.shape[:2] != (B, N):
        raise ValueError("gate must be [B,N,G]")
    G = gate.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not both_branch and (idx is None or cnt is None):
        _, idx, cnt, _ = route(None, gate=gate)
    if not both_branch:
        _need(idx, "idx", shape=(B, G, N), dtype=torch.int32, device=dev)
        _need(cnt, "cnt", shape=(B, G), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(Q)
    _need(out, "out", shape=Q.shape, dtype=Q.dtype, device=dev)
    if both_branch:
        if diff is None:
            diff = torch.empty((B, N), dtype=torch.float32, device=dev)
        _need(diff, "diff", shape=(B, N), dtype=torch.float32, device=dev)
    else:
        diff = None
    flags = FLAG_BOTH_BRANCH if both_branch else 0
    nbytes = int(L.swiattn_prefill_workspace_size(B, N, Hq, Hkv, G, d, W, code, flags))
    ws = _workspace(nbytes, dev, workspace)
    ptrs = (_p(Q), _p(K), _p(V), _p(gate), _p(idx if not both_branch else None),
            _p(cnt if not both_branch else None), _p(out), _p(diff))
    if offset:
        rc = L.swiattn_prefill_offset(*ptrs, B, N, Hq, Hkv, G, d, W, int(anchors), int(offset),
                                      float(scale), code, flags, _p(ws), ws.numel(), _stream(dev),
                                      _events(events))
    elif anchors:
        rc = L.swiattn_prefill_anchored(*ptrs, B, N, Hq, Hkv, G, d, W, int(anchors), float(scale),
                                        code, flags, _p(ws), ws.numel(), _stream(dev),
                                        _events(events))
    else:
        rc = L.swiattn_prefill_ex(*ptrs, B, N, Hq, Hkv, G, d, W, float(scale), code, flags,
                                  _p(ws), ws.numel(), _stream(dev), _events(events))
    _check(rc, "swiattn_prefill")
    return out, diff


def prefill_branches(Q, K, V, gate, W, *, scale=None, anchors=0, out=None, workspace=None, events=None):
    """Both-branch prefill that also returns the branch outputs
    (swiattn_prefill_branches).  Returns (O, diff, O_full, O_swa); out, if
    given, is that tuple of preallocated tensors."""
    L = lib()
    _need(Q, "Q")
    code = _dtype_code(Q)
    B, N, Hq, d = Q.shape
    dev = Q.device
    _need(K, "K", dtype=Q.dtype, device=dev)
    if K.dim() != 4 or K.shape[0] != B or K.shape[1] != N or K.shape[3] != d:
        raise ValueError("K must be [B,N,Hkv,d]")
    Hkv = K.shape[2]
    _need(V, "V", shape=K.shape, dtype=Q.dtype, device=dev)
    _need(gate, "gate", dtype=torch.uint8, device=dev)
    if gate.dim() != 3 or gate.shape[:2] != (B, N):
        raise ValueError("gate must be [B,N,G]")
    G = gate.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = (torch.empty_like(Q), torch.empty((B, N), dtype=torch.float32, device=dev), torch.empty_like(Q),
               torch.empty_like(Q))
    O, diff, Of, Os = out
    for t, name in ((O, "O"), (Of, "O_full"), (Os, "O_swa")):
        _need(t, name, shape=Q.shape, dtype=Q.dtype, device=dev)
    _need(diff, "diff", shape=(B, N), dtype=torch.float32, device=dev)
    nbytes = int(L.swiattn_prefill_workspace_size(B, N, Hq, Hkv, G, d, W, code, FLAG_BOTH_BRANCH))
    ws = _workspace(nbytes, dev, workspace)
    rc = L.swiattn_prefill_branches(_p(Q), _p(K), _p(V), _p(gate), _p(O), _p(diff), _p(Of), _p(Os), B, N, Hq,
                                    Hkv, G, d, W, int(anchors), float(scale), code, _p(ws), ws.numel(),
                                    _stream(dev), _events(events))
    _check(rc, "swiattn_prefill_branches")
    return O, diff, Of, Os


def decode(q, Kc, Vc, cache_len, gate, W, *, scale=None, out=None, workspace=None, events=None,
           anchors=0, offset=0):
    """Routed decode.  q [B,Hq,d], Kc/Vc [B,Lmax,Hkv,d], cache_len int32 [B],
    gate uint8 [B,G].  Returns o [B,Hq,d].  events: as for prefill, recorded
    at the stage boundaries documented for swiattn_decode_ex.  anchors: global
    anchor keys of the window branch (swiattn_decode_anchored); offset: window
    offset of the layer (swiattn_decode_offset); both 0 calls
    swiattn_decode_ex."""
    L = lib()
    _need(q, "q")
    code = _dtype_code(q)
    B, Hq, d = q.shape
    dev = q.device
    _need(Kc, "Kc", dtype=q.dtype, device=dev)
    if Kc.dim() != 4 or Kc.shape[0] != B or Kc.shape[3] != d:
        raise ValueError("Kc must be [B,Lmax,Hkv,d]")
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    _need(Vc, "Vc", shape=Kc.shape, dtype=q.dtype, device=dev)
    _need(cache_len, "cache_len", shape=(B,), dtype=torch.int32, device=dev)
    _need(gate, "gate", dtype=torch.uint8, device=dev)
    if gate.dim() != 2 or gate.shape[0] != B:
        raise ValueError("gate must be [B,G]")
    G = gate.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", shape=q.shape, dtype=q.dtype, device=dev)
    nbytes = int(L.swiattn_decode_workspace_size(B, Lmax, Hq, Hkv, G, d, W, code))
    ws = _workspace(nbytes, dev, workspace)
    ptrs = (_p(q), _p(Kc), _p(Vc), _p(cache_len), _p(gate), _p(out))
    if offset:
        rc = L.swiattn_decode_offset(*ptrs, B, Lmax, Hq, Hkv, G, d, W, int(anchors), int(offset),
                                     float(scale), code, _p(ws), ws.numel(), _stream(dev),
                                     _events(events))
    elif anchors:
        rc = L.swiattn_decode_anchored(*ptrs, B, Lmax, Hq, Hkv, G, d, W, int(anchors), float(scale),
                                       code, _p(ws), ws.numel(), _stream(dev), _events(events))
    else:
        rc = L.swiattn_decode_ex(*ptrs, B, Lmax, Hq, Hkv, G, d, W, float(scale), code, _p(ws),
                                 ws.numel(), _stream(dev), _events(events))
    _check(rc, "swiattn_decode")
    return out


def decode_noalloc(q, Kc, Vc, cache_len, gate, W, *, scale=None, out=None):
    """Routed decode through swiattn_decode_noalloc: the same arguments and
    result as decode(), with the split-K workspace in the library's fixed
    per-GPU scratch (no workspace tensor).  Calls that overlap on one GPU
    race on that scratch."""
    L = lib()
    _need(q, "q")
    code = _dtype_code(q)
    B, Hq, d = q.shape
    dev = q.device
    _need(Kc, "Kc", dtype=q.dtype, device=dev)
    if Kc.dim() != 4 or Kc.shape[0] != B or Kc.shape[3] != d:
        raise ValueError("Kc must be [B,Lmax,Hkv,d]")
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    _need(Vc, "Vc", shape=Kc.shape, dtype=q.dtype, device=dev)
    _need(cache_len, "cache_len", shape=(B,), dtype=torch.int32, device=dev)
    _need(gate, "gate", dtype=torch.uint8, device=dev)
    if gate.dim() != 2 or gate.shape[0] != B:
        raise ValueError("gate must be [B,G]")
    G = gate.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", shape=q.shape, dtype=q.dtype, device=dev)
    rc = L.swiattn_decode_noalloc(_p(q), _p(Kc), _p(Vc), _p(cache_len), _p(gate), _p(out), B, Lmax, Hq,
                                  Hkv, G, d, W, float(scale), code, _stream(dev))
    _check(rc, "swiattn_decode_noalloc")
    return out


def decode_step(Hn, r, bias, q, k, v, Kc, Vc, cache_len, W, *, scale=None, gate=None, out=None,
                workspace=None, anchors=0):
    """One serving step: route the new tokens (Hn [B,hidden], r [hidden,G],
    bias [G] fp32), append k, v [B,Hkv,d] to the cache Kc/Vc [B,Lmax,Hkv,d]
    at position cache_len[b] (int32 [B], advanced in place), then decode q
    [B,Hq,d] over the updated cache.  Returns (o [B,Hq,d], gate uint8 [B,G]).
    anchors: global anchor keys of the window branch
    (swiattn_decode_step_anchored); 0 calls swiattn_decode_step."""
    L = lib()
    _need(q, "q")
    code = _dtype_code(q)
    B, Hq, d = q.shape
    dev = q.device
    _need(Hn, "Hn", dtype=q.dtype, device=dev)
    if Hn.dim() != 2 or Hn.shape[0] != B:
        raise ValueError("Hn must be [B,hidden]")
    hidden = Hn.shape[1]
    _need(r, "r", dtype=q.dtype, device=dev)
    if r.dim() != 2 or r.shape[0] != hidden:
        raise ValueError("r must be [hidden,G]")
    G = r.shape[1]
    _need(bias, "bias", shape=(G,), dtype=torch.float32, device=dev)
    _need(Kc, "Kc", dtype=q.dtype, device=dev)
    if Kc.dim() != 4 or Kc.shape[0] != B or Kc.shape[3] != d:
        raise ValueError("Kc must be [B,Lmax,Hkv,d]")
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    _need(Vc, "Vc", shape=Kc.shape, dtype=q.dtype, device=dev)
    _need(k, "k", shape=(B, Hkv, d), dtype=q.dtype, device=dev)
    _need(v, "v", shape=(B, Hkv, d), dtype=q.dtype, device=dev)
    _need(cache_len, "cache_len", shape=(B,), dtype=torch.int32, device=dev)
    if gate is None:
        gate = torch.empty((B, G), dtype=torch.uint8, device=dev)
    _need(gate, "gate", shape=(B, G), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", shape=q.shape, dtype=q.dtype, device=dev)
    nbytes = int(L.swiattn_decode_workspace_size(B, Lmax, Hq, Hkv, G, d, W, code))
    ws = _workspace(nbytes, dev, workspace)
    ptrs = (_p(Hn), _p(r), _p(bias), _p(q), _p(k), _p(v), _p(Kc), _p(Vc), _p(cache_len), _p(gate),
            _p(out))
    if anchors:
        rc = L.swiattn_decode_step_anchored(*ptrs, B, Lmax, hidden, Hq, Hkv, G, d, W, int(anchors),
                                            float(scale), code, _p(ws), ws.numel(), _stream(dev))
    else:
        rc = L.swiattn_decode_step(*ptrs, B, Lmax, hidden, Hq, Hkv, G, d, W, float(scale), code,
                                   _p(ws), ws.numel(), _stream(dev))
    _check(rc, "swiattn_decode_step")
    return out, gate

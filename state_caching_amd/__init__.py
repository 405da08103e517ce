"""Python binding of libhypic (gfx950): linear-attention state caching.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; torch supplies device memory and the current stream.  The three
entry points mirror the C ABI in include/hypic.h:

  segment_build(...) -> (T, S0)   cached pairs of segments
  compose(...)       -> S         fold pairs (and seam windows) into a state
  seam_advance(...)               advance states over seam windows

The library must be built (``python -m state_caching_amd.build``); importing
this module on a machine without it raises, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhypic.so")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_DEVICE, E_TOO_LARGE = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
RULE_DECAY, RULE_DELTA = 0, 1
GATE_HEAD_CONST, GATE_SCALAR, GATE_DIAG = 0, 1, 2
T_SCALAR, T_DIAG, T_DENSE = 0, 1, 2
PREC_FP32, PREC_SPLIT = 0, 1
WS_BUILD, WS_COMPOSE = 0, 1
MAX_SEG_PER_LAUNCH = 128
NOALLOC_SCRATCH_BYTES = 64 << 20   # static scratch of hypic_compose_noalloc

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_pi64 = ctypes.POINTER(ctypes.c_int64)
_pi32 = ctypes.POINTER(ctypes.c_int32)


class BuildDesc(ctypes.Structure):
    _fields_ = [("rule", _i32), ("gate_kind", _i32), ("in_dtype", _i32), ("n_seg", _i32),
                ("seg_start", _pi64), ("seg_len", _pi64),
                ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32),
                ("k", _vp), ("v", _vp), ("beta", _vp), ("gate", _vp),
                ("conv_w", _i32), ("k_l2norm", _i32), ("conv_from", _pi64),
                ("conv_wk", _vp), ("conv_wv", _vp), ("T_out", _vp), ("S0_out", _vp)]


class SeamDesc(ctypes.Structure):
    _fields_ = [("rule", _i32), ("in_dtype", _i32), ("w", _i32), ("conv_w", _i32),
                ("k_l2norm", _i32), ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32),
                ("n_win", _i32),
                ("xk", _vp), ("xv", _vp), ("tail_k", _vp), ("tail_v", _vp),
                ("conv_wk", _vp), ("conv_wv", _vp), ("beta", _vp), ("alpha", _vp),
                ("q", _vp), ("o", _vp), ("T_w", _vp), ("S_w0", _vp), ("gate_diag", _i32)]


class RopeDesc(ctypes.Structure):
    _fields_ = [("n_seg", _i32), ("seg_start", _pi64), ("seg_len", _pi64), ("delta", _pi64),
                ("h", _i32), ("d", _i32), ("rot_dim", _i32), ("pairing", _i32), ("dtype", _i32),
                ("base", ctypes.c_double), ("x_in", _vp), ("x_out", _vp)]


class ComposeDesc(ctypes.Structure):
    _fields_ = [("tform", _i32), ("prec", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32),
                ("n", _i32), ("n_slots", _i32), ("order", _pi32),
                ("T_pool", _vp), ("S0_pool", _vp), ("S_init", _vp), ("S_out", _vp),
                ("seams", ctypes.POINTER(SeamDesc)), ("group_len", _i32)]


class HypicError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({_lib().hypic_status_string(status).decode()})")
        self.status = status


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m state_caching_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.hypic_segment_build.argtypes = [ctypes.POINTER(BuildDesc), _vp, ctypes.c_size_t, _vp]
        lib.hypic_segment_build.restype = ctypes.c_int
        lib.hypic_compose.argtypes = [ctypes.POINTER(ComposeDesc), _vp, ctypes.c_size_t, _vp]
        lib.hypic_compose.restype = ctypes.c_int
        lib.hypic_compose_noalloc.argtypes = [ctypes.POINTER(ComposeDesc), _vp]
        lib.hypic_compose_noalloc.restype = ctypes.c_int
        lib.hypic_seam_advance.argtypes = [ctypes.POINTER(SeamDesc), _vp, _vp]
        lib.hypic_seam_advance.restype = ctypes.c_int
        lib.hypic_rope_rerotate.argtypes = [ctypes.POINTER(RopeDesc), _vp]
        lib.hypic_rope_rerotate.restype = ctypes.c_int
        lib.hypic_rope_rerotate_state.argtypes = [_i32, _i32, _i32, _i32, _i32, ctypes.c_double,
                                                  ctypes.c_int64, _vp, _vp, _vp]
        lib.hypic_rope_rerotate_state.restype = ctypes.c_int
        lib.hypic_workspace_size.argtypes = [_vp, ctypes.c_int]
        lib.hypic_workspace_size.restype = ctypes.c_size_t
        lib.hypic_status_string.argtypes = [ctypes.c_int]
        lib.hypic_status_string.restype = ctypes.c_char_p
        lib.hypic_version.restype = ctypes.c_int32
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises ImportError when not built)."""
    return _lib()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhypic must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != OK:
        raise HypicError(status, what)


def _i64_array(vals: Sequence[int]):
    arr = (ctypes.c_int64 * max(1, len(vals)))(*[int(x) for x in vals])
    return arr


def tform_of(rule: int, gate_kind: int) -> int:
    if rule == RULE_DELTA:
        return T_DENSE
    return T_DIAG if gate_kind == GATE_DIAG else T_SCALAR


def t_shape(tform: int, n: int, h_v: int, d_k: int):
    return {T_SCALAR: (n, h_v), T_DIAG: (n, h_v, d_k), T_DENSE: (n, h_v, d_k, d_k)}[tform]


def segment_build(rule: int, gate_kind: int, k: torch.Tensor, v: torch.Tensor,
                  beta: Optional[torch.Tensor], gate: torch.Tensor,
                  seg_start: Sequence[int], seg_len: Sequence[int],
                  conv_w: int = 0, conv_wk: Optional[torch.Tensor] = None,
                  conv_wv: Optional[torch.Tensor] = None,
                  conv_from: Optional[Sequence[int]] = None, k_l2norm: int = 0,
                  T_out: Optional[torch.Tensor] = None, S0_out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None):
    """Cached pairs (T_C, S_{C|0}) of the token ranges [seg_start[s], +seg_len[s]).

    k [N, h_k, d], v [N, h_v, d], beta [N, h_v], gate per gate_kind, on one
    CUDA device; returns (T, S0) fp32 tensors (T in scalar/diag/dense form).
    """
    n_seg = len(seg_len)
    N, h_k, d_k = k.shape
    _, h_v, d_v = v.shape
    dev = k.device
    # host-side bounds: every row a kernel reads must exist in the tensors
    if len(seg_start) != n_seg or v.shape[0] != N:
        raise ValueError("segment tables and token arrays disagree")
    for s0, ln in zip(seg_start, seg_len):
        if s0 < 0 or ln < 0 or s0 + ln > N:
            raise ValueError(f"token range [{s0}, {s0 + ln}) outside the {N} rows given")
    if beta is not None and tuple(beta.shape) != (N, h_v):
        raise ValueError("beta must be [N, h_v]")
    if gate_kind == GATE_SCALAR and tuple(gate.shape) != (N, h_v):
        raise ValueError("scalar gate must be [N, h_v]")
    if gate_kind == GATE_DIAG and tuple(gate.shape) != (N, h_v, d_k):
        raise ValueError("diagonal gate must be [N, h_v, d_k]")
    if gate_kind == GATE_HEAD_CONST and (tuple(gate.shape) != (h_v,) or gate.dtype != torch.float32):
        raise ValueError("per-head constant gate must be fp32 [h_v]")
    if conv_w > 0:
        if conv_from is None or len(conv_from) != n_seg or any(c < 0 for c in conv_from):
            raise ValueError("conv_from must list a non-negative first row per segment")
        if tuple(conv_wk.shape) != (h_k * d_k, conv_w) or tuple(conv_wv.shape) != (h_v * d_v, conv_w):
            raise ValueError("conv weights must be [h*d, conv_w]")
    for t in (k, v, beta, gate):
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on one device")
    tf = tform_of(rule, gate_kind)
    if T_out is None:
        T_out = torch.empty(t_shape(tf, n_seg, h_v, d_k), dtype=torch.float32, device=dev)
    if S0_out is None:
        S0_out = torch.empty((n_seg, h_v, d_k, d_v), dtype=torch.float32, device=dev)
    ss, sl = _i64_array(seg_start), _i64_array(seg_len)
    cf = _i64_array(conv_from) if conv_from is not None else None
    d = BuildDesc(rule=rule, gate_kind=gate_kind, in_dtype=_dtype_code(k), n_seg=n_seg,
                  seg_start=ctypes.cast(ss, _pi64), seg_len=ctypes.cast(sl, _pi64),
                  h_k=h_k, h_v=h_v, d_k=d_k, d_v=d_v,
                  k=_ptr(k), v=_ptr(v), beta=_ptr(beta), gate=_ptr(gate),
                  conv_w=conv_w, k_l2norm=k_l2norm,
                  conv_from=ctypes.cast(cf, _pi64) if cf is not None else None,
                  conv_wk=_ptr(conv_wk), conv_wv=_ptr(conv_wv),
                  T_out=_ptr(T_out), S0_out=_ptr(S0_out))
    L = _lib()
    need = L.hypic_workspace_size(ctypes.byref(d), WS_BUILD)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.hypic_segment_build(ctypes.byref(d), _ptr(workspace), wsz, _stream(stream)),
           "hypic_segment_build")
    return T_out, S0_out


@dataclass
class Seams:
    """Seam windows of the delta-rule family (see hypic.h for layouts)."""
    xk: torch.Tensor                       # [n_win, w, h_k, d]
    xv: torch.Tensor                       # [n_win, w, h_v, d]
    beta: torch.Tensor                     # [n_win, w, h_v]
    alpha: torch.Tensor                    # [n_win, w, h_v], or [n_win, w, h_v, d] (KDA)
    tail_k: Optional[torch.Tensor] = None  # [n_win, W-1, h_k, d]
    tail_v: Optional[torch.Tensor] = None  # [n_win, W-1, h_v, d]
    conv_wk: Optional[torch.Tensor] = None  # [h_k*d, W] fp32
    conv_wv: Optional[torch.Tensor] = None  # [h_v*d, W] fp32
    conv_w: int = 0
    k_l2norm: int = 0
    q: Optional[torch.Tensor] = None       # [n_win, w, h_k, d]
    o: Optional[torch.Tensor] = None       # [n_win, w, h_v, d] fp32
    T_w: Optional[torch.Tensor] = None     # [n_win, h_v, d, d] fp32
    S_w0: Optional[torch.Tensor] = None    # [n_win, h_v, d, d] fp32

    def desc(self) -> SeamDesc:
        n_win, w, h_k, d = self.xk.shape
        h_v = self.xv.shape[2]
        if tuple(self.xv.shape) != (n_win, w, h_v, d):
            raise ValueError("xv must be [n_win, w, h_v, d]")
        if tuple(self.beta.shape) != (n_win, w, h_v):
            raise ValueError("beta must be [n_win, w, h_v]")
        gate_diag = self.alpha.dim() == 4
        if tuple(self.alpha.shape) not in ((n_win, w, h_v), (n_win, w, h_v, d)):
            raise ValueError("alpha must be [n_win, w, h_v] or [n_win, w, h_v, d]")
        if self.conv_w > 1:
            if self.tail_k is None or tuple(self.tail_k.shape) != (n_win, self.conv_w - 1, h_k, d):
                raise ValueError("tail_k must be [n_win, conv_w-1, h_k, d]")
            if self.tail_v is None or tuple(self.tail_v.shape) != (n_win, self.conv_w - 1, h_v, d):
                raise ValueError("tail_v must be [n_win, conv_w-1, h_v, d]")
        if self.conv_w > 0:
            if tuple(self.conv_wk.shape) != (h_k * d, self.conv_w) or \
               tuple(self.conv_wv.shape) != (h_v * d, self.conv_w):
                raise ValueError("conv weights must be [h*d, conv_w]")
        if self.q is not None and tuple(self.q.shape) != (n_win, w, h_k, d):
            raise ValueError("q must be [n_win, w, h_k, d]")
        if self.o is not None and tuple(self.o.shape) != (n_win, w, h_v, d):
            raise ValueError("o must be [n_win, w, h_v, d]")
        for name in ("T_w", "S_w0"):
            t = getattr(self, name)
            if t is not None and tuple(t.shape) != (n_win, h_v, d, d):
                raise ValueError(f"{name} must be [n_win, h_v, d, d]")
        return SeamDesc(rule=RULE_DELTA, in_dtype=_dtype_code(self.xk), w=w, conv_w=self.conv_w,
                        k_l2norm=self.k_l2norm, h_k=h_k, h_v=h_v, d_k=d, d_v=d, n_win=n_win,
                        xk=_ptr(self.xk), xv=_ptr(self.xv), tail_k=_ptr(self.tail_k),
                        tail_v=_ptr(self.tail_v), conv_wk=_ptr(self.conv_wk),
                        conv_wv=_ptr(self.conv_wv), beta=_ptr(self.beta), alpha=_ptr(self.alpha),
                        q=_ptr(self.q), o=_ptr(self.o), T_w=_ptr(self.T_w), S_w0=_ptr(self.S_w0),
                        gate_diag=1 if gate_diag else 0)


def _compose_desc(T_pool, S0_pool, order, S_init, tform, prec, seams, S_out, group_len):
    """ComposeDesc for the pools and order (checked against each other), plus the
    ctypes objects it points to (kept alive by the caller)."""
    n_slots, h_v, d_k, d_v = S0_pool.shape
    if tuple(T_pool.shape) != t_shape(tform, n_slots, h_v, d_k):
        raise ValueError("T_pool shape does not match the transition form")
    if any(int(x) < 0 or int(x) >= n_slots for x in order):
        raise ValueError("order refers to a slot outside the pool")
    for t in (S_init, S_out):
        if t is not None and tuple(t.shape) != (h_v, d_k, d_v):
            raise ValueError("states must be [h_v, d_k, d_v]")
    if seams is not None and seams.xk.shape[0] != max(0, len(order) - 1):
        raise ValueError("compose needs one seam window per inner segment")
    n = len(order)
    ordr = (ctypes.c_int32 * max(1, n))(*[int(x) for x in order])
    sd = seams.desc() if seams is not None else None
    d = ComposeDesc(tform=tform, prec=prec, h_v=h_v, d_k=d_k, d_v=d_v, n=n, n_slots=n_slots,
                    order=ctypes.cast(ordr, _pi32), T_pool=_ptr(T_pool), S0_pool=_ptr(S0_pool),
                    S_init=_ptr(S_init), S_out=_ptr(S_out),
                    seams=ctypes.pointer(sd) if sd is not None else None, group_len=int(group_len))
    return d, (ordr, sd)


def compose_noalloc(T_pool: torch.Tensor, S0_pool: torch.Tensor, order: Sequence[int],
                    S_out: torch.Tensor, S_init: Optional[torch.Tensor] = None, tform: int = T_DENSE,
                    prec: int = PREC_SPLIT, seams: Optional[Seams] = None, stream=None,
                    group_len: int = 0):
    """compose() through hypic_compose_noalloc: the library's static scratch
    instead of a workspace, nothing allocated (S_out is the caller's)."""
    d, keep = _compose_desc(T_pool, S0_pool, order, S_init, tform, prec, seams, S_out, group_len)
    _check(_lib().hypic_compose_noalloc(ctypes.byref(d), _stream(stream)), "hypic_compose_noalloc")
    return S_out


def compose(T_pool: torch.Tensor, S0_pool: torch.Tensor, order: Sequence[int],
            S_init: Optional[torch.Tensor] = None, tform: int = T_DENSE, prec: int = PREC_SPLIT,
            seams: Optional[Seams] = None, S_out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, stream=None, group_len: int = 0):
    """S = fold_i (S <- T[order[i]] S + S0[order[i]]), seams before positions 1..

    group_len: 0 automatic, 1 serial fold, G >= 2 fold groups of G positions
    in parallel, then the group pairs in order (dense split compose only)."""
    n_slots, h_v, d_k, d_v = S0_pool.shape
    if S_out is None:
        S_out = torch.empty((h_v, d_k, d_v), dtype=torch.float32, device=S0_pool.device)
    d, keep = _compose_desc(T_pool, S0_pool, order, S_init, tform, prec, seams, S_out, group_len)
    L = _lib()
    need = L.hypic_workspace_size(ctypes.byref(d), WS_COMPOSE)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=S0_pool.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.hypic_compose(ctypes.byref(d), _ptr(workspace), wsz, _stream(stream)), "hypic_compose")
    return S_out


def seam_advance(S: torch.Tensor, seams: Seams, stream=None):
    """Advance S [h_v, d, d] (in place) over the windows of `seams`."""
    sd = seams.desc()
    if tuple(S.shape) != (sd.h_v, sd.d_k, sd.d_v) or S.dtype != torch.float32:
        raise ValueError("S must be fp32 [h_v, d, d]")
    _check(_lib().hypic_seam_advance(ctypes.byref(sd), _ptr(S), _stream(stream)),
           "hypic_seam_advance")
    return S


ROPE_HALF, ROPE_INTERLEAVED = 0, 1


def rope_rerotate(x: torch.Tensor, seg_start: Sequence[int], seg_len: Sequence[int],
                  delta: Sequence[int], rot_dim: Optional[int] = None, pairing: int = ROPE_HALF,
                  base: float = 10000.0, out: Optional[torch.Tensor] = None, stream=None):
    """Cached keys x [N, h, d] (fp32 or bf16) moved to new positions: rows of
    segment s turned by R(delta[s]) (hypic_rope_rerotate).  out=None: in place."""
    if x.dim() != 3:
        raise ValueError("x must be [N, h, d]")
    if out is None:
        out = x
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x")
    n = len(seg_start)
    if len(seg_len) != n or len(delta) != n:
        raise ValueError("seg_start, seg_len and delta must have one entry per segment")
    ss, sl, dl = _i64_array(seg_start), _i64_array(seg_len), _i64_array(delta)
    d = RopeDesc(n_seg=n, seg_start=ctypes.cast(ss, _pi64), seg_len=ctypes.cast(sl, _pi64),
                 delta=ctypes.cast(dl, _pi64), h=x.shape[1], d=x.shape[2],
                 rot_dim=x.shape[2] if rot_dim is None else int(rot_dim), pairing=int(pairing),
                 dtype=_dtype_code(x), base=float(base), x_in=_ptr(x), x_out=_ptr(out))
    _check(_lib().hypic_rope_rerotate(ctypes.byref(d), _stream(stream)), "hypic_rope_rerotate")
    return out


def rope_rerotate_state(S: torch.Tensor, delta: int, rot_dim: Optional[int] = None,
                        pairing: int = ROPE_HALF, base: float = 10000.0,
                        out: Optional[torch.Tensor] = None, stream=None):
    """States S [h, d_k, d_v] fp32 turned by R(delta) along d_k
    (hypic_rope_rerotate_state).  out=None: in place."""
    if S.dim() != 3 or S.dtype != torch.float32:
        raise ValueError("S must be fp32 [h, d_k, d_v]")
    if out is None:
        out = S
    h, d_k, d_v = S.shape
    _check(_lib().hypic_rope_rerotate_state(h, d_k, d_v, d_k if rot_dim is None else int(rot_dim),
                                            int(pairing), float(base), int(delta), _ptr(S), _ptr(out),
                                            _stream(stream)), "hypic_rope_rerotate_state")
    return out

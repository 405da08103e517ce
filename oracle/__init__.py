"""fp64 CPU oracle for linear-attention state caching (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of the benchmark, never by the library path.  It shares
no code with the GPU library; both read their inputs from ``synth``.

The arithmetic lives in ``oracle.c`` (plain C, double precision, token by
token).  This module only marshals numpy arrays into it and sequences the
steps the HYPIC reading notes describe:

* segment pair (T_C, S_{C|0}) by two runs of the recurrence (ch.2 secs.2, 4);
* composition S <- T_C S + S_{C|0} in prompt order (ch.2 sec.2, Eq. (6));
* seam window: the first w tokens of each inner segment are recomputed token
  by token from the running state before the body pair is applied
  (ch.2 sec.5, Figs. 7-8); the causal conv at a segment head reads the
  previous segment's last W-1 raw rows (ch.2 sec.6);
* full recompute: the recurrence over the whole concatenation, with the conv
  zero-padded only at the prompt start (the reference the composition must
  match, ch.2 sec.4);
* naive addition of zero-initial end states and its structural error
  (ch.1 sec.2, Eqs. (3)-(5), Table 2);
* rotary re-rotation of cached keys, K_b = R(b - a) K_a, and of the state of a
  scalar-transition layer, S_{C|b} = R(b - a) S_{C|a} (ch.2 sec.6, Eqs. (7)-(8)).

Readings of points the pages leave open are listed in the repository's
design notes; the ones that shape code here: GQA value head h reads key head
h // (h_v // h_k); the conv is y_t = sum_j w_j x_{t-(W-1)+j} with no bias and
no activation; keys are divided by their exact L2 norm (no epsilon).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DECAY, DELTA = 0, 1
GATE_SCALAR, GATE_DIAG = 0, 1


def build(force: bool = False, extra_flags=()) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               *extra_flags, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def compile_variant(out_path: str, defines=()) -> str:
    """Compile oracle.c to another path (used by the planted-mistake tests)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           *[f"-D{d}" for d in defines], _SRC, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


_P = ctypes.POINTER
_d = _P(ctypes.c_double)
_l = _P(ctypes.c_long)
_i = _P(ctypes.c_int)


class _Lib:
    def __init__(self, path):
        lib = ctypes.CDLL(path)
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_recur_batch.argtypes = [ctypes.c_int] * 5 + [
            _d, _l, ctypes.c_long,  # k
            _d, _l, ctypes.c_long,  # v
            _d, _l, ctypes.c_long,  # beta
            _d, _l, ctypes.c_long,  # g
            _d, _l, ctypes.c_long,  # q
            _d, _l, ctypes.c_long,  # o
            _i, _d]
        lib.orc_build_batch.argtypes = [ctypes.c_int] * 5 + [
            _d, _l, ctypes.c_long, _d, _l, ctypes.c_long, _d, _l, ctypes.c_long,
            _d, _l, ctypes.c_long, _i, _d, _d]
        lib.orc_apply_pair_batch.argtypes = [ctypes.c_int] * 3 + [_d, _d, _d]
        lib.orc_causal_conv.argtypes = [ctypes.c_int] * 3 + [
            _d, ctypes.c_long, _d, ctypes.c_long, _d, _d, ctypes.c_long]
        lib.orc_l2norm_rows.argtypes = [ctypes.c_long, ctypes.c_int, _d, ctypes.c_long]
        lib.orc_rope_rows.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_double, _d, _d]
        self.lib = lib


_lib_cache = {}


def lib(path: str | None = None) -> _Lib:
    path = path or build()
    if path not in _lib_cache:
        _lib_cache[path] = _Lib(path)
    return _lib_cache[path]


def threads() -> int:
    return int(lib().lib.orc_threads())


def set_threads(n: int) -> None:
    """Worker threads of the batched calls (OpenMP; 1 runs them serially)."""
    lib().lib.orc_set_threads(int(n))


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (any dtype): exact upcast
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _dp(a):
    return a.ctypes.data_as(_d) if a is not None else None


def _lp(a):
    return np.ascontiguousarray(a, dtype=np.int64).ctypes.data_as(_l)


def _code(rule, gate):
    r = DELTA if rule in ("delta", DELTA) else DECAY
    g = GATE_DIAG if gate in ("diag", GATE_DIAG) else GATE_SCALAR
    return r, g


# --------------------------------------------------------------------------
# low-level batched calls over (token range, head) units
# --------------------------------------------------------------------------

class Units:
    """Element offsets of token 0 of each unit in token-major arrays.

    ``units`` holds (start, end, key_slot, value_slot) tuples; arrays are
    k [N, nk, d_k], v [N, nv, d_v], beta [N, nv], g [N, nv] (scalar gate),
    [N, nv, d_k] (diagonal gate) or [nv] (one constant per head).
    """

    def __init__(self, units, nk, nv, d_k, d_v, gate_kind):
        self.n = len(units)
        ok, ov, ob, og, m = [], [], [], [], []
        for (s, e, kh, vh) in units:
            ok.append(s * nk * d_k + kh * d_k)
            ov.append(s * nv * d_v + vh * d_v)
            ob.append(s * nv + vh)
            if gate_kind == "diag":
                og.append(s * nv * d_k + vh * d_k)
            elif gate_kind == "scalar":
                og.append(s * nv + vh)
            else:
                og.append(vh)
            m.append(e - s)
        self.off_k = np.array(ok, np.int64)
        self.off_v = np.array(ov, np.int64)
        self.off_b = np.array(ob, np.int64)
        self.off_g = np.array(og, np.int64)
        self.m = np.array(m, np.int32)
        self.ldk, self.ldv, self.ldb = nk * d_k, nv * d_v, nv
        self.ldg = {"diag": nv * d_k, "scalar": nv}.get(gate_kind, 0)


def recur_units(rule, gate, u: Units, d_k, d_v, k, v, beta, g, S, q=None, o=None,
                off_q=None, ldq=0, off_o=None, ldo=0, path=None):
    """Run the recurrence for every unit from S[u] (modified in place)."""
    L = lib(path).lib
    r, gt = _code(rule, gate)
    zero = np.zeros(1)
    L.orc_recur_batch(r, gt, u.n, d_k, d_v,
                      _dp(k), _lp(u.off_k), u.ldk,
                      _dp(v) if v is not None else None, _lp(u.off_v), u.ldv,
                      _dp(beta) if beta is not None else _dp(zero), _lp(u.off_b),
                      u.ldb if beta is not None else 0,
                      _dp(g), _lp(u.off_g), u.ldg,
                      _dp(q), _lp(off_q if off_q is not None else [0] * u.n), ldq,
                      _dp(o), _lp(off_o if off_o is not None else [0] * u.n), ldo,
                      u.m.ctypes.data_as(_i), _dp(S))


def build_units(rule, gate, u: Units, d_k, d_v, k, v, beta, g, path=None):
    """(T_C, S_{C|0}) for every unit by the two-run construction."""
    L = lib(path).lib
    r, gt = _code(rule, gate)
    T = np.empty((u.n, d_k, d_k))
    S0 = np.empty((u.n, d_k, d_v))
    zero = np.zeros(1)
    L.orc_build_batch(r, gt, u.n, d_k, d_v,
                      _dp(k), _lp(u.off_k), u.ldk,
                      _dp(v), _lp(u.off_v), u.ldv,
                      _dp(beta) if beta is not None else _dp(zero), _lp(u.off_b),
                      u.ldb if beta is not None else 0,
                      _dp(g), _lp(u.off_g), u.ldg,
                      u.m.ctypes.data_as(_i), _dp(T), _dp(S0))
    return T, S0


def apply_pair(T, S0, S, path=None):
    """S <- T S + S0 per unit; T [n,dk,dk], S0 and S [n,dk,dv] (S in place)."""
    L = lib(path).lib
    n, dk, dv = S.shape
    L.orc_apply_pair_batch(n, dk, dv, _dp(T), _dp(S0), _dp(S))


def causal_conv(x, w, hist=None, path=None):
    """Depthwise causal conv: x [n, C], w [C, W], hist [W-1, C] or None."""
    L = lib(path).lib
    x = _f64(x)
    w = _f64(w)
    n, C = x.shape
    W = w.shape[1]
    y = np.empty((n, C))
    h = _f64(hist) if hist is not None else None
    L.orc_causal_conv(n, C, W, _dp(x), C, _dp(h), C, _dp(w), _dp(y), C)
    return y


def l2norm_rows(x, path=None):
    L = lib(path).lib
    x = np.array(x, dtype=np.float64, copy=True)
    shp = x.shape
    x2 = np.ascontiguousarray(x.reshape(-1, shp[-1]))
    L.orc_l2norm_rows(x2.shape[0], x2.shape[1], _dp(x2), x2.shape[1])
    return x2.reshape(shp)


def expand_dense(T, tform, d_k):
    """Dense d_k x d_k matrices from scalar [...] or diagonal [..., d_k] forms."""
    T = np.asarray(T, dtype=np.float64)
    if tform == "dense":
        return T
    if tform == "diag":
        out = np.zeros(T.shape + (d_k,))
        idx = np.arange(d_k)
        out[..., idx, idx] = T
        return out
    if tform == "scalar":
        return T[..., None, None] * np.eye(d_k)
    raise ValueError(tform)


# --------------------------------------------------------------------------
# workload-level sequencing
# --------------------------------------------------------------------------

class Slice:
    """fp64 inputs of a workload for tokens [start, end), restricted to some
    value heads (and the key heads they read).  Arrays are token-major:
    k [n, nk, d_k], v [n, nv, d_v], beta [n, nv], g per gate kind."""

    def __init__(self, wl, start, end, heads=None, conv_from=None, path=None):
        heads = list(range(wl.h_v)) if heads is None else list(heads)
        grp = wl.h_v // wl.h_k                     # GQA: value head h reads key head h // grp
        kheads = sorted({h // grp for h in heads})
        self.heads, self.kheads = heads, kheads
        self.kslot = [kheads.index(h // grp) for h in heads]
        self.n = end - start
        self.d_k, self.d_v = wl.d_k, wl.d_v
        self.gate_kind = wl.gate_kind
        if wl.conv_w > 0:
            self.k, self.v = _conv_inputs(wl, start, end, heads, kheads, conv_from, path)
        else:
            self.k = np.ascontiguousarray(_f64(wl.k[start:end])[:, kheads])
            self.v = np.ascontiguousarray(_f64(wl.v[start:end])[:, heads])
        self.beta = (np.ascontiguousarray(_f64(wl.beta[start:end])[:, heads])
                     if wl.beta is not None else None)
        if wl.gate_kind == "head_const":
            self.g = np.ascontiguousarray(_f64(wl.gate)[heads])
        else:
            self.g = np.ascontiguousarray(_f64(wl.gate[start:end])[:, heads])

    def units(self, ranges=None):
        ranges = [(0, self.n)] if ranges is None else ranges
        return Units([(s, e, self.kslot[i], i) for (s, e) in ranges
                      for i in range(len(self.heads))],
                     len(self.kheads), len(self.heads), self.d_k, self.d_v, self.gate_kind)


def _conv_inputs(wl, start, end, heads, kheads, conv_from, path):
    """Convolved inputs for tokens [start, end); keys then L2-normalised.

    The conv history is the raw rows [conv_from, start), at most W-1 of them,
    zero-padded in front when fewer exist.  conv_from=None reads the rows of
    the concatenation itself (zero before token 0).
    """
    W = wl.conv_w
    n = end - start
    if conv_from is None:
        conv_from = max(0, start - (W - 1))
    conv_from = max(conv_from, start - (W - 1))

    def run(x_all, w_all, hs, d):
        x = _f64(x_all[conv_from:end])[:, hs].reshape(end - conv_from, len(hs) * d)
        w = _f64(w_all).reshape(-1, d, W)[hs].reshape(len(hs) * d, W)
        hist = np.zeros((W - 1, len(hs) * d))
        have = start - conv_from
        if have > 0:
            hist[W - 1 - have:] = x[:have]
        return causal_conv(x[have:], w, hist, path).reshape(n, len(hs), d)

    yk = l2norm_rows(run(wl.k, wl.conv_wk, kheads, wl.d_k), path)
    yv = run(wl.v, wl.conv_wv, heads, wl.d_v)
    return np.ascontiguousarray(yk), np.ascontiguousarray(yv)


def build_pairs(wl, segs=None, heads=None, path=None):
    """Cached pairs of the workload's bodies, dense form.

    Returns T [len(segs), len(heads), d_k, d_k] and S0 [.., d_k, d_v].  With a
    conv, each segment is prefilled on its own: its conv history at the
    segment start is zero (the body never reads it when w >= W-1).
    """
    segs = list(range(wl.n_seg)) if segs is None else list(segs)
    heads = list(range(wl.h_v)) if heads is None else list(heads)
    body = wl.body_ranges()
    off = wl.seg_off()
    T = np.empty((len(segs), len(heads), wl.d_k, wl.d_k))
    S0 = np.empty((len(segs), len(heads), wl.d_k, wl.d_v))
    for si, j in enumerate(segs):
        s, e = body[j]
        sl = Slice(wl, s, e, heads, conv_from=off[j], path=path)
        t, s0 = build_units(wl.rule, sl.gate_kind, sl.units(), wl.d_k, wl.d_v,
                            sl.k, sl.v, sl.beta, sl.g, path)
        T[si], S0[si] = t, s0
    return T, S0


def recur_range(wl, start, end, S, heads=None, path=None, q=None):
    """Advance per-head states S [len(heads), d_k, d_v] over tokens [start, end).

    For conv workloads the history is the concatenation's previous W-1 raw
    rows (the cached segment-tail conv state at a seam; zeros at token 0).
    With q [end - start, h_k, d_k] (final queries of those tokens, all key
    heads) also returns the read-outs o_t = q_t^T S_t with the post-update
    state (Eq. (2)), [end - start, len(heads), d_v]: (S, o).
    """
    sl = Slice(wl, start, end, heads, path=path)
    S = np.array(S, dtype=np.float64, copy=True, order="C")
    if q is None:
        recur_units(wl.rule, sl.gate_kind, sl.units(), wl.d_k, wl.d_v,
                    sl.k, sl.v, sl.beta, sl.g, S, path=path)
        return S
    u = sl.units()
    qs = np.ascontiguousarray(_f64(q)[:, sl.kheads])   # laid out like sl.k
    o = np.zeros((sl.n, len(sl.heads), wl.d_v))         # laid out like sl.v
    recur_units(wl.rule, sl.gate_kind, u, wl.d_k, wl.d_v, sl.k, sl.v, sl.beta, sl.g, S,
                q=qs, o=o, off_q=u.off_k, ldq=u.ldk, off_o=u.off_v, ldo=u.ldv, path=path)
    return S, o


def compose(T, S0, S_init=None, wl=None, heads=None, seams=False, path=None, q=None):
    """Fold S <- T_j S + S0_j over j in prompt order (Eq. (6)).

    T, S0: [n, H, ...] dense fp64 (expand_dense turns scalar/diag forms into
    dense).  With seams=True (needs wl) the seam window of each inner
    segment is advanced token by token from the running state first.  With
    q [n - 1, w, h_k, d_k] (the final queries of every window, seams=True)
    the windows also read out o_t = q_t^T S_t as they advance (ch.2 sec.5:
    the recomputed tokens produce their outputs from the true prefix state);
    returns (S, o) with o [n - 1, w, len(heads), d_v].
    """
    n, H, dk, dv = S0.shape
    S = np.zeros((H, dk, dv)) if S_init is None else np.array(S_init, dtype=np.float64)
    wins = wl.window_ranges() if seams else []
    outs = []
    for j in range(n):
        if seams and j > 0:
            s, e = wins[j - 1]
            if q is None:
                S = recur_range(wl, s, e, S, heads=heads, path=path)
            else:
                S, oj = recur_range(wl, s, e, S, heads=heads, path=path, q=q[j - 1])
                outs.append(oj)
        apply_pair(np.ascontiguousarray(T[j]), np.ascontiguousarray(S0[j]), S, path)
    if q is None:
        return S
    o = np.stack(outs) if outs else np.zeros((0, 0, H, dv))
    return S, o


def _with_window_rows(wl, win):
    """A float64 copy of workload wl whose seam-window rows carry the given
    inputs: win["k"] [n_win, w, h_k, d_k] and win["v"] [n_win, w, h_v, d_v]
    (raw rows when the workload has a conv), win["beta"], win["alpha"]
    [n_win, w, h_v].  Every other row is the workload's own."""
    import dataclasses
    import torch
    k = torch.as_tensor(_f64(wl.k)).clone()
    v = torch.as_tensor(_f64(wl.v)).clone()
    beta = torch.as_tensor(_f64(wl.beta)).clone()
    gate = torch.as_tensor(_f64(wl.gate)).clone()
    for j, (s, e) in enumerate(wl.window_ranges()):
        k[s:e] = torch.as_tensor(_f64(win["k"][j]))
        v[s:e] = torch.as_tensor(_f64(win["v"][j]))
        beta[s:e] = torch.as_tensor(_f64(win["beta"][j]))
        gate[s:e] = torch.as_tensor(_f64(win["alpha"][j]))
    return dataclasses.replace(wl, k=k, v=v, beta=beta, gate=gate)


def compose_layers(wls, T, S0, q0, project, path=None):
    """A stack of gated-delta layers over one prompt (ch.2 sec.5, Figs. 7-8):
    the seam-window tokens are recomputed layer by layer, and what a window
    token reads out at layer l is what its inputs at layer l+1 are made from.

    wls[l]: layer l's workload (its cached bodies; layer 0's window rows too);
    T[l], S0[l]: layer l's cached pairs (dense, all heads); q0: layer 0's
    window queries [n_win, w, h_k, d_k].  project(l, o) maps layer l's
    read-outs o [n_win, w, h_v, d_v] to layer l+1's window inputs: a dict with
    "k", "v", "beta", "alpha" (see _with_window_rows) and "q".  Each layer is
    compose(..., seams=True, q=...) token by token over its windows.
    Returns [(S_l, o_l)] per layer.
    """
    out = []
    win = None
    for l, wl in enumerate(wls):
        q = q0
        if win is not None:
            wl = _with_window_rows(wl, win)
            q = win["q"]
        S, o = compose(T[l], S0[l], wl=wl, seams=True, path=path, q=q)
        out.append((S, o))
        if l + 1 < len(wls):
            win = project(l, o)
    return out


def full_recompute(wl, S_init=None, heads=None, path=None):
    """Recur over the whole concatenation from S_init (zero by default)."""
    heads = list(range(wl.h_v)) if heads is None else list(heads)
    S = (np.zeros((len(heads), wl.d_k, wl.d_v)) if S_init is None
         else np.array(S_init, dtype=np.float64))
    return recur_range(wl, 0, wl.n_tokens, S, heads=heads, path=path)


def naive_sum(S0):
    """Naive addition of zero-initial end states (the baseline of Eq. (4))."""
    return np.sum(np.asarray(S0, dtype=np.float64), axis=0)


def relF(x, ref, floor=2.0 ** -126):
    """Relative Frobenius error ||x - ref|| / max(||ref||, floor); 0 when equal."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.linalg.norm((x - ref).ravel()))
    if num == 0.0:
        return 0.0
    return num / max(float(np.linalg.norm(ref.ravel())), floor)


def angle_deg(x, ref):
    """Angle between x and ref viewed as flat vectors, in degrees."""
    x = np.asarray(x, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    nx, nr = np.linalg.norm(x), np.linalg.norm(ref)
    if nx == 0.0 or nr == 0.0:
        return 0.0 if nx == nr else 90.0
    c = float(np.dot(x, ref) / (nx * nr))
    return float(np.degrees(np.arccos(min(1.0, max(-1.0, c)))))


def rope_rotate(x, delta, rot_dim=None, pairing=0, base=10000.0, path=None):
    """R(delta) applied to the last axis of x (every vector; delta a scalar, or an
    array broadcast over the leading axes).  rot_dim leading entries form the
    rotated pairs (pairing 0: (i, i + rot_dim/2); 1: (2i, 2i + 1)), theta_i =
    base^(-2i/rot_dim); the rest pass through.  fp64 copy returned."""
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    rot = d if rot_dim is None else int(rot_dim)
    rows = np.ascontiguousarray(x.reshape(-1, d))
    # delta: a scalar, or an array broadcast over the leading axes of x
    dl = np.ascontiguousarray(np.broadcast_to(np.asarray(delta, dtype=np.float64), x.shape[:-1]).reshape(-1))
    lib(path).lib.orc_rope_rows(rows.shape[0], d, rot, int(pairing), float(base), _dp(dl), _dp(rows))
    return rows.reshape(x.shape)


def rope_rotate_state(S, delta, rot_dim=None, pairing=0, base=10000.0, path=None):
    """S [..., d_k, d_v] with R(delta) applied along d_k (every column of S), the
    linear-state form of ch.2 sec.6, Eq. (7)."""
    St = np.swapaxes(np.asarray(S, dtype=np.float64), -1, -2)
    return np.swapaxes(rope_rotate(St, delta, rot_dim, pairing, base, path), -1, -2).copy()

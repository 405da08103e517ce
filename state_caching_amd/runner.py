"""Host-side sequencing of a synthetic workload through libhypic.

Marshalling only: segment tables, gathering of seam-window and tail rows by
indexing, device placement.  The arithmetic of the method runs in the
library's kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (BF16, F32, GATE_DIAG, GATE_HEAD_CONST, GATE_SCALAR, PREC_FP32, PREC_SPLIT,
               RULE_DECAY, RULE_DELTA, Seams, compose, segment_build, tform_of)

_RULE = {"decay": RULE_DECAY, "delta": RULE_DELTA}
_GATE = {"head_const": GATE_HEAD_CONST, "scalar": GATE_SCALAR, "diag": GATE_DIAG}


class DeviceWorkload:
    """A synth.Workload's tensors on one device, plus its segment tables."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.device = torch.device(device)
        mv = lambda t: None if t is None else t.to(self.device).contiguous()
        self.k, self.v, self.beta, self.gate = mv(wl.k), mv(wl.v), mv(wl.beta), mv(wl.gate)
        self.conv_wk, self.conv_wv = mv(wl.conv_wk), mv(wl.conv_wv)
        self.rule = _RULE[wl.rule]
        self.gate_kind = _GATE[wl.gate_kind]
        self.tform = tform_of(self.rule, self.gate_kind)
        self.prec = PREC_FP32 if wl.dtype == torch.float32 else PREC_SPLIT
        body = wl.body_ranges()
        self.seg_start = [s for s, _ in body]
        self.seg_len = [e - s for s, e in body]
        off = wl.seg_off()
        self.conv_from = [off[j] for j in range(wl.n_seg)]
        self.seams: Optional[Seams] = self._gather_seams() if wl.seam_w > 0 else None

    def _gather_seams(self) -> Seams:
        wl = self.wl
        starts = [s for s, _ in wl.window_ranges()]
        w, W = wl.seam_w, wl.conv_w
        idx = torch.tensor([s + t for s in starts for t in range(w)], device=self.device)
        n_win = len(starts)

        def rows(x, ix, n_per):
            return x.index_select(0, ix).reshape(n_win, n_per, *x.shape[1:]).contiguous()

        sm = Seams(xk=rows(self.k, idx, w), xv=rows(self.v, idx, w),
                   beta=rows(self.beta, idx, w), alpha=rows(self.gate, idx, w),
                   conv_w=W, k_l2norm=1 if W > 0 else 0,
                   conv_wk=self.conv_wk, conv_wv=self.conv_wv)
        if W > 1:
            tix = torch.tensor([s - (W - 1) + t for s in starts for t in range(W - 1)],
                               device=self.device)
            sm.tail_k = rows(self.k, tix, W - 1)
            sm.tail_v = rows(self.v, tix, W - 1)
        return sm

    def build(self, segs=None, stream=None):
        """(T, S0) of the bodies (all segments, or the listed indices)."""
        segs = list(range(self.wl.n_seg)) if segs is None else list(segs)
        conv = self.wl.conv_w
        return segment_build(self.rule, self.gate_kind, self.k, self.v, self.beta, self.gate,
                             [self.seg_start[j] for j in segs], [self.seg_len[j] for j in segs],
                             conv_w=conv, conv_wk=self.conv_wk if conv else None,
                             conv_wv=self.conv_wv if conv else None,
                             conv_from=[self.conv_from[j] for j in segs] if conv else None,
                             k_l2norm=1 if conv else 0, stream=stream)

    def compose(self, T, S0, S_init=None, order=None, seams=True, prec=None, S_out=None,
                stream=None, group_len=0):
        order = list(range(S0.shape[0])) if order is None else list(order)
        return compose(T, S0, order, S_init=S_init, tform=self.tform,
                       prec=self.prec if prec is None else prec,
                       seams=self.seams if seams else None, S_out=S_out, stream=stream,
                       group_len=group_len)


def compose_layers(layers, project, S_init=None, stream=None):
    """Compose a stack of layers bottom to top, each with its seam windows
    recomputed and read out (HYPIC reading notes ch.2 sec.5, Figs. 7-8: a
    recomputed window token's output at one layer is what its inputs at the
    next layer are made from, so the layers run in order).

    layers[l] = (T, S0, order, seams, tform, prec): layer l's cached pairs and
    Seams, whose tails and conv weights are that layer's own; layer 0's
    window rows and queries are in its Seams.  project(l, o) receives layer
    l's read-outs o [n_win, w, h_v, d_v] (fp32, device) and returns layer
    l+1's window inputs as a dict of device tensors shaped like the Seams
    fields "xk", "xv", "beta", "alpha", "q" (the caller's model: projections,
    norms, activations).  Host-side sequencing only: every layer's compose
    runs in the library.  S_init: None (zero prefix state at every layer) or
    one state [h_v, d_k, d_v] per layer.  Returns [(S_l, o_l)] per layer.
    """
    if S_init is not None and len(S_init) != len(layers):
        raise ValueError("S_init needs one state per layer")
    out = []
    nxt = None
    for l, (T, S0, order, seams, tform, prec) in enumerate(layers):
        if seams is None:
            raise ValueError("every layer needs its seam windows")
        if nxt is not None:
            for name in ("xk", "xv", "beta", "alpha", "q"):
                ref = getattr(seams, name) if name != "q" else seams.xk
                t = nxt[name]
                if t.device != S0.device:
                    raise ValueError(f"layer {l}: window input {name} is on another device")
                setattr(seams, name, t.to(ref.dtype).contiguous())
        elif seams.q is None:
            raise ValueError("layer 0 needs its window queries")
        n_win, w = seams.xk.shape[0], seams.xk.shape[1]
        h_v, d_v = S0.shape[1], S0.shape[3]
        seams.o = torch.empty((n_win, w, h_v, d_v), dtype=torch.float32, device=S0.device)
        S = compose(T, S0, list(order), S_init=None if S_init is None else S_init[l], tform=tform,
                    prec=prec, seams=seams, stream=stream)
        out.append((S, seams.o))
        if l + 1 < len(layers):
            nxt = project(l, seams.o)
    return out

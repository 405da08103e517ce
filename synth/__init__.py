"""Seeded synthetic inputs for linear-attention state caching.

This module holds random draws and input distributions only: no recurrence,
no transition product, no composition, no convolution and no normalisation
that belongs to the method.  Both the fp64 CPU oracle (``oracle/``) and the
GPU library binding (``state_caching_amd``) take their inputs from here, so
the two see exactly the same bits.

Workloads mirror the shapes the HYPIC reading notes discuss (page
"HYPIC ... reading notes", ch. 1 sec. 2 Table 2; ch. 2 secs. 2-7; ch. 3
sec. 6): cold prompts of equal segments, a slow-decay RetNet head at 256
tokens, segments of 512 tokens and more, a ~100k-token prompt.

Draw convention (one numpy PCG64 generator per workload, seeded with the
workload's seed): arrays are drawn in the order k, v, beta-logits,
gate-logits, then conv weights, each over the whole concatenation of the
prompt's tokens, in float64, then rounded to float32 and, for bf16
workloads, to bfloat16 by round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

RULE_DECAY = "decay"   # T_i = gate, u_i = k v^T            (RetNet, Mamba2, GLA)
RULE_DELTA = "delta"   # T_i = g (I - b k k^T), u = b k v^T (GDN, DeltaNet)

GATE_HEAD_CONST = "head_const"  # one constant per value head  [h_v]        (RetNet)
GATE_SCALAR = "scalar"          # one scalar per token and head [N, h_v]    (GDN, Mamba2)
GATE_DIAG = "diag"              # one vector per token and head [N, h_v, d_k] (GLA)


@dataclass
class Workload:
    """One synthetic prompt for one linear-attention layer.

    ``seg_len`` lists the raw token count of each segment in prompt order.
    ``seam_w`` > 0 marks every segment but the first as inner: its first
    ``seam_w`` tokens form the seam window and its cached pair covers the
    rest (the body).  ``conv_w`` > 0 means ``k``/``v`` hold the raw inputs of
    a depthwise causal convolution of that width (weights ``conv_wk``,
    ``conv_wv``), after which keys are L2-normalised.
    """

    name: str
    rule: str
    gate_kind: str
    dtype: torch.dtype
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    seg_len: List[int]
    k: torch.Tensor                    # [N, h_k, d_k]   (raw x_k when conv_w > 0)
    v: torch.Tensor                    # [N, h_v, d_v]   (raw x_v when conv_w > 0)
    beta: Optional[torch.Tensor]       # [N, h_v] (delta rule only)
    gate: torch.Tensor                 # per gate_kind; values in (0, 1]
    conv_w: int = 0
    conv_wk: Optional[torch.Tensor] = None   # [h_k*d_k, conv_w] float32
    conv_wv: Optional[torch.Tensor] = None   # [h_v*d_v, conv_w] float32
    seam_w: int = 0
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_tokens(self) -> int:
        return int(sum(self.seg_len))

    @property
    def n_seg(self) -> int:
        return len(self.seg_len)

    def seg_off(self) -> List[int]:
        off = [0]
        for m in self.seg_len:
            off.append(off[-1] + int(m))
        return off

    def body_ranges(self):
        """(start, end) token range each cached pair covers, in prompt order."""
        off = self.seg_off()
        out = []
        for j in range(self.n_seg):
            skip = self.seam_w if (j > 0 and self.seam_w > 0) else 0
            out.append((off[j] + skip, off[j + 1]))
        return out

    def window_ranges(self):
        """(start, end) token range of each seam window (segments 2..n)."""
        if self.seam_w <= 0:
            return []
        off = self.seg_off()
        return [(off[j], off[j] + self.seam_w) for j in range(1, self.n_seg)]


def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    if dtype == torch.bfloat16:
        t = t.to(torch.bfloat16)
    elif dtype != torch.float32:
        raise ValueError(f"unsupported dtype {dtype}")
    return t.contiguous()


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z):
    return np.logaddexp(0.0, z)


def _unit_rows(x):
    # input distribution "N(0,1) then L2-normalised" along the last axis
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def gdn(seed, seg_len, h_k, h_v, d, dtype, alpha_div=1.0, name="gdn",
        conv_w=0, seam_w=0, beta_const=None):
    """Gated-delta workload.

    k ~ N(0,1) L2-normalised per (token, key head) (raw N(0,1) when conv_w>0),
    v ~ N(0,1), beta = sigmoid(N(0,1)), alpha = exp(-softplus(N(0,1))/alpha_div).
    With conv_w > 0 the conv weights are N(0, 1/conv_w) (std 0.5 at width 4).
    """
    rng = np.random.default_rng(seed)
    n = int(sum(seg_len))
    k = rng.standard_normal((n, h_k, d))
    if conv_w == 0:
        k = _unit_rows(k)
    v = rng.standard_normal((n, h_v, d))
    beta = _sigmoid(rng.standard_normal((n, h_v)))
    if beta_const is not None:
        beta = np.full_like(beta, beta_const)
    alpha = np.exp(-_softplus(rng.standard_normal((n, h_v))) / alpha_div)
    wk = wv = None
    if conv_w > 0:
        sd = 1.0 / np.sqrt(conv_w)
        wk = _round(rng.standard_normal((h_k * d, conv_w)) * sd, torch.float32)
        wv = _round(rng.standard_normal((h_v * d, conv_w)) * sd, torch.float32)
    return Workload(name=name, rule=RULE_DELTA, gate_kind=GATE_SCALAR, dtype=dtype,
                    h_k=h_k, h_v=h_v, d_k=d, d_v=d, seg_len=list(seg_len),
                    k=_round(k, dtype), v=_round(v, dtype), beta=_round(beta, dtype),
                    gate=_round(alpha, dtype), conv_w=conv_w, conv_wk=wk, conv_wv=wv,
                    seam_w=seam_w, seed=seed)


def kda(seed, seg_len, h_k, h_v, d, dtype, gate_div=1.0, name="kda", conv_w=0, seam_w=0):
    """Delta rule with a diagonal gate (KDA row of Table 1).

    k ~ N(0,1) L2-normalised per (token, key head) (raw N(0,1) when conv_w>0),
    v ~ N(0,1), beta = sigmoid(N(0,1)), g = exp(-softplus(N(0,1))/gate_div) per
    key dimension and value head, [N, h_v, d].  Draw order as for gdn.
    """
    rng = np.random.default_rng(seed)
    n = int(sum(seg_len))
    k = rng.standard_normal((n, h_k, d))
    if conv_w == 0:
        k = _unit_rows(k)
    v = rng.standard_normal((n, h_v, d))
    beta = _sigmoid(rng.standard_normal((n, h_v)))
    g = np.exp(-_softplus(rng.standard_normal((n, h_v, d))) / gate_div)
    wk = wv = None
    if conv_w > 0:
        sd = 1.0 / np.sqrt(conv_w)
        wk = _round(rng.standard_normal((h_k * d, conv_w)) * sd, torch.float32)
        wv = _round(rng.standard_normal((h_v * d, conv_w)) * sd, torch.float32)
    return Workload(name=name, rule=RULE_DELTA, gate_kind=GATE_DIAG, dtype=dtype,
                    h_k=h_k, h_v=h_v, d_k=d, d_v=d, seg_len=list(seg_len),
                    k=_round(k, dtype), v=_round(v, dtype), beta=_round(beta, dtype),
                    gate=_round(g, dtype), conv_w=conv_w, conv_wk=wk, conv_wv=wv, seam_w=seam_w,
                    seed=seed)


def retnet(seed, seg_len, h, d, dtype=torch.float32, name="retnet", gammas=None):
    """Scalar-decay workload: gamma_h = 1 - 2^-(5+h), k, v ~ N(0,1)/sqrt(d)."""
    rng = np.random.default_rng(seed)
    n = int(sum(seg_len))
    k = rng.standard_normal((n, h, d)) / np.sqrt(d)
    v = rng.standard_normal((n, h, d)) / np.sqrt(d)
    if gammas is None:
        gammas = [1.0 - 2.0 ** -(5 + i) for i in range(h)]
    g = torch.tensor(gammas, dtype=torch.float64).to(torch.float32)
    return Workload(name=name, rule=RULE_DECAY, gate_kind=GATE_HEAD_CONST, dtype=dtype,
                    h_k=h, h_v=h, d_k=d, d_v=d, seg_len=list(seg_len),
                    k=_round(k, dtype), v=_round(v, dtype), beta=None, gate=g, seed=seed)


def gla(seed, seg_len, h, d, dtype=torch.bfloat16, literal=True, name="gla"):
    """Diagonal-gate workload, k, v ~ N(0,1).

    literal=True:  g = exp(-softplus(z)) / 16   (every gate below 1/16)
    literal=False: g = exp(-softplus(z) / 16)   (slow decay, typical g ~ 0.95)
    """
    rng = np.random.default_rng(seed)
    n = int(sum(seg_len))
    k = rng.standard_normal((n, h, d))
    v = rng.standard_normal((n, h, d))
    z = rng.standard_normal((n, h, d))
    g = np.exp(-_softplus(z)) / 16.0 if literal else np.exp(-_softplus(z) / 16.0)
    return Workload(name=name, rule=RULE_DECAY, gate_kind=GATE_DIAG, dtype=dtype,
                    h_k=h, h_v=h, d_k=d, d_v=d, seg_len=list(seg_len),
                    k=_round(k, dtype), v=_round(v, dtype), beta=None,
                    gate=_round(g, dtype), seed=seed)


# Named synthetic workloads (the seed is fixed per workload).
WORKLOADS = ("gdn_d16_2x64_fp32", "retnet_d64_8h_4x256_fp32", "gla_d128_16h_8x512_bf16",
             "gdn_gqa_d128_8x4096_bf16", "gdn_d128_32h_100x1024_seams_bf16",
             "gla_d128_16h_8x512_bf16_slow", "gdn_gqa_d128_8x4096_bf16_slow",
             "kda_gqa_d128_8x4096_bf16", "gdn_d128_32h_100x1024_seams_bf16_slow")


def workload(name: str) -> Workload:
    """A named workload.  The *_slow companions keep the transition operators
    far from 0 (slow decay), so that products of many of them stay measurable."""
    if name == "gdn_d16_2x64_fp32":
        return gdn(0, [64, 64], 1, 1, 16, torch.float32, name=name)
    if name == "retnet_d64_8h_4x256_fp32":
        return retnet(1, [256] * 4, 8, 64, name=name)
    if name == "gla_d128_16h_8x512_bf16":
        return gla(2, [512] * 8, 16, 128, literal=True, name=name)
    if name == "gdn_gqa_d128_8x4096_bf16":
        return gdn(3, [4096] * 8, 16, 32, 128, torch.bfloat16, name=name)
    if name == "gdn_d128_32h_100x1024_seams_bf16":
        return gdn(4, [1024] * 100, 32, 32, 128, torch.bfloat16, conv_w=4, seam_w=8, name=name)
    if name == "gla_d128_16h_8x512_bf16_slow":
        return gla(2, [512] * 8, 16, 128, literal=False, name=name)
    if name == "gdn_d128_32h_100x1024_seams_bf16_slow":
        return gdn(4, [1024] * 100, 32, 32, 128, torch.bfloat16, alpha_div=1024.0, conv_w=4, seam_w=8,
                   name=name)
    if name == "kda_gqa_d128_8x4096_bf16":
        return kda(5, [4096] * 8, 16, 32, 128, torch.bfloat16, name=name)
    if name == "gdn_gqa_d128_8x4096_bf16_slow":
        return gdn(3, [4096] * 8, 16, 32, 128, torch.bfloat16, alpha_div=4096.0, name=name)
    raise ValueError(name)


def random_pairs(seed, n_slots, h, d_k, d_v, tform="dense", rho=0.9):
    """Synthetic cached pairs for composition-only tests.

    dense: T = rho * G / (2 sqrt(d_k)) with G ~ N(0,1) (spectral norm ~ rho);
    diag:  T = rho * U(0,1) per key dim;  scalar: T = rho * U(0,1).
    S0 ~ N(0,1).  All float32.
    """
    rng = np.random.default_rng(seed)
    if tform == "dense":
        T = rho * rng.standard_normal((n_slots, h, d_k, d_k)) / (2.0 * np.sqrt(d_k))
    elif tform == "diag":
        T = rho * rng.random((n_slots, h, d_k))
    elif tform == "scalar":
        T = rho * rng.random((n_slots, h))
    else:
        raise ValueError(tform)
    S0 = rng.standard_normal((n_slots, h, d_k, d_v))
    return _round(T, torch.float32), _round(S0, torch.float32)


def rope_keys(seed, n_tokens, h, d, dtype=torch.bfloat16):
    """Cached full-attention keys [n_tokens, h, d]: standard normal, drawn by a
    seeded torch CPU generator, then rounded to dtype."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn((n_tokens, h, d), generator=g).to(dtype)


ROPE_32K = dict(seed=6, n_tokens=8 * 4096, h=16, d=128,
                seg_start=[4096 * i for i in range(8)], seg_len=[4096] * 8,
                delta=[4096 * i + 517 for i in range(8)])
"""The 32k-token prompt's cached keys (8 segments x 4096, 16 KV heads, d = 128)
and the shifts that move segment i to start 4096 i + 517 tokens later."""


def layer_projection(seed, h_k, h_v, d):
    """Weights of a synthetic layer-to-layer map for seam windows: a window
    token's read-out of one layer, flattened to x [h_v * d], gives the next
    layer's raw key and value rows x Wk [h_k * d], x Wv [h_v * d], its final
    query x Wq [h_k * d] (L2-normalised per head by the user of these
    weights), and the logits of its write strength x wb [h_v] and gate
    x wa [h_v].  Entries N(0, 1 / (h_v d)); float32 values held as float64."""
    rng = np.random.default_rng(seed)
    n = h_v * d
    sd = 1.0 / np.sqrt(n)
    out = {}
    for name, m in (("Wk", h_k * d), ("Wv", h_v * d), ("Wq", h_k * d), ("wb", h_v), ("wa", h_v)):
        out[name] = _round(rng.standard_normal((n, m)) * sd, torch.float32).double().numpy()
    return out


def window_queries(seed, n_win, w, h_k, d):
    """Final queries of seam-window tokens [n_win, w, h_k, d]: N(0,1) rows,
    L2-normalised, float32."""
    rng = np.random.default_rng(seed)
    return _round(_unit_rows(rng.standard_normal((n_win, w, h_k, d))), torch.float32)


def random_state(seed, h, d_k, d_v):
    rng = np.random.default_rng(seed)
    return _round(rng.standard_normal((h, d_k, d_v)), torch.float32)

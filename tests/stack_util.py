"""Synthetic layer-to-layer map for seam windows (the caller's model in a
multi-layer stack), in two precisions from the same seeded weights
(``synth.layer_projection``): fp64 numpy for the oracle side and fp32 torch
for the device side.  Neither is part of the method: a real model puts its
attention output, MLP and next-layer projections here."""
from __future__ import annotations

import numpy as np


def project_np(P, h_k, h_v, d, norm_k):
    """o [n_win, w, h_v, d] -> next layer's window inputs (fp64); keys are
    L2-normalised per head when norm_k (no conv), queries always."""
    def f(l, o):
        n_win, w = o.shape[:2]
        x = np.asarray(o, dtype=np.float64).reshape(n_win, w, h_v * d)
        W = P[l]
        k = (x @ W["Wk"]).reshape(n_win, w, h_k, d)
        if norm_k:
            k = k / np.linalg.norm(k, axis=-1, keepdims=True)
        q = (x @ W["Wq"]).reshape(n_win, w, h_k, d)
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
        return {"k": k, "v": (x @ W["Wv"]).reshape(n_win, w, h_v, d), "q": q,
                "beta": 1.0 / (1.0 + np.exp(-(x @ W["wb"]))),
                "alpha": np.exp(-np.logaddexp(0.0, x @ W["wa"]))}
    return f


def project_torch(P, h_k, h_v, d, norm_k, device):
    """The same map in fp32 on the device, returning Seams field names."""
    import torch
    Wt = [{k: torch.tensor(v, dtype=torch.float32, device=device) for k, v in W.items()} for W in P]

    def f(l, o):
        n_win, w = o.shape[:2]
        x = o.reshape(n_win * w, h_v * d).float()
        W = Wt[l]
        k = (x @ W["Wk"]).reshape(n_win, w, h_k, d)
        if norm_k:
            k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)
        q = (x @ W["Wq"]).reshape(n_win, w, h_k, d)
        q = q / torch.linalg.vector_norm(q, dim=-1, keepdim=True)
        return {"xk": k, "xv": (x @ W["Wv"]).reshape(n_win, w, h_v, d), "q": q,
                "beta": torch.sigmoid(x @ W["wb"]).reshape(n_win, w, h_v),
                "alpha": torch.exp(-torch.nn.functional.softplus(x @ W["wa"])).reshape(n_win, w, h_v)}
    return f

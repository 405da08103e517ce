"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import pytest
import torch

import oracle

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def case(msg: str):
    """Name the case on stdout before a GPU step (survives a lost box)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def max_relF(gpu: np.ndarray, ref: np.ndarray, unit_axes: int):
    """Largest relative Frobenius error over the leading `unit_axes` axes."""
    g = gpu.reshape(-1, *gpu.shape[unit_axes:])
    r = ref.reshape(-1, *ref.shape[unit_axes:])
    errs = [oracle.relF(g[i], r[i]) for i in range(g.shape[0])]
    return max(errs) if errs else 0.0


def head_relF(gpu: np.ndarray, ref: np.ndarray):
    """Largest relative Frobenius error over the heads of states [h, d_k, d_v]
    (every head is its own unit: a pooled error would hide a bad head)."""
    return max_relF(gpu, ref, 1)


def expand_T(T: np.ndarray, tform: int, d: int) -> np.ndarray:
    name = {0: "scalar", 1: "diag", 2: "dense"}[tform]
    return oracle.expand_dense(T, name, d)

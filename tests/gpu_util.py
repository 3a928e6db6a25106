"""Helpers for the GPU parity tests (tensor plumbing and error measures only)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    """Progress line, flushed at once so a run that dies still names its last case."""
    print(*a, file=sys.stderr, flush=True)


def dev(x: np.ndarray, bf16: bool = False) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def max_rel_rows(got: np.ndarray, want: np.ndarray) -> float:
    """Max over rows of max_j |got - want| / max_j |want| (rows = all but the last axis)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    w = np.asarray(want, dtype=np.float64).reshape(-1, want.shape[-1])
    num = np.abs(g - w).max(axis=1)
    den = np.abs(w).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())

"""Oracle: self-conditioning embedding average (float64).

Test infrastructure only (see the package docstring).

Between denoising steps the model conditions on the previous prediction's full
softmax, turned into the probability-weighted average of the token embeddings
([P1] section "안정성을 위한 셀프 컨디셔닝"; [P3] section
"Mehanizam odlučivanja o gotovim tokenima"). The gated MLP that injects the average
into the canvas embedding needs trained weights and is not part of this path.

Readings: the probabilities are the temperature-1 softmax over all canvas positions
(accepted or not); given probabilities are used as they are; raw embedding rows,
no extra scale.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    l = np.asarray(logits, dtype=np.float64)
    w = np.exp(l - l.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def selfcond_embed(embed: np.ndarray, probs: np.ndarray = None, logits: np.ndarray = None) -> np.ndarray:
    """out[i, :] = sum_v p[i, v] * E[v, :], with p given or the softmax of logits."""
    if probs is None:
        probs = softmax_rows(logits)
    p = np.asarray(probs, dtype=np.float64)
    e = np.asarray(embed, dtype=np.float64)
    return p @ e

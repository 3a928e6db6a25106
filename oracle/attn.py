"""Oracle: mixed-mode attention over a canvas plus a committed KV prefix (float64).

Test infrastructure only (see the package docstring).

What is computed, and where the pages state it:
  * one weight set, two attention modes: causal for prefill/commit ("encoder mode"),
    bidirectional for denoising ("decoder mode") - [P1] section "듀얼 모드 운영",
    [P2] section "블록 자기회귀 노이즈 제거 (Block Autoregressive Denoising)",
    [P3] section "Zašto je difuzijsko generiranje teksta drugačije?";
  * the mode is chosen per request inside one batch - [P1] section
    "동적 퍼-시퀀스 인과적 어텐션";
  * sliding-window layers: a causal request sees the W tokens before it, a
    bidirectional one sees W on each side, 2W+1 in all - [P1] section
    "대칭 슬라이딩 윈도우 어텐션", [P3] (the +-W windows of decoder mode).

Readings taken where the pages leave a step open:
  * the one-sided window holds the W preceding tokens plus the token itself (W+1 keys);
  * window bounds are absolute positions over [cache || new tokens], clipped to the
    request's own keys; requests never see each other;
  * query head h reads KV head floor(h / G), G = Hq / Hkv;
  * score = <q, k> * scale with scale = 1/sqrt(D) unless given; no bias or softcap;
  * lse is the natural log of the sum of exp(score) over the key set.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

CAUSAL, BIDIR = 0, 1


def key_range(mode: int, prefix_len: int, num_q: int, window: int, i: int) -> Tuple[int, int]:
    """Inclusive key range [lo, hi] (request-local key rows) of new token i.

    The token sits at absolute position q = prefix_len + i. A causal query sees keys
    up to itself; a bidirectional one sees up to the request's last key. A window
    W >= 0 keeps keys within W positions on the sides the mode allows.
    """
    q = prefix_len + i
    last = prefix_len + num_q - 1
    lo = 0 if window < 0 else max(0, q - window)
    if mode == CAUSAL:
        hi = q
    else:
        hi = last if window < 0 else min(last, q + window)
    return lo, hi


def _seq_fields(s):
    if isinstance(s, dict):
        return s["q_start"], s["num_q"], s["kv_start"], s["prefix_len"], s["mode"]
    if hasattr(s, "q_start"):
        return s.q_start, s.num_q, s.kv_start, s.prefix_len, s.mode
    return tuple(s)


def attn_mixed(seqs: Sequence, window: int, q: np.ndarray, k: np.ndarray, v: np.ndarray,
               num_q_heads: int, num_kv_heads: int, scale: Optional[float] = None,
               rows: Optional[Iterable[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Masked softmax attention for every request of a mixed batch.

    q [sum N, Hq, D]; k, v [sum (P+N), Hkv, D]; returns out [sum N, Hq, D] and
    lse [sum N, Hq], both float64. With `rows` (global query-row indices) only those
    rows are computed; the others are left NaN.
    """
    total_q, hq, d = q.shape
    assert hq == num_q_heads and k.shape[1] == num_kv_heads and num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(d)
    out = np.full((total_q, hq, d), np.nan)
    lse = np.full((total_q, hq), np.nan)
    wanted = None if rows is None else set(int(r) for r in rows)
    for s in seqs:
        q_start, num_q, kv_start, prefix_len, mode = _seq_fields(s)
        todo = [i for i in range(num_q) if wanted is None or (q_start + i) in wanted]
        if not todo:
            continue
        for g in range(num_kv_heads):
            # this request's keys and values for KV head g, upcast exactly to float64
            keys = np.asarray(k[kv_start:kv_start + prefix_len + num_q, g, :], dtype=np.float64)
            vals = np.asarray(v[kv_start:kv_start + prefix_len + num_q, g, :], dtype=np.float64)
            for i in todo:
                row = q_start + i
                lo, hi = key_range(mode, prefix_len, num_q, window, i)
                for h in range(g * group, (g + 1) * group):
                    x = (keys[lo:hi + 1] @ np.asarray(q[row, h, :], dtype=np.float64)) * scale
                    mx = x.max()
                    w = np.exp(x - mx)
                    z = w.sum()
                    out[row, h, :] = (w / z) @ vals[lo:hi + 1]
                    lse[row, h] = mx + np.log(z)
    return out, lse


def attn_rows_for_heads(seqs: Sequence, window: int, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                        num_q_heads: int, num_kv_heads: int, rows: List[int],
                        scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Same as attn_mixed restricted to `rows`, returned densely as [len(rows), Hq, D]."""
    out, lse = attn_mixed(seqs, window, q, k, v, num_q_heads, num_kv_heads, scale, rows)
    return out[rows], lse[rows]

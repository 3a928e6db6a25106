"""Oracle: the DiffusionSampler's denoise step (float64 statistics, exact integer selection).

Test infrastructure only (see the package docstring).

What is computed, and where the pages state it:
  * full softmax over the vocabulary at every canvas position, its entropy and a
    confidence - [P1] section "샘플링 루프와 엔트로피 경계 디노이징", [P3] section
    "Mehanizam odlučivanja o gotovim tokenima";
  * a candidate token drawn at every position - [P1] same section;
  * acceptance from most to least confident while the running entropy total stays
    within a fixed budget - [P1] same section, [P3] same section;
  * positions not accepted are re-noised to random tokens (uniform-state diffusion,
    self-correction) - [P2] sections "아키텍처 (The Architecture)" and
    "Diffusion에 스도쿠가 흥미로운 이유";
  * convergence when the argmax has been stable for several steps and the mean
    per-token entropy is under a threshold, or a step limit is reached - [P1]
    "샘플링 루프와 엔트로피 경계 디노이징"; [P2] Sudoku showcase (48-step limit,
    adaptive stopping).

Readings taken where the pages leave a step open:
  * confidence c = -H (entropy in nats); order by c descending, then position
    ascending; a max-probability confidence is available as an option;
  * the accepted set is the longest confidence-ordered prefix whose entropy total is
    <= budget (the position that would cross the budget is rejected), at least
    min_accept positions; totals are exact sums of floor(H * 2^40) in integers,
    taken from the entropies as stored (float32);
  * the argmax is the lowest index among maximal logits;
  * stable count: number of consecutive steps whose whole-canvas argmax equals the
    previous step's (0 at step 0); mean entropy test is strict, in the same fixed
    point; the combinator is (stable>=k AND mean<tau) OR steps>=L by default, with
    the all-OR form as an option;
  * candidates are inverse-CDF draws at temperature 1 from one 24-bit uniform;
  * on the step that converges, positions not accepted take their argmax.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

from .philox import uniform24, renoise_token, STREAM_RENOISE, STREAM_INIT

CONF_NEG_ENTROPY, CONF_MAX_PROB = 0, 1
CONV_AND, CONV_OR = 0, 1
FIXED_SHIFT = 40  # entropies are summed as integers in units of 2^-40 nats


def row_stats(logits: np.ndarray) -> Dict[str, np.ndarray]:
    """Per-row softmax statistics of logits [M, V] (finite or -inf entries).

    Returns float64 max, sum of exp(l - max), entropy (nats), max probability and
    the int64 argmax (lowest index among the maxima).
    """
    l = np.asarray(logits, dtype=np.float64)
    if l.ndim == 1:
        l = l[None, :]
    m = l.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("every logits row needs at least one finite value")
    argmax = np.argmax(l, axis=1)  # numpy returns the first occurrence of the maximum
    w = np.exp(l - m[:, None])
    z = w.sum(axis=1)
    p = w / z[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        logp = np.where(p > 0, np.log(np.where(p > 0, p, 1.0)), 0.0)
    entropy = np.maximum(0.0, -(p * logp).sum(axis=1))
    return {"max": m, "sum": z, "entropy": entropy, "max_prob": 1.0 / z, "argmax": argmax.astype(np.int64)}


def candidate(logits_row: np.ndarray, u: float) -> int:
    """Inverse-CDF draw: the first token whose cumulative probability exceeds u;
    if rounding leaves u above the total, the last token with nonzero probability."""
    l = np.asarray(logits_row, dtype=np.float64)
    w = np.exp(l - l.max())
    p = w / w.sum()
    cdf = np.cumsum(p)
    hit = np.nonzero(cdf > u)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(p > 0)[0][-1])


def _fixed(h32: float) -> int:
    return int(math.floor(float(np.float32(h32)) * 2.0 ** FIXED_SHIFT))


def select(entropy32: np.ndarray, conf32: np.ndarray, budget: float, min_accept: int) -> np.ndarray:
    """Entropy-bounded acceptance over one request's positions.

    Positions are visited from most to least confident (ties: lower position first);
    each is accepted while the exact running total of entropies stays <= budget.
    Returns a bool mask.
    """
    n = len(entropy32)
    order = sorted(range(n), key=lambda i: (-float(conf32[i]), i))
    limit = int(math.floor(float(np.float32(budget)) * 2.0 ** FIXED_SHIFT))
    accept = np.zeros(n, dtype=bool)
    total = 0
    taken = 0
    for rank, i in enumerate(order):
        total += _fixed(entropy32[i])
        if total <= limit or rank < min(min_accept, n):
            accept[i] = True
            taken += 1
        else:
            break
    return accept


def convergence(argmax: np.ndarray, prev_argmax: np.ndarray, stable_prev: int, step: int,
                entropy32: np.ndarray, tau: float, stable_k: int, step_limit: int,
                combine: int = CONV_AND):
    """One step of convergence bookkeeping for one request. Returns
    (converged, stable, mean_entropy)."""
    n = len(entropy32)
    same = step > 0 and bool(np.all(np.asarray(argmax) == np.asarray(prev_argmax)))
    stable = stable_prev + 1 if same else 0
    total = sum(_fixed(h) for h in entropy32)
    threshold = math.ceil(float(np.float32(tau)) * n * 2.0 ** FIXED_SHIFT)
    low = total < threshold
    steps_done = step + 1
    if combine == CONV_AND:
        conv = (stable >= stable_k and low) or steps_done >= step_limit
    else:
        conv = stable >= stable_k or low or steps_done >= step_limit
    return bool(conv), stable, total / 2.0 ** FIXED_SHIFT / n


def sampler_step(logits: np.ndarray, reqs: Sequence, vocab: int, budget: float, min_accept: int,
                 canvas: np.ndarray, prev_argmax: np.ndarray, stable_count: Sequence[int],
                 conf_mode: int = CONF_NEG_ENTROPY, renoise: bool = True, stable_k: int = 3,
                 tau: float = 0.05, step_limit: int = 48, combine: int = CONV_AND,
                 entropy_in: Optional[np.ndarray] = None, conf_in: Optional[np.ndarray] = None,
                 with_candidates: bool = True, stats: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, object]:
    """One denoise step of the sampler over the rows of several requests.

    reqs: (row_start, num_rows, seed, step) per request. logits [M, V]; canvas and
    prev_argmax [M] int. With entropy_in (and conf_in for the max-probability
    confidence) the selection reads those float32 values instead of its own.
    Returns float64 statistics, float32 entropy/conf as stored, candidates, the
    acceptance mask, the new canvas and per-request bookkeeping. stats: row_stats of
    these logits when the caller already has them (they depend on each row alone);
    None computes them here.
    """
    st = row_stats(logits) if stats is None else stats
    m_rows = st["max"].shape[0]
    entropy32 = st["entropy"].astype(np.float32) if entropy_in is None else np.asarray(entropy_in, np.float32)
    if conf_mode == CONF_NEG_ENTROPY:
        conf32 = -entropy32
    else:
        conf32 = st["max_prob"].astype(np.float32) if conf_in is None else np.asarray(conf_in, np.float32)
    cand = np.full(m_rows, -1, dtype=np.int64)
    accept = np.zeros(m_rows, dtype=bool)
    new_canvas = np.array(canvas, dtype=np.int64, copy=True)
    new_prev = np.array(prev_argmax, dtype=np.int64, copy=True)
    out_stable, out_conv, out_mean, out_nacc = [], [], [], []
    for r, (row_start, num_rows, seed, step) in enumerate(reqs):
        rows = slice(row_start, row_start + num_rows)
        if with_candidates:
            for j in range(num_rows):
                u = uniform24(seed, step, j)
                cand[row_start + j] = candidate(logits[row_start + j], u)
        acc = select(entropy32[rows], conf32[rows], budget, min_accept)
        accept[rows] = acc
        conv, stable, mean = convergence(st["argmax"][rows], prev_argmax[rows], int(stable_count[r]), step,
                                         entropy32[rows], tau, stable_k, step_limit, combine)
        for j in range(num_rows):
            i = row_start + j
            if acc[j]:
                new_canvas[i] = cand[i]
            elif conv:
                new_canvas[i] = st["argmax"][i]
            elif renoise:
                new_canvas[i] = renoise_token(seed, step, j, vocab, STREAM_RENOISE)
        new_prev[rows] = st["argmax"][rows]
        out_stable.append(stable)
        out_conv.append(conv)
        out_mean.append(mean)
        out_nacc.append(int(acc.sum()))
    return {"stats": st, "entropy32": entropy32, "conf32": conf32, "cand": cand, "accept": accept,
            "canvas": new_canvas, "prev_argmax": new_prev, "stable_count": np.array(out_stable),
            "converged": np.array(out_conv), "mean_entropy": np.array(out_mean),
            "num_accepted": np.array(out_nacc)}


def init_canvas(reqs: Sequence, vocab: int) -> np.ndarray:
    """Initial canvas: a uniform random token at every position (stream 2)."""
    total = max(r[0] + r[1] for r in reqs)
    canvas = np.zeros(total, dtype=np.int64)
    for row_start, num_rows, seed, step in reqs:
        for j in range(num_rows):
            canvas[row_start + j] = renoise_token(seed, step, j, vocab, STREAM_INIT)
    return canvas

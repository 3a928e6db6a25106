"""Pins for the sampler oracle: closed-form entropies, scipy's entropy, shift
invariance, brute-force acceptance over all subsets, exact quantile checks of the
inverse-CDF draw, Philox against numpy's Philox, and hand-worked fixtures.

Pages: [P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM",
section "샘플링 루프와 엔트로피 경계 디노이징"; [P3] "DiffusionGemma u vLLM: prvi
diskretni difuzijski model ...", section "Mehanizam odlučivanja o gotovim tokenima".
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.stats

from oracle.philox import philox4x64_10, uniform24, renoise_token, MASK64
from oracle.sampler import (row_stats, candidate, select, convergence, sampler_step,
                            CONV_AND, CONV_OR, CONF_MAX_PROB, FIXED_SHIFT)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- row statistics --------------------------------------------------------------------

@pytest.mark.parametrize("V", [1, 2, 8, 4096])
def test_all_equal_row(V):
    """P-S1: an all-equal row has H = ln V, Z = V, argmax 0, max probability 1/V."""
    st = row_stats(np.full((1, V), 3.25))
    assert st["argmax"][0] == 0
    assert abs(st["entropy"][0] - math.log(V)) < 1e-12
    assert abs(st["sum"][0] - V) < 1e-9
    assert abs(st["max_prob"][0] - 1.0 / V) < 1e-15


def test_one_hot_row():
    """P-S2: one finite entry among -inf gives H = 0 and that token as argmax."""
    row = np.full((1, 16), -np.inf)
    row[0, 11] = 2.0
    st = row_stats(row)
    assert st["entropy"][0] == 0.0 and st["argmax"][0] == 11 and st["sum"][0] == 1.0


@pytest.mark.parametrize("V,n,x,y", [(8, 3, 1.0, -0.5), (100, 1, 5.0, 0.0), (4096, 17, 0.25, -2.0)])
def test_two_level_closed_form(V, n, x, y):
    """P-S3: n logits at x and V-n at y have
    H = -n a ln a - (V-n) b ln b with a = e^x / (n e^x + (V-n) e^y), b likewise."""
    row = np.full(V, y)
    row[:n] = x
    zz = n * math.exp(x) + (V - n) * math.exp(y)
    a, b = math.exp(x) / zz, math.exp(y) / zz
    want = -n * a * math.log(a) - (V - n) * b * math.log(b)
    st = row_stats(row[None])
    assert abs(st["entropy"][0] - want) < 1e-12
    assert st["argmax"][0] == (0 if x > y else n)


def test_entropy_matches_scipy_and_shift_invariance():
    """P-S3/P-S4: random rows match scipy.stats.entropy of their softmax; adding a
    constant to a row changes nothing."""
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((6, 50)) * np.array([0.1, 0.5, 1, 3, 10, 30])[:, None]
    st = row_stats(rows)
    for r in range(6):
        e = np.exp(rows[r] - rows[r].max())
        assert abs(st["entropy"][r] - scipy.stats.entropy(e / e.sum())) < 1e-12
    st2 = row_stats(rows + 7.0)
    for key in ("entropy", "sum", "max_prob"):
        np.testing.assert_allclose(st2[key], st[key], rtol=1e-12, atol=1e-13)
    assert np.array_equal(st2["argmax"], st["argmax"])


def test_argmax_lowest_index_on_ties():
    row = np.array([[0.0, 5.0, 1.0, 5.0, 5.0]])
    assert row_stats(row)["argmax"][0] == 1


def test_all_minus_inf_row_rejected():
    with pytest.raises(ValueError):
        row_stats(np.full((1, 4), -np.inf))


# ---- candidate draw --------------------------------------------------------------------

def test_candidate_exact_quantiles():
    """P-S6: with evenly spaced u the draw returns each token exactly as often as its
    probability mass predicts (inverse CDF), for a row with known probabilities."""
    p = np.array([1, 2, 0, 5, 0, 8], dtype=np.float64) / 16.0
    logits = np.where(p > 0, np.log(np.where(p > 0, p, 1)), -np.inf)
    counts = np.zeros(6, dtype=int)
    n = 16 * 64
    for j in range(n):
        counts[candidate(logits, (j + 0.5) / n)] += 1
    assert list(counts) == [64, 128, 0, 320, 0, 512]
    assert candidate(logits, 1.0) == 5  # u above the total: last token with mass


def test_candidate_boundaries_are_strict():
    """The draw is the first token whose cumulative mass is strictly above u: u = 0
    never picks a zero-mass token, and u on a cumulative boundary moves to the next."""
    p = np.array([0.0, 0.25, 0.25, 0.5])
    logits = np.where(p > 0, np.log(np.where(p > 0, p, 1)), -np.inf)
    assert candidate(logits, 0.0) == 1
    assert candidate(logits, 0.25) == 2
    assert candidate(logits, 0.5) == 3


def test_candidate_chi_square_with_philox_uniforms():
    """P-S6: draws driven by the Philox uniforms follow the softmax (chi-square, V = 8)."""
    logits = np.log(np.array([0.05, 0.1, 0.15, 0.2, 0.05, 0.25, 0.1, 0.1]))
    p = np.exp(logits) / np.exp(logits).sum()
    n = 20000
    counts = np.zeros(8)
    for j in range(n):
        counts[candidate(logits, uniform24(12345, 7, j))] += 1
    chi2 = scipy.stats.chisquare(counts, n * p)
    assert chi2.pvalue > 1e-3


# ---- Philox ----------------------------------------------------------------------------

@pytest.mark.parametrize("counter,key", [((0, 0, 0, 0), (0, 0)), ((5, 7, 1, 0), (123, 0)),
                                         ((1, 2, 3, 4), (2**63 + 5, 99)),
                                         ((MASK64, MASK64, 0, 9), (0xDEADBEEF, 0xFEED))])
def test_philox_matches_numpy(counter, key):
    """P-S7: numpy's Philox4x64-10 increments its 256-bit counter before each block,
    so the block for counter c is the first output from state c - 1."""
    c = sum(int(x) << (64 * i) for i, x in enumerate(counter))
    prev = (c - 1) % (1 << 256)
    state = [(prev >> (64 * i)) & MASK64 for i in range(4)]
    # exact uint64 arrays: a Python list of large ints would pass through float64
    bg = np.random.Philox(counter=np.array(state, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    want = tuple(int(x) for x in bg.random_raw(4))
    assert philox4x64_10(counter, key) == want


def test_uniform_and_renoise_ranges():
    us = [uniform24(1, 0, j) for j in range(2000)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert all(float(np.float32(u)) == u for u in us)  # 24 bits: exact in float32
    assert 0.45 < np.mean(us) < 0.55
    toks = [renoise_token(9, 3, j, 10) for j in range(5000)]
    assert min(toks) == 0 and max(toks) == 9
    assert scipy.stats.chisquare(np.bincount(toks, minlength=10)).pvalue > 1e-3


# ---- acceptance ------------------------------------------------------------------------

def test_acceptance_hand_fixture():
    with open(os.path.join(GOLDEN, "acceptance_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        h = np.array(c["entropy"], dtype=np.float32)
        got = select(h, -h, c["budget"], c["min_accept"])
        assert list(got) == c["accept"], c["why"]


def _brute_force_accept(h32, conf32, budget, min_accept):
    """Among all subsets that are closed under 'more confident than a member' and whose
    exact entropy total fits the budget, the largest one (or the min_accept most
    confident positions if that is larger)."""
    n = len(h32)
    key = [(-float(conf32[i]), i) for i in range(n)]
    fixed = [math.floor(float(h32[i]) * 2.0 ** FIXED_SHIFT) for i in range(n)]
    limit = math.floor(float(np.float32(budget)) * 2.0 ** FIXED_SHIFT)
    best = frozenset()
    for bits in range(1 << n):
        s = frozenset(i for i in range(n) if bits >> i & 1)
        closed = all(j in s for i in s for j in range(n) if key[j] < key[i])
        if closed and sum(fixed[i] for i in s) <= limit and len(s) > len(best):
            best = s
    forced = frozenset(sorted(range(n), key=lambda i: key[i])[:min(min_accept, n)])
    return best if len(best) >= len(forced) else forced


@pytest.mark.parametrize("trial", range(40))
def test_acceptance_brute_force(trial):
    """P-S5: the oracle's accepted set equals the brute-force optimum on N <= 10, and
    the three invariants hold (ordering, budget, maximality)."""
    rng = np.random.default_rng(100 + trial)
    n = int(rng.integers(1, 11))
    h = rng.choice([0.0, 0.25, 0.5, 1.0, 1.5, 2.0, 3.0], size=n).astype(np.float32) \
        if trial % 2 else (rng.random(n) * 4).astype(np.float32)
    budget = float(rng.random() * 8)
    min_accept = int(rng.integers(0, 3))
    conf = -h if trial % 3 else rng.random(n).astype(np.float32)
    got = select(h, conf, budget, min_accept)
    want = _brute_force_accept(h, conf, budget, min_accept)
    assert set(np.nonzero(got)[0]) == set(want)
    acc = [i for i in range(n) if got[i]]
    rej = [i for i in range(n) if not got[i]]
    key = lambda i: (-float(conf[i]), i)
    if acc and rej:
        assert max(key(i) for i in acc) < min(key(i) for i in rej)
    if len(acc) > min(min_accept, n):
        assert float(np.sum(h[acc].astype(np.float64))) <= np.float32(budget) + 1e-9
    if rej:
        nxt = min(rej, key=key)
        assert float(np.sum(h[acc].astype(np.float64))) + float(h[nxt]) > np.float32(budget) - 1e-9 \
            or len(acc) <= min(min_accept, n)


def test_acceptance_budget_never_binds_above_ln_v():
    """With B > ln V even one position of maximal entropy is always affordable."""
    h = np.full(256, np.float32(math.log(262144)))
    acc = select(h, -h, 128.0, 1)
    assert acc.sum() == int(128.0 // float(h[0]))


# ---- convergence -----------------------------------------------------------------------

def test_convergence_hand_fixture():
    with open(os.path.join(GOLDEN, "convergence_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        for name, comb in (("and", CONV_AND), ("or", CONV_OR)):
            stable, prev, first = 0, None, None
            for t, (am, me) in enumerate(zip(c["argmax"], c["mean_entropy"])):
                am = np.array(am)
                h = np.full(len(am), me, dtype=np.float32)
                conv, stable, mean = convergence(am, prev if prev is not None else am * 0 - 1, stable, t, h,
                                                 c["tau"], c["stable_k"], c["step_limit"], comb)
                assert stable == c["stable"][t], (c["why"], t)
                assert abs(mean - me) < 1e-12
                if conv and first is None:
                    first = t
                prev = am
            assert first == c["first_converged"][name], (name, c["why"])


# ---- whole step --------------------------------------------------------------------------

def test_sampler_step_canvas_rules():
    """Accepted positions take their candidate, the rest a re-noise token (or keep
    their token with re-noising off); on the converging step the rest take the argmax."""
    rng = np.random.default_rng(5)
    V = 32
    logits = rng.standard_normal((12, V)) * np.linspace(0.1, 8, 12)[:, None]
    reqs = [(0, 8, 77, 0), (8, 4, 88, 2)]
    canvas = np.arange(12) % V
    prev = np.full(12, -1)
    out = sampler_step(logits, reqs, V, budget=3.0, min_accept=1, canvas=canvas, prev_argmax=prev,
                       stable_count=[0, 0], step_limit=48)
    assert not out["converged"].any()
    for (row_start, n, seed, step) in reqs:
        for j in range(n):
            i = row_start + j
            if out["accept"][i]:
                assert out["canvas"][i] == out["cand"][i]
            else:
                assert out["canvas"][i] == renoise_token(seed, step, j, V)
    keep = sampler_step(logits, reqs, V, 3.0, 1, canvas, prev, [0, 0], renoise=False)
    assert np.array_equal(keep["canvas"][~keep["accept"]], canvas[~keep["accept"]])
    last = sampler_step(logits, reqs, V, 3.0, 1, canvas, prev, [0, 0], step_limit=1)
    assert last["converged"].all()
    st = last["stats"]
    assert np.array_equal(last["canvas"][~last["accept"]], st["argmax"][~last["accept"]])
    assert np.array_equal(last["prev_argmax"], st["argmax"])
    mp = sampler_step(logits, reqs, V, 3.0, 1, canvas, prev, [0, 0], conf_mode=CONF_MAX_PROB)
    assert np.allclose(mp["conf32"], (1.0 / st["sum"]).astype(np.float32))

"""GPU parity of dg_sampler_step against the CPU oracle, through the C ABI.

Bars: fp32 entropies within 1e-5 absolute; argmax and row max exact; acceptance
masks, canvas re-noise tokens and convergence bookkeeping bit-exact when the GPU
selection is fed the oracle's entropies (DG_ENTROPY_IN); candidates, being random
draws, are checked by the bracket test C(c-1) - 1e-6 <= u < C(c) + 1e-6 against the
oracle's float64 CDF with the same Philox uniform (the kernels' fp32 sums put the
draw's target within 190 * 2^-24 = 1.1e-5 of the exact one at worst; the largest
distance from a bracket measured over 30,720 full-size draws is 1.5e-7).
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from oracle.philox import uniform24, renoise_token, STREAM_INIT
from oracle.sampler import sampler_step, row_stats, CONV_AND, CONV_OR, CONF_MAX_PROB, CONF_NEG_ENTROPY
from workloads import logits as synth_logits, sampler_case, request_seeds, round_to_bf16
from tests.gpu_util import DEV, dev, host, say

pytestmark = pytest.mark.gpu


def _bracket_ok(row: np.ndarray, u: float, c: int, tol: float = 1e-6) -> bool:
    l = row.astype(np.float64)
    p = np.exp(l - l.max())
    p /= p.sum()
    if not (0 <= c < len(p)) or p[c] == 0:
        return False
    cdf = np.cumsum(p)
    lo = cdf[c - 1] if c > 0 else 0.0
    return lo - tol <= u < cdf[c] + tol


def _run(logits_np, bf16, reqs, V, budget, min_accept=1, conf_mode=CONF_NEG_ENTROPY, renoise=1, stable_k=3,
         tau=0.05, step_limit=48, combine=CONV_AND, canvas0=None, prev0=None, stable0=None, ld=None, label=""):
    """Run the GPU step twice (own entropies; oracle entropies fed in) and compare."""
    say(f"[sampler] {label}: M={logits_np.shape[0]} V={V} bf16={bf16} reqs={len(reqs)}")
    M = logits_np.shape[0]
    R = len(reqs)
    rng = np.random.default_rng(7)
    canvas0 = rng.integers(0, V, M).astype(np.int32) if canvas0 is None else canvas0
    prev0 = np.full(M, -1, np.int32) if prev0 is None else prev0
    stable0 = np.zeros(R, np.int32) if stable0 is None else stable0
    if ld is not None and ld != V:
        full = np.full((M, ld), -7.0, np.float32)  # padding past V must be ignored
        full[:, :V] = logits_np
        lt = dev(full, bf16)[:, :V]
    else:
        lt = dev(logits_np, bf16)
    kw = dict(min_accept=min_accept, conf_mode=conf_mode, renoise=renoise, stable_k=stable_k, tau=tau,
              step_limit=step_limit, combine=combine)

    def fresh():
        b = dg.SamplerBuffers(M, R, DEV)
        b.canvas.copy_(torch.from_numpy(canvas0))
        b.prev_argmax.copy_(torch.from_numpy(prev0))
        b.stable_count.copy_(torch.from_numpy(stable0))
        return b

    b = fresh()
    dg.dg_sampler_step(lt, reqs, V, b, budget, **kw)
    torch.cuda.synchronize()
    ref = sampler_step(logits_np, reqs, V, budget, min_accept, canvas0.astype(np.int64), prev0.astype(np.int64),
                       stable0, conf_mode=conf_mode, renoise=bool(renoise), stable_k=stable_k, tau=tau,
                       step_limit=step_limit, combine=combine, with_candidates=False)
    st = ref["stats"]
    covered = np.zeros(M, bool)
    for (r0, n, _, _) in reqs:
        covered[r0:r0 + n] = True
    ent = host(b.entropy)
    err = np.abs(ent.astype(np.float64) - st["entropy"]).max()
    say(f"  entropy max abs err {err:.3e}")
    assert err <= 1e-5
    assert np.array_equal(host(b.argmax), st["argmax"].astype(np.int32))
    assert np.array_equal(host(b.row_max).astype(np.float64), st["max"])
    # Row sums are fp32: a lane adds its 64 terms in sequence (63 roundings), a
    # 256-thread tree adds 8 levels, and up to 16 chunk sums are merged in order with
    # one scaling each; about 90 roundings of 2^-24 (5.4e-6) in the worst case, plus
    # under 3e-7 from the fp32 exponent arguments of the dominant terms.
    np.testing.assert_allclose(host(b.row_sum), st["sum"], rtol=1e-5)
    if conf_mode == CONF_MAX_PROB:
        np.testing.assert_allclose(host(b.conf), st["max_prob"], rtol=1e-5)
    else:
        assert np.array_equal(host(b.conf), -ent)
    cand = host(b.cand)
    for (r0, n, seed, step) in reqs:
        for j in range(n):
            u = uniform24(seed, step, j)
            assert _bracket_ok(logits_np[r0 + j], u, int(cand[r0 + j])), (label, r0 + j, cand[r0 + j])
    assert np.all(cand[~covered] == -1)

    # selection replayed on the oracle's entropies: bit-exact
    b2 = fresh()
    b2.entropy.copy_(torch.from_numpy(ref["entropy32"]))
    if conf_mode == CONF_MAX_PROB:
        b2.conf.copy_(torch.from_numpy(st["max_prob"].astype(np.float32)))
    dg.dg_sampler_step(lt, reqs, V, b2, budget, flags=dg.DG_ENTROPY_IN, **kw)
    torch.cuda.synchronize()
    conf_in = st["max_prob"].astype(np.float32) if conf_mode == CONF_MAX_PROB else None
    ref2 = sampler_step(logits_np, reqs, V, budget, min_accept, canvas0.astype(np.int64), prev0.astype(np.int64),
                        stable0, conf_mode=conf_mode, renoise=bool(renoise), stable_k=stable_k, tau=tau,
                        step_limit=step_limit, combine=combine, entropy_in=ref["entropy32"], conf_in=conf_in,
                        with_candidates=False)
    acc = host(b2.accept).astype(bool)
    assert np.array_equal(acc[covered], ref2["accept"][covered]), label
    canvas = host(b2.canvas)
    cand2 = host(b2.cand)
    want = ref2["canvas"].copy()
    want[ref2["accept"]] = cand2[ref2["accept"]]  # accepted positions take the GPU's own draw
    assert np.array_equal(canvas[covered], want[covered].astype(np.int32)), label
    assert np.array_equal(canvas[~covered], canvas0[~covered])
    assert np.array_equal(host(b2.prev_argmax)[covered], ref2["prev_argmax"][covered].astype(np.int32))
    assert np.array_equal(host(b2.stable_count), ref2["stable_count"].astype(np.int32))
    assert np.array_equal(host(b2.converged).astype(bool), ref2["converged"])
    assert np.array_equal(host(b2.num_accepted), ref2["num_accepted"].astype(np.int32))
    np.testing.assert_allclose(host(b2.mean_entropy), ref2["mean_entropy"], rtol=1e-6, atol=1e-7)
    say(f"  ok: accepted {ref2['num_accepted'].tolist()} converged {ref2['converged'].tolist()}")
    return b2, ref2


def test_fp32_256x4096():
    c = sampler_case(1)
    l = synth_logits(1, c.total_rows, c.vocab, bf16=False)
    _run(l, False, [(0, 256, request_seeds(1, 1)[0], 0)], c.vocab, c.budget, label="fp32 256x4096")


def test_bf16_256x262144():
    c = sampler_case(2)
    l = synth_logits(2, c.total_rows, c.vocab, bf16=True)
    _run(l, True, [(0, 256, request_seeds(2, 1)[0], 0)], c.vocab, c.budget, label="bf16 256x262144")


def test_bf16_two_denoise_requests_512x262144():
    c = sampler_case(4)
    l = synth_logits(4, c.total_rows, c.vocab, bf16=True)
    s = request_seeds(4, 2)
    _run(l, True, [(0, 256, s[0], 3), (256, 256, s[1], 5)], c.vocab, c.budget, label="bf16 two requests 512x262144")


def test_bf16_four_long_context_requests_1024x262144():
    """The long-context batch: four 256-position canvases in one call, at different steps."""
    c = sampler_case(5)
    l = synth_logits(5, c.total_rows, c.vocab, bf16=True)
    s = request_seeds(5, 4)
    _run(l, True, [(0, 256, s[0], 0), (256, 256, s[1], 7), (512, 256, s[2], 2), (768, 256, s[3], 30)], c.vocab,
         c.budget, label="bf16 four requests 1024x262144")


@pytest.mark.parametrize("bf16", [False, True])
def test_edge_rows(bf16):
    """-inf entries, a one-hot row, an all-equal row, argmax ties, tiny vocabulary."""
    V = 8
    rows = np.array([
        [0, 0, 0, 0, 0, 0, 0, 0],
        [-np.inf, -np.inf, 3, -np.inf, -np.inf, -np.inf, -np.inf, -np.inf],
        [1, 5, 2, 5, -np.inf, 5, 0, -1],
        [-np.inf, 0.5, 0.25, -np.inf, 2, 2, -3, 1],
        [100, 99, 98, -100, -np.inf, 0, 1, 2],
        [-30, -30.5, -31, -29, -29, -40, -np.inf, -35],
    ], dtype=np.float32)
    l = round_to_bf16(rows) if bf16 else rows
    _run(l, bf16, [(0, 3, 11, 0), (3, 3, 12, 4)], V, budget=1.0, label=f"edge rows bf16={bf16}")


@pytest.mark.parametrize("bf16,V,ld", [(False, 5003, 5008), (True, 16390, 16392), (True, 40000, 40000),
                                       (False, 12, 16)])
def test_ragged_vocab_and_row_stride(bf16, V, ld):
    """Vocabularies that end mid-chunk and mid-vector, with padded rows (ld > V)."""
    rng = np.random.default_rng(V)
    l = (rng.standard_normal((37, V)) * rng.uniform(0.1, 10, (37, 1))).astype(np.float32)
    if bf16:
        l = round_to_bf16(l)
    _run(l, bf16, [(0, 20, 5, 1), (20, 17, 6, 2)], V, budget=6.0, ld=ld, label=f"ragged V={V} ld={ld}")


def test_rows_outside_requests_and_options():
    """Rows no request covers keep their canvas and get cand -1; max-probability
    confidence, no re-noising, min_accept, both convergence combinators."""
    rng = np.random.default_rng(3)
    V = 1000
    l = round_to_bf16((rng.standard_normal((12, V)) * rng.uniform(0.1, 5, (12, 1))).astype(np.float32))
    reqs = [(2, 4, 99, 2), (7, 3, 98, 0)]
    for kw in (dict(conf_mode=CONF_MAX_PROB), dict(renoise=0), dict(min_accept=3, budget=0.0),
               dict(combine=CONV_OR, tau=50.0), dict(step_limit=1)):
        budget = kw.pop("budget", 4.0)
        _run(l, True, reqs, V, budget, label=f"options {kw}", **kw)


def test_stability_counting_and_convergence():
    """prev_argmax equal to this step's argmax counts as a stable step (step > 0)."""
    rng = np.random.default_rng(4)
    V = 296  # row stride must be a multiple of 8
    l = (rng.standard_normal((16, V)) * 4).astype(np.float32)
    am = row_stats(l)["argmax"].astype(np.int32)
    prev = am.copy()
    prev[12] = (prev[12] + 1) % V  # second request not stable
    for comb in (CONV_AND, CONV_OR):
        _run(l, False, [(0, 10, 1, 4), (10, 6, 2, 4)], V, 8.0, prev0=prev, stable0=np.array([2, 5], np.int32),
             stable_k=3, tau=5.0, combine=comb, label=f"stability comb={comb}")


def test_selection_ties_and_signed_zero_entropies():
    """Entropies fed in (DG_ENTROPY_IN) in groups of exactly equal values, with +0 and
    -0 among them (equal confidences) and a budget that cuts inside a tie group: ties
    rank by position, so the accepted set is the oracle's bit for bit."""
    M, V = 256, 64
    rng = np.random.default_rng(21)
    l = (rng.standard_normal((M, V)) * 2).astype(np.float32)
    vals = np.array([0.0, -0.0, 0.75, 0.75, 1.5, 0.125, 2.0, 0.125], np.float32)
    ent = np.repeat(vals, M // len(vals))[rng.permutation(M)].astype(np.float32)
    ent[rng.integers(0, M, 20)] = -0.0
    for budget in (3.3, 10.0, 40.1):
        ref = sampler_step(l, [(0, M, 3, 1)], V, budget, 1, np.zeros(M, np.int64), np.full(M, -1, np.int64), [0],
                           entropy_in=ent, with_candidates=False)
        b = dg.SamplerBuffers(M, 1, DEV)
        b.entropy.copy_(torch.from_numpy(ent))
        dg.dg_sampler_step(dev(l), [(0, M, 3, 1)], V, b, budget, flags=dg.DG_ENTROPY_IN)
        torch.cuda.synchronize()
        acc = host(b.accept).astype(bool)
        say(f"[sampler] ties, budget {budget}: accepted {int(acc.sum())} (oracle {int(ref['accept'].sum())})")
        assert np.array_equal(acc, ref["accept"])
        assert host(b.num_accepted)[0] == ref["num_accepted"][0]
        # a tie group straddles the cut: its accepted members are its lowest positions
        assert 0 < acc.sum() < M


def test_converged_flag_into_pinned_host_memory():
    """The selection writes the converged flag straight into pinned host memory (read
    by the host after the step completes, with no copy on the stream); over several
    steps in a row, alternating between two host slots, every flag equals the one the
    same step writes to a device buffer."""
    rng = np.random.default_rng(11)
    V = 512
    l = dev((rng.standard_normal((64, V)) * 6).astype(np.float32))
    reqs = [(0, 40, 5, 0), (40, 24, 6, 0)]
    host_slots = torch.zeros(2, 2, dtype=torch.int32, pin_memory=True)
    bd, bh = dg.SamplerBuffers(64, 2, DEV), dg.SamplerBuffers(64, 2, DEV)
    for t in range(6):
        r = [(r0, n, sd, t) for (r0, n, sd, _) in reqs]
        dg.dg_sampler_step(l, r, V, bd, 2.0, stable_k=2, tau=0.0, combine=CONV_OR)
        ph = dg.prepare_sampler(l, r, V, bh, 2.0, stable_k=2, tau=0.0, combine=CONV_OR)
        ph.args.converged = host_slots[t % 2].data_ptr()
        ph()
        ev = torch.cuda.Event()
        ev.record()
        ev.synchronize()
        want = host(bd.converged)
        say(f"[sampler] pinned flag step {t}: {host_slots[t % 2].tolist()} (device {want.tolist()})")
        assert np.array_equal(host_slots[t % 2].numpy(), want)
    assert host_slots[1].tolist() == [1, 1]  # the logits never change: stable for 2 steps by step 2


def test_init_canvas():
    M, V = 300, 262144
    b = dg.SamplerBuffers(M, 2, DEV)
    reqs = [(0, 256, 1234, 0), (256, 44, 5678, 9)]
    dg.dg_sampler_step(None, reqs, V, b, 128.0, flags=dg.DG_INIT_CANVAS, num_rows=M)
    torch.cuda.synchronize()
    canvas = host(b.canvas)
    for (r0, n, seed, step) in reqs:
        want = [renoise_token(seed, step, j, V, STREAM_INIT) for j in range(n)]
        assert np.array_equal(canvas[r0:r0 + n], np.array(want, np.int32))
    assert np.all(host(b.prev_argmax) == -1) and np.all(host(b.stable_count) == 0)
    assert np.all(host(b.converged) == 0)


def test_repeat_is_bit_identical():
    c = sampler_case(1)
    l = dev(synth_logits(1, 256, c.vocab, bf16=False))
    outs = []
    for _ in range(2):
        b = dg.SamplerBuffers(256, 1, DEV)
        dg.dg_sampler_step(l, [(0, 256, 42, 3)], c.vocab, b, c.budget)
        torch.cuda.synchronize()
        outs.append([host(getattr(b, n)).copy() for n in ("entropy", "row_sum", "cand", "accept", "canvas")])
    for a, bb in zip(*outs):
        assert np.array_equal(a, bb)


def test_split_call_equals_one_call():
    """DG_SKIP_SELECT then DG_SELECT_ONLY (same arguments) give exactly the results of one
    call, over three steps of two requests with their state carried."""
    c = sampler_case(4)
    V, M = 40000, 512
    l = dev(synth_logits(4, M, V, bf16=True), True)
    reqs0 = [(0, 256, 11, 0), (256, 256, 12, 0)]
    names = ("entropy", "conf", "row_max", "row_sum", "argmax", "cand", "accept", "canvas", "prev_argmax",
             "stable_count", "num_accepted", "converged", "mean_entropy", "probs", "probs_scale")
    bufs = []
    for _ in range(2):
        b = dg.SamplerBuffers(M, 2, DEV, vocab=V, probs_dtype=torch.bfloat16)
        dg.dg_sampler_step(None, reqs0, V, b, c.budget, flags=dg.DG_INIT_CANVAS, num_rows=M)
        bufs.append(b)
    for step in range(3):
        reqs = [(r0, n, seed, step) for r0, n, seed, _ in reqs0]
        dg.dg_sampler_step(l, reqs, V, bufs[0], c.budget)
        dg.dg_sampler_step(l, reqs, V, bufs[1], c.budget, flags=dg.DG_SKIP_SELECT)
        dg.dg_sampler_step(None, reqs, V, bufs[1], c.budget, flags=dg.DG_SELECT_ONLY, num_rows=M)
        torch.cuda.synchronize()
        for n in names:
            a, b = host(getattr(bufs[0], n)), host(getattr(bufs[1], n))
            assert np.array_equal(a, b, equal_nan=True), (step, n)
    say("[sampler] split call == one call over 3 steps")


@pytest.mark.parametrize("bf16,V", [(True, 262144), (False, 4096), (True, 40000), (False, 12)])
def test_block_scaled_probabilities(bf16, V):
    """w * scale per DG_PROB_BLOCK reproduces the softmax: within the rounding of w to the
    logits dtype (unit roundoff 2^-8 for bf16) plus fp32 arithmetic in the scale
    (1e-5 relative), and exactly 0 where p is 0."""
    rng = np.random.default_rng(V + bf16)
    M = 40 if V > 100000 else 9
    l = (rng.standard_normal((M, V)) * rng.uniform(0.1, 10, (M, 1))).astype(np.float32)
    l[1, ::3] = -np.inf
    if bf16:
        l = round_to_bf16(l)
    ld = (V + 7) // 8 * 8
    full = np.zeros((M, ld), np.float32)
    full[:, :V] = l
    lt = dev(full, bf16)[:, :V]
    b = dg.SamplerBuffers(M, 1, DEV, vocab=V, probs_dtype=lt.dtype)
    dg.dg_sampler_step(lt, [(0, M, 3, 0)], V, b, 16.0)
    torch.cuda.synchronize()
    w = host(b.probs).astype(np.float64)
    sc = host(b.probs_scale).astype(np.float64)
    blk = np.arange(V) // dg.DG_PROB_BLOCK
    p = w * sc[:, blk]
    ref = np.exp(l.astype(np.float64) - l.max(axis=1, keepdims=True))
    ref /= ref.sum(axis=1, keepdims=True)
    tol = 2.0 ** -8 + 1e-5 if bf16 else 1e-5
    nz = ref > 1e-30
    rel = np.abs(p[nz] - ref[nz]) / ref[nz]
    say(f"[sampler] block-scaled probs V={V} bf16={bf16}: max rel {rel.max():.3e}")
    assert rel.max() <= tol
    assert np.all(p[ref == 0] == 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=2e-3 if bf16 else 1e-5)


def test_selection_max_canvas_1024():
    """One request of DG_MAX_CANVAS = 1024 positions (four positions per thread of the
    selection's rank sort), with a previous state: entropies, argmax, candidates and,
    with the oracle's entropies fed in, the selection bit-exact."""
    M, V = 1024, 16384
    rng = np.random.default_rng(1024)
    l = round_to_bf16((rng.standard_normal((M, V)) * np.exp(rng.uniform(np.log(0.1), np.log(10), (M, 1))))
                      .astype(np.float32))
    prev = row_stats(l)["argmax"].astype(np.int32)
    prev[rng.integers(0, M, 5)] += 1  # a few positions changed their argmax
    for budget, comb in ((128.0, CONV_OR), (700.0, CONV_AND), (5000.0, CONV_AND)):
        _run(l, True, [(0, M, 777, 6)], V, budget, prev0=prev, stable0=np.array([4], np.int32), combine=comb,
             label=f"canvas 1024 budget {budget}")


def test_max_requests_64():
    """DG_MAX_REQS = 64 requests in one call: ragged canvases (1 to 40 positions, rows
    between them that no request owns), each at its own step and seed with its own
    stable count; everything per request against the oracle."""
    rng = np.random.default_rng(64)
    V = 4096
    reqs, row = [], 0
    for r in range(64):
        row += int(rng.integers(0, 3))  # gaps: rows outside every request
        n = int(rng.integers(1, 41))
        reqs.append((row, n, int(rng.integers(0, 2**63 - 1)), int(rng.integers(0, 20))))
        row += n
    M = row + 2
    l = (rng.standard_normal((M, V)) * np.exp(rng.uniform(np.log(0.1), np.log(10), (M, 1)))).astype(np.float32)
    prev = row_stats(l)["argmax"].astype(np.int32)
    prev[rng.integers(0, M, 20)] += 1
    stable0 = rng.integers(0, 5, 64).astype(np.int32)
    for comb in (CONV_AND, CONV_OR):
        _run(l, False, reqs, V, 9.0, prev0=prev, stable0=stable0, combine=comb, tau=2.5,
             label=f"64 requests comb={comb}")


def test_vocab_540000_33_chunks():
    """A vocabulary of 540000 bf16 entries: 33 row-pass chunks, the last one ragged (the
    finalize merges more chunk statistics than one per lane of its first pass)."""
    rng = np.random.default_rng(540000)
    V = 540000
    l = round_to_bf16((rng.standard_normal((9, V)) * rng.uniform(0.1, 10, (9, 1))).astype(np.float32))
    _run(l, True, [(0, 5, 31, 2), (6, 3, 32, 0)], V, budget=20.0, label="vocab 540000 (33 chunks)")

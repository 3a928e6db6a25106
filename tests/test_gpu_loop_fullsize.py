"""The 256-position canvas's denoise loop at its full size, every step against the oracle,
through the C ABI and the same step driver the benchmark times.

Workload: bf16 attention of a 256-token bidirectional canvas over a 4096-token prefix
(16 query / 8 KV heads x 256), the sampler over bf16 logits [256 x 262144] with a
128-nat budget, self-conditioning against a bf16 embedding table [262144 x 2048]. The
logits of step t come from the synthetic loop driver (position i reads its settled
pool row once i < 32 t, a noise row before), so every position has settled by step 8.
The loop ([P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion
LLM", section "샘플링 루프와 엔트로피 경계 디노이징") runs under both convergence rules:
  * stable >= 3 or mean entropy < 0.05 or 48 steps: converges after 12 steps;
  * (stable >= 3 and mean entropy < 0.05) or 48 steps: the mean entropy never falls
    under 0.05 with these logits, so it runs to the 48-step limit.

Two chains run side by side on the GPU, each step:
  A. the step exactly as the benchmark runs it (the GPU's own entropies). Checked:
     entropies within 1e-5 of the oracle's; argmax exact; every candidate inside the
     oracle's float64 CDF bracket of its uniform; the selection, canvas, stable count,
     converged flag and mean entropy bit-exact with the oracle's selection run on the
     entropies the GPU stored (and on the GPU chain's own previous state);
  B. the same step with the oracle's entropies fed in (DG_ENTROPY_IN), against the
     oracle's own chain: accepted set, canvas, previous argmax, stable count, accepted
     count, converged flag and mean entropy bit-exact at every step (accepted positions
     take the GPU's candidate, a random draw checked by its bracket).
Attention and self-conditioning are checked at step 0 and at the last step on sampled
rows (max-relative error per row <= 2e-2).
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from block_denoising_step_amd.step import DenoiseStep
from oracle.attn import attn_mixed
from oracle.philox import uniform24, renoise_token
from oracle.sampler import row_stats, sampler_step, init_canvas, select, convergence, CONV_AND, CONV_OR
from oracle.selfcond import selfcond_embed
from workloads import attn_case, embed_table, driver_pool, driver_rows, request_seeds
from tests.gpu_util import DEV, host, max_rel_rows, say

pytestmark = pytest.mark.gpu

CANVAS, HQ, HKV = 256, 16, 8
VOCAB, EMBED = 262144, 2048
BUDGET, STABLE_K, TAU, LIMIT = 128.0, 3, 0.05, 48
SETTLE = 9  # steps >= 8 read the settled rows: 9 distinct logits tensors cover every step
# Bracket slack of a candidate against the float64 CDF. The kernels sum 2^y terms in fp32
# along a path of at most about 190 roundings (64-term lane sums, block and wave trees,
# the chunk merge, the three scans of the draw), so the assured bound is 190 * 2^-24 =
# 1.1e-5; the errors are far smaller in practice (largest distance from a bracket over
# the 30,720 draws of both loops: 1.5e-7), and the bar is set at 1e-6, under a third of
# one token's mass on the flattest rows (p = 3.8e-6 at 262144 entries).
CAND_TOL = 1e-6
ATTN_ROWS = [0, 1, 63, 64, 127, 128, 191, 192, 255]
SC_ROWS = [0, 31, 32, 128, 200, 255]


@pytest.fixture(scope="module")
def world():
    say("[loop] drawing the inputs (attention case, embedding table, driver pool)")
    case = attn_case(2)
    q_np, k_np, v_np = case.tensors()
    E_np = embed_table(2, VOCAB, EMBED, bf16=True)
    pool_np = driver_pool(VOCAB, bf16=True)
    say("[loop] oracle statistics and CDFs of the 512 pool rows")
    stats = {}
    cdf = np.empty(pool_np.shape, np.float64)
    for i in range(0, pool_np.shape[0], 32):
        st = row_stats(pool_np[i:i + 32])
        for key, val in st.items():
            stats.setdefault(key, []).append(val)
        l = pool_np[i:i + 32].astype(np.float64)
        w = np.exp(l - l.max(axis=1, keepdims=True))
        np.cumsum(w / w.sum(axis=1, keepdims=True), axis=1, out=cdf[i:i + 32])
    stats = {key: np.concatenate(v) for key, v in stats.items()}
    to = lambda x: torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    q, k, v, E, pool = to(q_np), to(k_np), to(v_np), to(E_np), to(pool_np)
    logits = [pool[torch.from_numpy(driver_rows(t)).to(DEV)].contiguous() for t in range(SETTLE)]
    attn_want, attn_lse = attn_mixed(case.seqs, -1, q_np, k_np, v_np, HQ, HKV, rows=ATTN_ROWS)
    return dict(case=case, q=q, k=k, v=v, E=E, E_np=E_np, pool_np=pool_np, stats=stats, cdf=cdf, logits=logits,
                attn_want=attn_want, attn_lse=attn_lse)


def _step_stats(stats, t):
    rows = driver_rows(t)
    return {key: val[rows] for key, val in stats.items()}, rows


def _check_candidates(cdf, rows, cand, seed, t, tally):
    """Every candidate inside its CDF bracket within CAND_TOL; also tally how often it is
    the float64 inverse-CDF token itself."""
    for j in range(CANVAS):
        u = uniform24(seed, t, j)
        c = int(cand[j])
        row = cdf[rows[j]]
        assert 0 <= c < row.shape[0], (t, j, c)
        lo = row[c - 1] if c > 0 else 0.0
        assert lo - CAND_TOL <= u < row[c] + CAND_TOL, (t, j, c, u, lo, row[c])
        exact = int(np.searchsorted(row, u, side="right"))
        tally["draws"] += 1
        tally["exact"] += int(exact == c)
        tally["far"] += int(abs(exact - c) > 1)
        dist = 0.0 if lo <= u < row[c] else min(abs(u - lo), abs(u - row[c]))
        tally["max_dist"] = max(tally["max_dist"], dist)


@pytest.mark.parametrize("combine,want_steps", [(CONV_OR, 12), (CONV_AND, LIMIT)])
def test_denoise_loop_fullsize(world, combine, want_steps):
    w = world
    case = w["case"]
    seed = request_seeds(2, 1)[0]
    mk = lambda: DenoiseStep(w["q"], w["k"], w["v"], case.seqs, -1, HQ, HKV, w["logits"], w["E"], BUDGET,
                             STABLE_K, TAU, LIMIT, combine=combine, seed=seed)
    A, B = mk(), mk()
    A.start_block(seed)
    B.start_block(seed)
    torch.cuda.synchronize()
    canvas0 = init_canvas([(0, CANVAS, seed, 0)], VOCAB)
    assert np.array_equal(host(A.bufs.canvas), canvas0.astype(np.int32))
    # oracle chain (B's reference) and the A chain's previous state as the GPU left it
    o_canvas, o_prev, o_stable = canvas0.copy(), np.full(CANVAS, -1, np.int64), [0]
    a_prev = np.full(CANVAS, -1, np.int64)
    a_stable = 0
    a_canvas = canvas0.copy()
    tally = {"draws": 0, "exact": 0, "far": 0, "max_dist": 0.0}
    max_ent = 0.0
    steps = None
    for t in range(LIMIT):
        which = min(t, SETTLE - 1)
        st, rows = _step_stats(w["stats"], t)
        ent32 = st["entropy"].astype(np.float32)
        # chain B: the oracle's entropies fed in
        B.bufs.entropy.copy_(torch.from_numpy(ent32))
        A.enqueue(t, which)
        B.enqueue(t, which, flags=dg.DG_ENTROPY_IN)
        torch.cuda.synchronize()

        # ---- chain A: the benchmark's step
        ent = host(A.bufs.entropy)
        err = float(np.abs(ent.astype(np.float64) - st["entropy"]).max())
        max_ent = max(max_ent, err)
        assert err <= 1e-5, (t, err)
        am = host(A.bufs.argmax)
        assert np.array_equal(am, st["argmax"].astype(np.int32)), t
        assert np.array_equal(host(A.bufs.row_max).astype(np.float64), st["max"]), t
        cand = host(A.bufs.cand)
        _check_candidates(w["cdf"], rows, cand, seed, t, tally)
        acc = select(ent, -ent, BUDGET, 1)
        assert np.array_equal(host(A.bufs.accept).astype(bool), acc), t
        conv, stable, mean = convergence(am, a_prev, a_stable, t, ent, TAU, STABLE_K, LIMIT, combine)
        assert host(A.bufs.stable_count)[0] == stable and bool(host(A.bufs.converged)[0]) == conv, t
        assert float(host(A.bufs.mean_entropy)[0]) == np.float32(mean), t
        want = a_canvas.copy()
        want[acc] = cand[acc]
        if not conv:
            for j in np.nonzero(~acc)[0]:
                want[j] = renoise_token(seed, t, int(j), VOCAB, 1)
        else:
            want[~acc] = am[~acc]
        a_canvas = host(A.bufs.canvas).astype(np.int64)
        assert np.array_equal(a_canvas, want), t
        assert np.array_equal(host(A.bufs.prev_argmax), am), t
        a_prev, a_stable = am.astype(np.int64), stable

        # ---- chain B: fed the oracle's entropies, against the oracle's chain
        logits_t = None  # the oracle's statistics come from the pool rows (stats=)
        ref = sampler_step(logits_t, [(0, CANVAS, seed, t)], VOCAB, BUDGET, 1, o_canvas, o_prev, o_stable,
                           stable_k=STABLE_K, tau=TAU, step_limit=LIMIT, combine=combine, with_candidates=False,
                           stats=st)
        b_acc = host(B.bufs.accept).astype(bool)
        assert np.array_equal(b_acc, ref["accept"]), t
        b_cand = host(B.bufs.cand)
        _check_candidates(w["cdf"], rows, b_cand, seed, t, tally)
        want_b = ref["canvas"].copy()
        want_b[ref["accept"]] = b_cand[ref["accept"]]  # accepted positions take the GPU's own draw
        b_canvas = host(B.bufs.canvas).astype(np.int64)
        assert np.array_equal(b_canvas, want_b), t
        assert np.array_equal(host(B.bufs.prev_argmax), ref["prev_argmax"].astype(np.int32)), t
        assert host(B.bufs.stable_count)[0] == ref["stable_count"][0], t
        assert host(B.bufs.num_accepted)[0] == ref["num_accepted"][0], t
        assert bool(host(B.bufs.converged)[0]) == bool(ref["converged"][0]), t
        assert float(host(B.bufs.mean_entropy)[0]) == np.float32(ref["mean_entropy"][0]), t
        o_canvas, o_prev, o_stable = b_canvas, ref["prev_argmax"], list(ref["stable_count"])
        say(f"[loop comb={combine}] step {t}: accepted A {int(acc.sum())} B {int(b_acc.sum())}, stable {stable}, "
            f"mean H {mean:.4f}, converged {conv}; entropy err {err:.2e}")

        if t == 0 or conv:
            # attention and self-conditioning of this step on sampled rows
            aerr = max_rel_rows(host(A.attn_out)[ATTN_ROWS], w["attn_want"][ATTN_ROWS])
            lerr = float(np.abs(host(A.lse)[ATTN_ROWS] - w["attn_lse"][ATTN_ROWS]).max())
            sc_want = selfcond_embed(w["E_np"], logits=w["pool_np"][rows[SC_ROWS]])
            serr = max_rel_rows(host(A.sc_out)[SC_ROWS], sc_want)
            say(f"  step {t}: attention max-rel {aerr:.3e} lse {lerr:.2e}; self-conditioning max-rel {serr:.3e}")
            assert aerr <= 2e-2 and lerr <= 1e-3 and serr <= 2e-2, (t, aerr, lerr, serr)
        assert conv == bool(ref["converged"][0]), t
        if conv:
            steps = t + 1
            break
    say(f"[loop comb={combine}] converged after {steps} steps; entropy max err {max_ent:.2e}; candidates: "
        f"{tally['exact']}/{tally['draws']} equal the float64 inverse-CDF token, {tally['far']} more than one "
        f"token away, largest distance from the bracket {tally['max_dist']:.2e}")
    assert steps == want_steps

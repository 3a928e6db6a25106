"""dg_sampler_step_noalloc (the sampler on the library's static scratch, for callers that
cannot allocate) against dg_sampler_step on a caller-owned workspace, through the C ABI:
every output bit-equal, on two calls in a row, the second with a smaller input (fewer
rows and a smaller vocabulary, so it reads scratch entries the first call left behind
only where it wrote them itself). A call that needs more than the scratch holds fails
with DG_ERR_WORKSPACE and launches nothing."""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from workloads import logits as synth_logits, round_to_bf16
from tests.gpu_util import DEV, dev, host, say

pytestmark = pytest.mark.gpu

NAMES = ("entropy", "conf", "row_max", "row_sum", "argmax", "cand", "accept", "canvas", "prev_argmax",
         "stable_count", "num_accepted", "converged", "mean_entropy", "probs", "probs_scale")


def _pair(lt, reqs, V, bf16, budget, steps=2):
    """Run the same call sequence (init, then `steps` steps) with and without the scratch."""
    M = lt.shape[0]
    bufs = [dg.SamplerBuffers(M, len(reqs), DEV, vocab=V, probs_dtype=lt.dtype) for _ in range(2)]
    for b in bufs:
        dg.dg_sampler_step(None, reqs, V, b, budget, flags=dg.DG_INIT_CANVAS, num_rows=M)
    for t in range(steps):
        r = [(r0, n, seed, t) for (r0, n, seed, _) in reqs]
        dg.dg_sampler_step(lt, r, V, bufs[0], budget, stable_k=2, tau=0.01)
        dg.dg_sampler_step_noalloc(lt, r, V, bufs[1], budget, stable_k=2, tau=0.01)
        torch.cuda.synchronize()
        for n in NAMES:
            a, b = host(getattr(bufs[0], n)), host(getattr(bufs[1], n))
            assert np.array_equal(a, b, equal_nan=True), (M, V, t, n)
    say(f"[noalloc] M={M} V={V} bf16={bf16}: {steps} steps bit-equal to dg_sampler_step")


def test_noalloc_equals_workspace_call_twice_second_smaller():
    # first call: the step's shape (256 rows over a 262144-entry bf16 vocabulary, 0.6 MB of scratch)
    l1 = dev(synth_logits(2, 256, 262144, bf16=True), True)
    _pair(l1, [(0, 256, 99, 0)], 262144, True, 128.0)
    # second call, smaller: 70 rows in two requests over a ragged 5003-entry fp32 vocabulary
    rng = np.random.default_rng(5003)
    V = 5003
    l2 = (rng.standard_normal((70, V)) * rng.uniform(0.1, 8, (70, 1))).astype(np.float32)
    full = np.zeros((70, 5008), np.float32)
    full[:, :V] = l2
    _pair(dev(full)[:, :V], [(0, 40, 7, 0), (45, 25, 8, 0)], V, False, 20.0)


def test_noalloc_refuses_a_call_past_the_scratch():
    """2048 rows x 262144 (bf16) need 4.7 MB of workspace, more than the 4 MiB scratch."""
    M, V = 2048, 262144
    lt = torch.zeros(M, V, device=DEV, dtype=torch.bfloat16)
    b = dg.SamplerBuffers(M, 2, DEV)
    a = dg.make_sampler_args(lt, [(0, 1024, 1, 0), (1024, 1024, 2, 0)], V, b, 128.0)
    need = dg.sampler_workspace_size(a)
    assert need > dg.DG_NOALLOC_SCRATCH_BYTES
    before = host(b.canvas).copy()
    with pytest.raises(dg.DgError) as e:
        dg.dg_sampler_step_noalloc(lt, [(0, 1024, 1, 0), (1024, 1024, 2, 0)], V, b, 128.0)
    assert e.value.status == dg.DG_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.array_equal(host(b.canvas), before)

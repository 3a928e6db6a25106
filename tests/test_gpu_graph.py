"""A denoise step recorded once in a HIP graph and replayed as successive steps, through
the C ABI: the sampler reads each request's step from a device counter (step_counter),
which the selection advances, so the recorded launches need no per-step argument.

The loop the pages describe denoises a canvas step after step until it converges
([P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM", section
"샘플링 루프와 엔트로피 경계 디노이징"); a serving loop replays one recorded step.

Bar: every replay equals, bit for bit, the eager step with the same step index passed
from the host (attention output, selection, canvas, candidates, entropies, state,
self-conditioning output), with eager work and synchronisations between the replays,
two graphs alternating over two logits buffers; the counter holds t + 1 after step t.
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from workloads import Seq, BIDIR, normal, sigmas
from tests.gpu_util import DEV, dev, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 4, 2, 64
P, N, V, EMB = 192, 64, 512, 128
BUDGET, STABLE_K, TAU, LIMIT = 6.0, 3, 0.05, 40
STEPS = 10
SEED = 4242


def _inputs():
    q = dev(normal(8101, (N, HQ, D)))
    k = dev(normal(8102, (P + N, HKV, D)))
    v = dev(normal(8103, (P + N, HKV, D)))
    E = dev(normal(8104, (V, EMB), std=0.02))
    logits = [dev((normal(8110 + i, (N, V)) * sigmas(8120 + i, N)[:, None]).astype(np.float32)) for i in range(2)]
    return q, k, v, E, logits


class _Step:
    """The three calls of a step on their own buffers; the sampler optionally reads a
    device step counter."""

    def __init__(self, q, k, v, E, logits, counter=None, budget=BUDGET):
        n, hq, hkv = q.shape[0], q.shape[1], k.shape[1]
        prefix, vocab = k.shape[0] - n, E.shape[0]
        self.attn_out = torch.empty_like(q)
        self.bufs = dg.SamplerBuffers(n, 1, DEV, vocab=vocab, probs_dtype=logits[0].dtype)
        self.sc = torch.empty(n, E.shape[1], device=DEV, dtype=E.dtype)
        self.attn = dg.prepare_attn(q, k, v, self.attn_out, [Seq(0, n, 0, prefix, BIDIR)], -1, hq, hkv)
        kw = dict(stable_k=STABLE_K, tau=TAU, step_limit=LIMIT, combine=dg.DG_CONV_OR)
        if counter is not None:
            kw["step_counter"] = counter
        self.samp = [dg.prepare_sampler(l, [(0, n, SEED, 0)], vocab, self.bufs, budget, **kw) for l in logits]
        self.init = dg.prepare_sampler(None, [(0, n, SEED, 0)], vocab, self.bufs, budget, flags=dg.DG_INIT_CANVAS,
                                       num_rows=n, **({"step_counter": counter} if counter is not None else {}))
        self.selfcond = dg.prepare_selfcond(self.bufs.probs, E, self.sc, p_scale=self.bufs.probs_scale)

    def enqueue(self, t, host_step=None):
        if host_step is not None:
            self.samp[t % 2].args._keep[0].step = host_step
        self.attn()
        self.samp[t % 2]()
        self.selfcond()

    def snapshot(self):
        b = self.bufs
        return {name: t.detach().cpu().clone() for name, t in
                [("attn", self.attn_out), ("canvas", b.canvas), ("accept", b.accept), ("cand", b.cand),
                 ("entropy", b.entropy), ("argmax", b.argmax), ("prev_argmax", b.prev_argmax),
                 ("stable", b.stable_count), ("converged", b.converged), ("num_accepted", b.num_accepted),
                 ("mean_entropy", b.mean_entropy), ("selfcond", self.sc)]}


def _bits_equal(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _replay_against_eager(q, k, v, E, logits, steps, budget=BUDGET):
    """Eager host-stepped calls, then two recorded graphs replayed alternately with the
    step read from a device counter; every replay is compared with the eager step."""
    eager = _Step(q, k, v, E, logits, budget=budget)
    eager.init()
    want = []
    for t in range(steps):
        eager.enqueue(t, host_step=t)
        torch.cuda.synchronize()
        want.append(eager.snapshot())
    counter = torch.full((1,), 777, dtype=torch.int32, device=DEV)
    rec = _Step(q, k, v, E, logits, counter, budget=budget)
    rec.init()
    graphs = []
    side = torch.cuda.Stream()
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            rec.enqueue(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for t in range(steps):
        graphs[t % 2].replay()
        torch.cuda.synchronize()
        got = rec.snapshot()
        for name, w in want[t].items():
            assert _bits_equal(got[name], w), (t, name)
        assert int(counter.item()) == t + 1
    return want


def test_step_shapes_replay_against_eager():
    """The step's shapes and dtypes: canvas 256 on a 4096-token prefix (16 q / 8 kv heads
    x 256, bf16), bf16 logits [256 x 262144], bf16 embedding table [262144 x 2048]."""
    g = torch.Generator(device=DEV)
    g.manual_seed(8201)
    bf = torch.bfloat16
    q = torch.randn(256, 16, 256, device=DEV, generator=g).to(bf)
    k = torch.randn(4352, 8, 256, device=DEV, generator=g).to(bf)
    v = torch.randn(4352, 8, 256, device=DEV, generator=g).to(bf)
    E = (torch.randn(262144, 2048, device=DEV, generator=g) * 0.02).to(bf)
    sig = torch.exp(torch.empty(256, 1, device=DEV).uniform_(-2.3, 2.3, generator=g))
    logits = [(torch.randn(256, 262144, device=DEV, generator=g) * sig).to(bf) for _ in range(2)]
    want = _replay_against_eager(q, k, v, E, logits, steps=6, budget=128.0)
    say(f"[graph] step shapes: 6 replays equal the eager steps; accepted at the last step "
        f"{int(want[-1]['num_accepted'][0])}")


def test_recorded_step_replays_as_successive_steps():
    q, k, v, E, logits = _inputs()
    # eager: the host passes step t
    eager = _Step(q, k, v, E, logits)
    eager.init()
    want = []
    for t in range(STEPS):
        eager.enqueue(t, host_step=t)
        torch.cuda.synchronize()
        want.append(eager.snapshot())
    # recorded: one graph per logits buffer, the step read from the device counter
    counter = torch.full((1,), 12345, dtype=torch.int32, device=DEV)
    rec = _Step(q, k, v, E, logits, counter)
    rec.init()  # eager; sets the counter to 0
    torch.cuda.synchronize()
    assert int(counter.item()) == 0
    graphs = []
    side = torch.cuda.Stream()
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            rec.enqueue(i)
        graphs.append(g)
    torch.cuda.synchronize()
    assert int(counter.item()) == 0, "recording must not run the step"
    for t in range(STEPS):
        graphs[t % 2].replay()
        torch.cuda.synchronize()
        got = rec.snapshot()
        for name, w in want[t].items():
            assert _bits_equal(got[name], w), (t, name)
        assert int(counter.item()) == t + 1
        # eager work of the program's own between replays
        _ = (rec.attn_out.float().sum() + rec.sc.sum()).item()
    say(f"[graph] {STEPS} replays equal the eager steps; converged at the end: {bool(want[-1]['converged'][0])}")
    # a new block: the eager init resets the counter, and the replays start over at step 0
    rec.init()
    graphs[0].replay()
    torch.cuda.synchronize()
    assert int(counter.item()) == 1
    eager.init()
    eager.enqueue(0, host_step=0)
    torch.cuda.synchronize()
    w0 = eager.snapshot()
    got = rec.snapshot()
    for name in ("canvas", "accept", "cand", "stable", "selfcond"):
        assert _bits_equal(got[name], w0[name]), name


def test_step_counter_split_calls_advance_once():
    """DG_SKIP_SELECT reads the counter without advancing it; DG_SELECT_ONLY advances it."""
    _, _, _, _, logits = _inputs()
    counter = torch.zeros(1, dtype=torch.int32, device=DEV)
    bufs = dg.SamplerBuffers(N, 1, DEV)
    bref = dg.SamplerBuffers(N, 1, DEV)
    for b in (bufs, bref):
        dg.dg_sampler_step(None, [(0, N, SEED, 0)], V, b, BUDGET, flags=dg.DG_INIT_CANVAS, num_rows=N,
                           step_counter=counter if b is bufs else None)
    for t in range(3):
        dg.dg_sampler_step(logits[t % 2], [(0, N, SEED, 999)], V, bufs, BUDGET, flags=dg.DG_SKIP_SELECT,
                           step_counter=counter)
        torch.cuda.synchronize()
        assert int(counter.item()) == t
        dg.dg_sampler_step(logits[t % 2], [(0, N, SEED, 999)], V, bufs, BUDGET, flags=dg.DG_SELECT_ONLY,
                           step_counter=counter)
        dg.dg_sampler_step(logits[t % 2], [(0, N, SEED, t)], V, bref, BUDGET)
        torch.cuda.synchronize()
        assert int(counter.item()) == t + 1
        for name in ("canvas", "cand", "accept", "stable_count"):
            assert torch.equal(getattr(bufs, name), getattr(bref, name)), (t, name)

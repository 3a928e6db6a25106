"""GPU parity of dg_selfcond_embed against the CPU oracle, through the C ABI.

Bar: max-relative error per output row (max_j |g - o| / max_j |o|) <= 2e-2, for
bf16 with fp32 accumulation and for fp32; one-hot probability rows return the
embedding row bit-exactly.
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from oracle.selfcond import selfcond_embed, softmax_rows
from oracle.sampler import row_stats
from workloads import logits as synth_logits, embed_table, round_to_bf16
from tests.gpu_util import DEV, dev, host, max_rel_rows, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _stats_dev(l_np):
    st = row_stats(l_np)
    return dev(st["max"].astype(np.float32)), dev(st["sum"].astype(np.float32))


def test_fp32_256x4096x256_probs_and_fused():
    E = embed_table(1, 4096, 256, bf16=False)
    l = synth_logits(1, 256, 4096, bf16=False)
    want = selfcond_embed(E, logits=l)
    Et, lt = dev(E), dev(l)
    out = torch.empty(256, 256, device=DEV)
    p = dev(softmax_rows(l).astype(np.float32))
    dg.dg_selfcond_embed(p, Et, out)
    torch.cuda.synchronize()
    e1 = max_rel_rows(host(out), want)
    rm, rs = _stats_dev(l)
    out2 = torch.empty(256, 256, device=DEV)
    dg.dg_selfcond_embed(lt, Et, out2, row_max=rm, row_sum=rs)
    torch.cuda.synchronize()
    e2 = max_rel_rows(host(out2), want)
    say(f"[selfcond] fp32 256x4096x256: probs max-rel {e1:.3e}, fused max-rel {e2:.3e}")
    assert e1 <= TOL and e2 <= TOL
    assert e1 < 1e-4 and e2 < 1e-4  # fp32 path is far inside the bar


def test_bf16_256x262144x2048_sampled_rows():
    V, d, M = 262144, 2048, 256
    E = embed_table(2, V, d, bf16=True)
    l = synth_logits(2, M, V, bf16=True)
    Et, lt = dev(E, True), dev(l, True)
    rm, rs = _stats_dev(l)
    out = torch.empty(M, d, device=DEV, dtype=torch.bfloat16)
    dg.dg_selfcond_embed(lt, Et, out, row_max=rm, row_sum=rs)
    torch.cuda.synchronize()
    rows = [0, 1, 17, 63, 128, 200, 254, 255]
    want = selfcond_embed(E, logits=l[rows])
    err = max_rel_rows(host(out)[rows], want)
    say(f"[selfcond] bf16 256x262144x2048 fused, rows {rows}: max-rel {err:.3e}")
    assert err <= TOL
    # materialised-probability mode on the same rows
    p = dev(softmax_rows(l).astype(np.float32), True)
    out2 = torch.empty(M, d, device=DEV, dtype=torch.bfloat16)
    dg.dg_selfcond_embed(p, Et, out2)
    torch.cuda.synchronize()
    want2 = selfcond_embed(E, probs=round_to_bf16(softmax_rows(l[rows]).astype(np.float32)))
    err2 = max_rel_rows(host(out2)[rows], want2)
    say(f"[selfcond] bf16 256x262144x2048 probs: max-rel {err2:.3e}")
    assert err2 <= TOL


@pytest.mark.parametrize("bf16,V,d", [(False, 3000, 256), (True, 3000, 256), (True, 3008, 256), (True, 3008, 1024)])
def test_one_hot_bit_exact(bf16, V, d):
    """P-C1 on the GPU: one-hot rows return exactly the embedding row (V = 3008 takes
    the LDS-DMA kernel - its 128 x 512 tile when d is a multiple of 512 - and V = 3000
    the register-staged one)."""
    M = 70
    E = embed_table(9, V, d, bf16=bf16)
    rng = np.random.default_rng(1)
    hot = rng.integers(0, V, M)
    p = np.zeros((M, V), np.float32)
    p[np.arange(M), hot] = 1.0
    out = torch.empty(M, d, device=DEV, dtype=torch.bfloat16 if bf16 else torch.float32)
    dg.dg_selfcond_embed(dev(p, bf16), dev(E, bf16), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), E[hot])


@pytest.mark.parametrize("bf16,M,V,d", [(True, 130, 1000, 256), (False, 5, 77, 128), (True, 1, 262144, 128),
                                        (True, 300, 4104, 384), (True, 300, 4096, 512), (True, 129, 8192, 1536),
                                        (False, 100, 5000, 384)])
def test_ragged_shapes(bf16, M, V, d):
    """M not a multiple of the tile, V ending mid-step and mid-vector, small d."""
    rng = np.random.default_rng(M + V)
    l = (rng.standard_normal((M, V)) * rng.uniform(0.1, 10, (M, 1))).astype(np.float32)
    E = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
    if bf16:
        l, E = round_to_bf16(l), round_to_bf16(E)
    # pad the vocabulary stride to a multiple of 8 as the ABI requires
    ldp = (V + 7) // 8 * 8
    lp = np.zeros((M, ldp), np.float32)
    lp[:, :V] = l
    lt = dev(lp, bf16)[:, :V]
    rm, rs = _stats_dev(l)
    out = torch.empty(M, d, device=DEV, dtype=torch.bfloat16 if bf16 else torch.float32)
    dg.dg_selfcond_embed(lt, dev(E, bf16), out, row_max=rm, row_sum=rs)
    torch.cuda.synchronize()
    err = max_rel_rows(host(out), selfcond_embed(E, logits=l))
    say(f"[selfcond] ragged M={M} V={V} d={d} bf16={bf16}: max-rel {err:.3e}")
    assert err <= TOL


def test_repeat_is_bit_identical():
    V, d, M = 65536, 512, 256
    E = dev(embed_table(3, V, d, bf16=True), True)
    l = synth_logits(3, M, V, bf16=True)
    rm, rs = _stats_dev(l)
    lt = dev(l, True)
    outs = []
    for _ in range(2):
        o = torch.empty(M, d, device=DEV, dtype=torch.bfloat16)
        dg.dg_selfcond_embed(lt, E, o, row_max=rm, row_sum=rs)
        torch.cuda.synchronize()
        outs.append(host(o))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("bf16,M,V,d", [(True, 256, 262144, 2048), (True, 1024, 262144, 2048), (False, 256, 4096, 256),
                                        (True, 300, 40000, 384), (True, 64, 8200, 128)])
def test_block_scaled_from_sampler(bf16, M, V, d):
    """The sampler's block-scaled probabilities feed self-conditioning directly; the
    result matches the oracle's softmax-weighted average."""
    rng = np.random.default_rng(M + V + d)
    l = (rng.standard_normal((M, V)) * rng.uniform(0.1, 10, (M, 1))).astype(np.float32)
    E = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
    if bf16:
        l, E = round_to_bf16(l), round_to_bf16(E)
    ld = (V + 7) // 8 * 8
    full = np.zeros((M, ld), np.float32)
    full[:, :V] = l
    lt = dev(full, bf16)[:, :V]
    b = dg.SamplerBuffers(M, 1, DEV, vocab=V, probs_dtype=lt.dtype)
    dg.dg_sampler_step(lt, [(0, min(M, 1024), 5, 0)], V, b, 64.0)
    out = torch.empty(M, d, device=DEV, dtype=lt.dtype)
    dg.dg_selfcond_embed(b.probs, dev(E, bf16), out, p_scale=b.probs_scale)
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, M // 2, M - 1] + list(range(0, M, max(1, M // 8)))))
    err = max_rel_rows(host(out)[rows], selfcond_embed(E, logits=l[rows]))
    say(f"[selfcond] block-scaled M={M} V={V} d={d} bf16={bf16}: max-rel {err:.3e}")
    assert err <= TOL

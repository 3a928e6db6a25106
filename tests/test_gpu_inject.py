"""GPU parity of dg_selfcond_inject against the CPU oracle, through the C ABI.

Bar: max-relative error per output row <= 2e-2 for bf16 (fp32 accumulation; the
gate/up product and the GeGLU output are stored in bf16, and the oracle rounds the same
two intermediates), and far inside it for fp32. Canvas tokens outside [0, vocab) are
clamped into it (the header's rule), so the expected values use the clamped tokens.
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from oracle.inject import selfcond_inject
from workloads import normal, embed_table, round_to_bf16
from tests.gpu_util import DEV, dev, host, max_rel_rows, say

pytestmark = pytest.mark.gpu


def _case(M, d, hidden, V, bf16, seed, E=None):
    rng = np.random.default_rng(seed)
    tokens = rng.integers(0, V, M).astype(np.int32)
    tokens[0], tokens[-1] = -5, V + 3  # clamped to 0 and V - 1
    if E is None:
        E = normal(seed + 1, (V, d), std=0.02, bf16=bf16)
    s = normal(seed + 2, (M, d), bf16=bf16)
    wgu = normal(seed + 3, (d, 2 * hidden), std=1.0 / np.sqrt(d), bf16=bf16)
    wd = normal(seed + 4, (hidden, d), std=1.0 / np.sqrt(hidden), bf16=bf16)
    out = torch.full((M, d), float("nan"), device=DEV, dtype=torch.bfloat16 if bf16 else torch.float32)
    dg.dg_selfcond_inject(torch.from_numpy(tokens).to(DEV), dev(E, bf16), dev(s, bf16), dev(wgu, bf16), dev(wd, bf16),
                          out)
    torch.cuda.synchronize()
    want = selfcond_inject(np.clip(tokens, 0, V - 1), E, s, wgu, wd,
                           round_to=(lambda x: round_to_bf16(x.astype(np.float32))) if bf16 else None)
    return max_rel_rows(host(out), want)


@pytest.mark.parametrize("M,d,hidden,V,bf16", [(77, 256, 384, 1000, False), (300, 512, 256, 5000, True),
                                               (1, 128, 128, 7, True), (256, 1024, 640, 4096, False),
                                               # both products split over K: the reduce's GeGLU and
                                               # gather epilogues, on a ragged row count
                                               (300, 1024, 1024, 5000, True)])
def test_shapes(M, d, hidden, V, bf16):
    err = _case(M, d, hidden, V, bf16, seed=M + d + hidden)
    say(f"[inject] M={M} d={d} hidden={hidden} V={V} bf16={bf16}: max-rel {err:.3e}")
    assert err <= 2e-2
    if not bf16:
        assert err < 1e-4


def test_step_shapes_canvas256_d2048_vocab262144():
    """The step's shapes: 256 canvas rows, d = 2048, hidden 2048, the 262144-row table."""
    E = embed_table(2, 262144, 2048, bf16=True)
    err = _case(256, 2048, 2048, 262144, True, seed=5150, E=E)
    say(f"[inject] canvas 256, d 2048, hidden 2048, vocab 262144: max-rel {err:.3e}")
    assert err <= 2e-2

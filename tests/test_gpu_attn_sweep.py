"""GPU parity of dg_attn_mixed on a seeded sweep of small mixed batches, through the
C ABI: every request's mode, prefix and length, the window, the head grouping, the
head dimension, forced key chunks and the paged layout are drawn per case, and every
output row is compared with the oracle (max-relative error per row <= 2e-2 for bf16,
1e-4 for fp32; lse within 1e-3). Also the 2048-token causal prefill on an empty cache,
whose key chunks are sized from its longest q tile, on rows across its q tiles and
chunk boundaries.
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from oracle.attn import attn_mixed
from oracle.kvcache import attn_mixed_paged
from workloads import pack_seqs, Seq, CAUSAL, BIDIR, normal
from tests.gpu_util import DEV, dev, host, max_rel_rows, say

pytestmark = pytest.mark.gpu


def _paged(seqs, k, v, B, rng):
    nbs = [-(-(s.prefix_len + s.num_q) // B) for s in seqs]
    order = rng.permutation(sum(nbs) + 1)
    kp = np.zeros(((sum(nbs) + 1) * B,) + k.shape[1:], np.float32)
    vp = np.zeros_like(kp)
    table, pseqs, used = [], [], 0
    for s, nb in zip(seqs, nbs):
        n = s.prefix_len + s.num_q
        start = len(table)
        for b in range(nb):
            blk = int(order[used])
            used += 1
            table.append(blk)
            lo, hi = b * B, min(n, (b + 1) * B)
            kp[blk * B:blk * B + hi - lo] = k[s.kv_start + lo:s.kv_start + hi]
            vp[blk * B:blk * B + hi - lo] = v[s.kv_start + lo:s.kv_start + hi]
        pseqs.append(Seq(s.q_start, s.num_q, start, s.prefix_len, s.mode))
    return kp, vp, np.array(table, np.int32), pseqs


@pytest.mark.parametrize("case", range(12))
def test_random_mixed_batches(case):
    rng = np.random.default_rng(7100 + case)
    D = int(rng.choice([64, 128, 256]))
    bf16 = bool(D == 256 or rng.random() < 0.6)
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * G
    window = int(rng.choice([-1, -1, 0, 17, 100]))
    spec = [(int(rng.integers(0, 700)), int(rng.integers(1, 300)), int(rng.integers(0, 2)))
            for _ in range(int(rng.integers(1, 4)))]
    chunk = int(rng.choice([0, 0, 64, 192]))
    paged = bool(rng.random() < 0.5)
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q = normal(7200 + case, (T, hq, D), bf16=bf16)
    k = normal(7300 + case, (S, hkv, D), bf16=bf16)
    v = normal(7400 + case, (S, hkv, D), bf16=bf16)
    say(f"[sweep {case}] D={D} bf16={bf16} hq={hq} hkv={hkv} W={window} spec={spec} chunk={chunk} paged={paged}")
    out = torch.full((T, hq, D), np.nan, device=DEV, dtype=torch.bfloat16 if bf16 else torch.float32)
    lse = torch.full((T, hq), np.nan, device=DEV, dtype=torch.float32)
    if paged:
        B = int(rng.choice([64, 128]))
        kp, vp, table, pseqs = _paged(seqs, k, v, B, rng)
        dg.dg_attn_mixed(dev(q, bf16), dev(kp, bf16), dev(vp, bf16), out, pseqs, window, hq, hkv, lse=lse,
                         kv_chunk=chunk, block_table=torch.from_numpy(table).to(DEV), block_size=B)
        want, wlse = attn_mixed_paged(pseqs, window, q, kp, vp, table, B, hq, hkv)
    else:
        dg.dg_attn_mixed(dev(q, bf16), dev(k, bf16), dev(v, bf16), out, seqs, window, hq, hkv, lse=lse,
                         kv_chunk=chunk)
        want, wlse = attn_mixed(seqs, window, q, k, v, hq, hkv)
    torch.cuda.synchronize()
    err = max_rel_rows(host(out), want)
    lerr = float(np.abs(host(lse) - wlse).max())
    say(f"  max-rel {err:.3e}  lse abs {lerr:.3e}")
    assert err <= (2e-2 if bf16 else 1e-4) and lerr <= 1e-3


def test_causal_prefill_2048_on_empty_cache():
    N, hq, hkv, D = 2048, 16, 8, 256
    seqs = [Seq(0, N, 0, 0, CAUSAL)]
    q = normal(7501, (N, hq, D), bf16=True)
    k = normal(7502, (N, hkv, D), bf16=True)
    v = normal(7503, (N, hkv, D), bf16=True)
    out = torch.empty(N, hq, D, device=DEV, dtype=torch.bfloat16)
    dg.dg_attn_mixed(dev(q, True), dev(k, True), dev(v, True), out, seqs, -1, hq, hkv)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 127, 128, 511, 1023, 1024, 1087, 1088, 1535, 2046, 2047]
    want, _ = attn_mixed(seqs, -1, q, k, v, hq, hkv, rows=rows)
    err = max_rel_rows(host(out)[rows], want[rows])
    say(f"[prefill 2048 causal] rows {rows}: max-rel {err:.3e}")
    assert err <= 2e-2

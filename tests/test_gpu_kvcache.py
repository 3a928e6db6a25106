"""GPU parity of the paged K/V path through the C ABI: dg_attn_mixed with block tables
(block_size > 0) and dg_kv_write.

Bar:
- paged attention equals contiguous attention bit for bit on the same key rows (the
  kernels and the plan are the same; only the row addresses differ), for every kernel
  family (fp32 and bf16 general kernels, the bf16 head_dim-256 128-row and 64-row
  kernels) - so the contiguous parity tests against the oracle carry over;
- paged attention against the paged oracle: max-relative error per row <= 2e-2, lse
  within 1e-3;
- dg_kv_write: the pools equal the oracle's bit for bit.
Pool rows that no request owns, and the tail of each request's last block, hold NaN:
a kernel that read them would turn its outputs into NaN.
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from oracle.kvcache import attn_mixed_paged, kv_write as ref_kv_write
from workloads import pack_seqs, Seq, CAUSAL, BIDIR, normal
from tests.gpu_util import DEV, dev, host, max_rel_rows, say

pytestmark = pytest.mark.gpu


def _paged(seqs, k, v, B, seed, spare=3):
    """Scatter each request's contiguous rows into pools of B-row blocks in a random
    order; returns (k_pool, v_pool, table, paged seqs) as NumPy arrays."""
    nbs = [-(-(s.prefix_len + s.num_q) // B) for s in seqs]
    total = sum(nbs) + spare
    order = np.random.default_rng(seed).permutation(total)
    kp = np.full((total * B,) + k.shape[1:], np.nan, dtype=k.dtype)
    vp = np.full((total * B,) + v.shape[1:], np.nan, dtype=v.dtype)
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


def _run(q, k, v, seqs, window, hq, hkv, bf16, kv_chunk=0, table=None, B=0):
    qt, kt, vt = dev(q, bf16), dev(k, bf16), dev(v, bf16)
    out = torch.full(qt.shape, np.nan, device=DEV, dtype=qt.dtype)
    lse = torch.full(qt.shape[:2], np.nan, device=DEV, dtype=torch.float32)
    tt = None if table is None else torch.from_numpy(table).to(DEV)
    dg.dg_attn_mixed(qt, kt, vt, out, seqs, window, hq, hkv, lse=lse, kv_chunk=kv_chunk, block_table=tt, block_size=B)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # label, spec [(prefix, num_q, mode)], window, hq, hkv, D, bf16, block size, kv_chunk
    ("fp32 d64 canvas 256 prefix 256 W=32 bidir", [(256, 256, BIDIR)], 32, 4, 4, 64, False, 64, 0),
    ("fp32 d64 canvas 256 prefix 256 W=32 causal", [(256, 256, CAUSAL)], 32, 4, 4, 64, False, 64, 0),
    ("bf16 d128 ragged causal G=4", [(300, 77, CAUSAL), (0, 45, BIDIR)], -1, 8, 2, 128, True, 128, 0),
    ("bf16 d256 canvas 256 prefix 4096 (128-row kernel)", [(4096, 256, BIDIR)], -1, 16, 8, 256, True, 256, 0),
    ("bf16 d256 canvas 256 prefix 16384 (64-row kernel)", [(16384, 256, BIDIR)], -1, 16, 8, 256, True, 64, 0),
    ("bf16 d256 mixed W=512 forced chunks", [(0, 300, CAUSAL), (1000, 256, BIDIR), (5000, 64, CAUSAL)], 512, 16, 8,
     256, True, 128, 256),
    ("bf16 d256 mixed global, ragged prefixes", [(1500, 200, BIDIR), (777, 256, CAUSAL), (9000, 33, BIDIR)], -1, 16, 8,
     256, True, 64, 0),
    ("bf16 d256 short chunks, ring edges", [(0, 1, BIDIR), (20, 13, BIDIR), (60, 5, BIDIR), (100, 29, CAUSAL),
                                            (150, 50, BIDIR)], -1, 16, 8, 256, True, 64, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_equals_contiguous_bitwise(case):
    label, spec, window, hq, hkv, D, bf16, B, chunk = case
    say(f"[paged] {label}: B={B} chunk={chunk}")
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q = normal(311, (T, hq, D), bf16=bf16)
    k = normal(312, (S, hkv, D), bf16=bf16)
    v = normal(313, (S, hkv, D), bf16=bf16)
    # the 64-row kernel case lowers the planner's threshold (test hook) so that its
    # request, which the default sends to the 128-row kernel, runs there
    with dg.wide_min_sub(16 if "64-row kernel" in label else 0):
        out_c, lse_c = _run(q, k, v, seqs, window, hq, hkv, bf16, chunk)
        kp, vp, table, pseqs = _paged(seqs, k, v, B, seed=314)
        out_p, lse_p = _run(q, kp, vp, pseqs, window, hq, hkv, bf16, chunk, table, B)
    assert not torch.isnan(out_c).any()
    assert torch.equal(out_p.view(torch.int16) if bf16 else out_p.view(torch.int32),
                       out_c.view(torch.int16) if bf16 else out_c.view(torch.int32)), label
    assert torch.equal(lse_p.view(torch.int32), lse_c.view(torch.int32)), label


@pytest.mark.parametrize("bf16,D,B", [(True, 256, 64), (False, 64, 128)])
def test_paged_against_paged_oracle(bf16, D, B):
    spec = [(130, 64, BIDIR), (0, 70, CAUSAL), (200, 19, BIDIR)]
    hq, hkv = (16, 8) if D == 256 else (4, 2)
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q = normal(321, (T, hq, D), bf16=bf16)
    k = normal(322, (S, hkv, D), bf16=bf16)
    v = normal(323, (S, hkv, D), bf16=bf16)
    kp, vp, table, pseqs = _paged(seqs, k, v, B, seed=324)
    for window in (-1, 40):
        say(f"[paged-oracle] bf16={bf16} D={D} B={B} W={window}")
        out, lse = _run(q, kp, vp, pseqs, window, hq, hkv, bf16, 0, table, B)
        want, wlse = attn_mixed_paged(pseqs, window, q, kp, vp, table, B, hq, hkv)
        err = max_rel_rows(host(out), want)
        lerr = float(np.abs(host(lse) - wlse).max())
        say(f"  max-rel {err:.3e}  lse abs {lerr:.3e}")
        assert err <= 2e-2 and lerr <= 1e-3
        if not bf16:
            assert err < 1e-4


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("bf16,hkv,D,B", [(True, 8, 256, 64), (False, 2, 64, 16), (True, 1, 8, 1)])
def test_kv_write_matches_oracle(bf16, hkv, D, B):
    rng = np.random.default_rng(331)
    nblocks = 64 if B >= 16 else 600
    pool_rows = nblocks * B
    kp = normal(332, (pool_rows, hkv, D), bf16=bf16)
    vp = normal(333, (pool_rows, hkv, D), bf16=bf16)
    new_k = normal(334, (500, hkv, D), bf16=bf16)
    new_v = normal(335, (500, hkv, D), bf16=bf16)
    perm = rng.permutation(nblocks).astype(np.int32)
    # request 0: positions 100..399; request 1: positions 0..63; request 2: a ragged
    # draft at 37..135 whose table holds entries outside the pool (skipped rows)
    seqs = [(0, 300, 0, 100), (300, 64, 0 + (400 + B - 1) // B, 0), (364, 99, 0, 37)]
    t1 = (400 + B - 1) // B
    need = max(t1 + (64 + B - 1) // B, (136 + B - 1) // B)
    table = np.concatenate([perm[:t1], perm[t1:need]]).astype(np.int32)
    table3 = table.copy()
    table3[(60 // B) % len(table3)] = -1
    table3[(120 // B) % len(table3)] = nblocks + 5
    # request 2 reads its own table copy, appended after the first
    full = np.concatenate([table, table3]).astype(np.int32)
    seqs[2] = (364, 99, len(table), 37)
    say(f"[kv_write] bf16={bf16} Hkv={hkv} D={D} B={B}")
    want_k, want_v = ref_kv_write(kp, vp, new_k, new_v, seqs[:2], full, B)
    # request 2 writes rows that requests 0 and 1 may also own: it runs in its own call
    want_k, want_v = ref_kv_write(want_k, want_v, new_k, new_v, seqs[2:], full, B)
    kpt, vpt = dev(kp, bf16), dev(vp, bf16)
    tt = torch.from_numpy(full).to(DEV)
    dg.dg_kv_write(dev(new_k, bf16), dev(new_v, bf16), kpt, vpt, seqs[:2], tt, B)
    dg.dg_kv_write(dev(new_k, bf16), dev(new_v, bf16), kpt, vpt, seqs[2:], tt, B)
    torch.cuda.synchronize()
    assert torch.equal(_bits(kpt), _bits(dev(want_k, bf16)))
    assert torch.equal(_bits(vpt), _bits(dev(want_v, bf16)))


def test_prefill_commit_and_draft_through_kv_write_then_paged_attention():
    """A request's life on the paged cache: a prefill written through the table, a
    first canvas draft, a second draft over the same positions; paged attention of the
    canvas then equals contiguous attention on [prefill || second draft], bit for bit."""
    B, hq, hkv, D, P, N = 64, 16, 8, 256, 1000, 256
    nb = -(-(P + N) // B) + 2
    table = np.random.default_rng(341).permutation(nb)[:-(-(P + N) // B)].astype(np.int32)
    pref_k, pref_v = normal(342, (P, hkv, D), bf16=True), normal(343, (P, hkv, D), bf16=True)
    d1 = normal(344, (N, hkv, D), bf16=True)
    d2k, d2v = normal(345, (N, hkv, D), bf16=True), normal(346, (N, hkv, D), bf16=True)
    q = normal(347, (N, hq, D), bf16=True)
    kpt = torch.full((nb * B, hkv, D), float("nan"), device=DEV, dtype=torch.bfloat16)
    vpt = torch.full_like(kpt, float("nan"))
    tt = torch.from_numpy(table).to(DEV)
    dg.dg_kv_write(dev(pref_k, True), dev(pref_v, True), kpt, vpt, [(0, P, 0, 0)], tt, B)
    dg.dg_kv_write(dev(d1, True), dev(d1, True), kpt, vpt, [(0, N, 0, P)], tt, B)
    dg.dg_kv_write(dev(d2k, True), dev(d2v, True), kpt, vpt, [(0, N, 0, P)], tt, B)
    qt = dev(q, True)
    out_p = torch.empty_like(qt)
    dg.dg_attn_mixed(qt, kpt, vpt, out_p, [Seq(0, N, 0, P, BIDIR)], -1, hq, hkv, block_table=tt, block_size=B)
    kc, vc = dev(np.concatenate([pref_k, d2k]), True), dev(np.concatenate([pref_v, d2v]), True)
    out_c = torch.empty_like(qt)
    dg.dg_attn_mixed(qt, kc, vc, out_c, [Seq(0, N, 0, P, BIDIR)], -1, hq, hkv)
    torch.cuda.synchronize()
    assert not torch.isnan(out_c).any()
    assert torch.equal(out_p.view(torch.int16), out_c.view(torch.int16))

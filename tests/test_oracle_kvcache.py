"""Pins for the paged K/V oracle: each test checks it against something other than
itself - the contiguous attention oracle (itself pinned to torch SDPA) on a pool that
holds the contiguous layout, invariance under a permutation of the pool's blocks,
brute force over pool rows on tiny inputs, and copy round trips.

Pages: [P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM",
sections "샘플링 루프와 엔트로피 경계 디노이징" and "ModelState 인터페이스";
[P3] "DiffusionGemma u vLLM: ...", section "Integracija u vLLM infrastrukturu".
"""
import numpy as np
import pytest

from oracle.attn import attn_mixed, key_range, CAUSAL, BIDIR
from oracle.kvcache import attn_mixed_paged, kv_write, gather_rows
from workloads import Seq, pack_seqs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _contiguous_pool(seqs, k, v, B):
    """Lay each request's rows out block-aligned, in order: returns pools, table, paged seqs."""
    kp, vp, table, pseqs = [], [], [], []
    blk = 0
    for s in seqs:
        n = s.prefix_len + s.num_q
        nb = -(-n // B)
        rows_k = np.zeros((nb * B,) + k.shape[1:])
        rows_v = np.zeros((nb * B,) + v.shape[1:])
        rows_k[:n] = k[s.kv_start:s.kv_start + n]
        rows_v[:n] = v[s.kv_start:s.kv_start + n]
        kp.append(rows_k)
        vp.append(rows_v)
        pseqs.append(Seq(s.q_start, s.num_q, len(table), s.prefix_len, s.mode))
        table.extend(range(blk, blk + nb))
        blk += nb
    return np.concatenate(kp), np.concatenate(vp), np.array(table, np.int32), pseqs


SPECS = [[(0, 7, CAUSAL)], [(5, 9, BIDIR)], [(13, 3, CAUSAL), (4, 6, BIDIR), (0, 5, BIDIR)]]


@pytest.mark.parametrize("spec", SPECS)
@pytest.mark.parametrize("B", [1, 4, 8])
@pytest.mark.parametrize("window", [-1, 2])
def test_in_order_pool_equals_contiguous(spec, B, window):
    """A pool holding each request's rows in order, block-aligned, gives exactly the
    contiguous result."""
    seqs = pack_seqs(spec)
    hq, hkv, D = 4, 2, 8
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q, k, v = _rand((T, hq, D), 1), _rand((S, hkv, D), 2), _rand((S, hkv, D), 3)
    kp, vp, table, pseqs = _contiguous_pool(seqs, k, v, B)
    want = attn_mixed(seqs, window, q, k, v, hq, hkv)
    got = attn_mixed_paged(pseqs, window, q, kp, vp, table, B, hq, hkv)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])


@pytest.mark.parametrize("B", [2, 4])
def test_block_permutation_invariance(B):
    """Moving the pool's blocks and the table entries with them changes nothing."""
    seqs = pack_seqs([(9, 5, BIDIR), (6, 4, CAUSAL)])
    hq, hkv, D = 2, 1, 4
    q = _rand((9, hq, D), 4)
    k, v = _rand((24, hkv, D), 5), _rand((24, hkv, D), 6)
    kp, vp, table, pseqs = _contiguous_pool(seqs, k, v, B)
    nb = kp.shape[0] // B
    perm = np.random.default_rng(7).permutation(nb)  # block b moves to perm[b]
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    for b in range(nb):
        kq[perm[b] * B:(perm[b] + 1) * B] = kp[b * B:(b + 1) * B]
        vq[perm[b] * B:(perm[b] + 1) * B] = vp[b * B:(b + 1) * B]
    want = attn_mixed_paged(pseqs, -1, q, kp, vp, table, B, hq, hkv)
    got = attn_mixed_paged(pseqs, -1, q, kq, vq, perm[table].astype(np.int32), B, hq, hkv)
    np.testing.assert_array_equal(got[0], want[0])


def test_brute_force_over_pool_rows():
    """Per (query, head): softmax attention summed key by key, each key row located
    in the pool by the block-table rule, on a scrambled tiny pool."""
    B, hq, hkv, D = 4, 2, 2, 3
    rng = np.random.default_rng(8)
    kp, vp = rng.standard_normal((40, hkv, D)), rng.standard_normal((40, hkv, D))
    table = np.array([7, 2, 9, 0, 5, 3, 1], np.int32)
    seqs = [Seq(0, 4, 0, 6, BIDIR), Seq(4, 3, 3, 10, CAUSAL)]
    q = rng.standard_normal((7, hq, D))
    got, _ = attn_mixed_paged(seqs, 3, q, kp, vp, table, B, hq, hkv)
    for s in seqs:
        for i in range(s.num_q):
            lo, hi = key_range(s.mode, s.prefix_len, s.num_q, 3, i)
            for h in range(hq):
                num, den = np.zeros(D), 0.0
                for j in range(lo, hi + 1):
                    r = table[s.kv_start + j // B] * B + j % B
                    w = np.exp(np.dot(q[s.q_start + i, h], kp[r, h]) / np.sqrt(D))
                    num += w * vp[r, h]
                    den += w
                np.testing.assert_allclose(got[s.q_start + i, h], num / den, rtol=1e-12, atol=1e-12)


def test_kv_write_round_trip_and_untouched_rows():
    """Rows written at positions pos.. read back in order; every other row keeps its value."""
    B = 4
    rng = np.random.default_rng(9)
    kp, vp = rng.standard_normal((32, 2, 8)), rng.standard_normal((32, 2, 8))
    new_k, new_v = rng.standard_normal((10, 2, 8)), rng.standard_normal((10, 2, 8))
    table = np.array([6, 1, 4, 3, 7, 0], np.int32)
    seqs = [(0, 6, 0, 3), (6, 4, 3, 5)]  # request A: positions 3..8; request B: positions 5..8
    k2, v2 = kv_write(kp, vp, new_k, new_v, seqs, table, B)
    got_a = gather_rows(k2, table, 0, 9, B)[3:9]
    got_b = gather_rows(v2, table, 3, 9, B)[5:9]
    np.testing.assert_array_equal(got_a, new_k[0:6])
    np.testing.assert_array_equal(got_b, new_v[6:10])
    written = set()
    for src, num, ts, pos in seqs:
        for i in range(num):
            p = pos + i
            written.add(int(table[ts + p // B]) * B + p % B)
    for r in range(32):
        if r not in written:
            np.testing.assert_array_equal(k2[r], kp[r])
            np.testing.assert_array_equal(v2[r], vp[r])
    assert len(written) == 10


def test_kv_write_skips_entries_outside_the_pool():
    B = 2
    kp = np.zeros((8, 1, 8))
    new = np.arange(4 * 8, dtype=np.float64).reshape(4, 1, 8) + 1
    table = np.array([1, -1, 9, 2], np.int32)  # blocks 1 and 2 exist (4 blocks), -1 and 9 do not
    k2, _ = kv_write(kp, kp, new, new, [(0, 4, 0, 1)], table, B)
    # positions 1..4: p=1 -> block 1 row 3; p=2,3 -> entry -1 (skipped); p=4 -> entry 9 (skipped)
    np.testing.assert_array_equal(k2[3], new[0])
    assert np.count_nonzero(k2) == 8  # one row of 8 values written


def test_prefill_then_draft_rewrite_matches_contiguous():
    """A prefill written through the table, then a canvas written twice (the later draft
    wins), gives the attention of the contiguous layout holding the prefill and the
    second draft."""
    B, hq, hkv, D, P, N = 4, 2, 1, 4, 10, 5
    rng = np.random.default_rng(10)
    prefix_k, prefix_v = rng.standard_normal((P, hkv, D)), rng.standard_normal((P, hkv, D))
    d1 = rng.standard_normal((N, hkv, D))
    d2k, d2v = rng.standard_normal((N, hkv, D)), rng.standard_normal((N, hkv, D))
    table = np.array([3, 0, 2, 5], np.int32)
    kp, vp = np.zeros((24, hkv, D)), np.zeros((24, hkv, D))
    kp, vp = kv_write(kp, vp, prefix_k, prefix_v, [(0, P, 0, 0)], table, B)
    kp, vp = kv_write(kp, vp, d1, d1, [(0, N, 0, P)], table, B)
    kp, vp = kv_write(kp, vp, d2k, d2v, [(0, N, 0, P)], table, B)
    q = rng.standard_normal((N, hq, D))
    got = attn_mixed_paged([Seq(0, N, 0, P, BIDIR)], -1, q, kp, vp, table, B, hq, hkv)
    want = attn_mixed([Seq(0, N, 0, P, BIDIR)], -1, q, np.concatenate([prefix_k, d2k]),
                      np.concatenate([prefix_v, d2v]), hq, hkv)
    np.testing.assert_array_equal(got[0], want[0])

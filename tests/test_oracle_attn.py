"""Pins for the attention oracle: each test checks it against something other than
itself - a library routine (torch SDPA in float64 on the CPU), closed-form key
counts from the window rule, degenerate windows and structural invariants.

Pages: [P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM",
sections "듀얼 모드 운영", "동적 퍼-시퀀스 인과적 어텐션", "대칭 슬라이딩 윈도우 어텐션".
"""
import itertools

import numpy as np
import pytest
import torch

from oracle.attn import attn_mixed, key_range, CAUSAL, BIDIR
from workloads import Seq, pack_seqs


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _expand_kv(k, group):
    # GQA: query head h reads KV head h // group
    return np.repeat(k, group, axis=1)


def _sdpa(q, k, v, mask=None, causal=False):
    """torch scaled_dot_product_attention on CPU float64; q [N,H,D], k/v [L,H,D]."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, is_causal=causal)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("P,N", [(0, 7), (5, 9), (16, 16), (13, 3)])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 1)])
def test_global_causal_equals_sdpa_is_causal(P, N, hq, hkv):
    """P-A2: causal global = rows [P, P+N) of causal SDPA over the whole sequence."""
    D = 8
    L = P + N
    qfull = _rand((L, hq, D), 1)
    k = _rand((L, hkv, D), 2)
    v = _rand((L, hkv, D), 3)
    q = qfull[P:]
    out, _ = attn_mixed([Seq(0, N, 0, P, CAUSAL)], -1, q, k, v, hq, hkv)
    g = hq // hkv
    ref = _sdpa(qfull, _expand_kv(k, g), _expand_kv(v, g), causal=True)[P:]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P,N", [(0, 7), (5, 9), (16, 16)])
def test_global_bidir_equals_unmasked_sdpa(P, N):
    """P-A2: bidirectional global = unmasked SDPA of the N queries over all P+N keys."""
    hq, hkv, D = 4, 2, 8
    q = _rand((N, hq, D), 4)
    k = _rand((P + N, hkv, D), 5)
    v = _rand((P + N, hkv, D), 6)
    out, lse = attn_mixed([Seq(0, N, 0, P, BIDIR)], -1, q, k, v, hq, hkv)
    ref = _sdpa(q, _expand_kv(k, 2), _expand_kv(v, 2))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse against the log-sum-exp of the raw scores
    s = np.einsum("nhd,khd->nhk", q, _expand_kv(k, 2)) / np.sqrt(D)
    mx = s.max(-1, keepdims=True)
    np.testing.assert_allclose(lse, (mx + np.log(np.exp(s - mx).sum(-1, keepdims=True)))[..., 0], rtol=1e-12)


def _page_mask(mode, P, N, W):
    """Dense allowed[i, key] from per-pair predicates, one (query, key) pair at a time."""
    allowed = np.zeros((N, P + N), dtype=bool)
    for i, key in itertools.product(range(N), range(P + N)):
        pos = P + i
        if mode == CAUSAL:
            ok = key <= pos and (W < 0 or pos - key <= W)
        else:
            ok = W < 0 or abs(pos - key) <= W
        allowed[i, key] = ok
    return allowed


@pytest.mark.parametrize("mode", [CAUSAL, BIDIR])
@pytest.mark.parametrize("W", [-1, 0, 1, 2, 3, 100])
@pytest.mark.parametrize("P,N", [(0, 5), (4, 6), (16, 16), (9, 2)])
def test_dense_mask_brute_force(mode, W, P, N):
    """P-A1: masked SDPA (library) with a mask built pair by pair from the window rule."""
    hq, hkv, D = 2, 1, 4
    q = _rand((N, hq, D), 7)
    k = _rand((P + N, hkv, D), 8)
    v = _rand((P + N, hkv, D), 9)
    out, _ = attn_mixed([Seq(0, N, 0, P, mode)], W, q, k, v, hq, hkv)
    mask = _page_mask(mode, P, N, W)
    ref = _sdpa(q, _expand_kv(k, 2), _expand_kv(v, 2), mask=mask[None, None].repeat(hq, 1))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def _key_sets_via_onehot(mode, P, N, W):
    """With Q = 0 the weights are uniform over the key set; a one-hot V per key reads
    the set back from the output, and lse = ln |set|."""
    L = P + N
    q = np.zeros((N, 1, L))
    k = _rand((L, 1, L), 10)
    v = np.eye(L)[:, None, :]
    out, lse = attn_mixed([Seq(0, N, 0, P, mode)], W, q, k, v, 1, 1)
    return out[:, 0, :], lse[:, 0]


def test_window_cover_bidir_canvas256_prefix256():
    """P-A3: a bidirectional query sees 2W+1 keys where the window fits (the canvas
    of 256 tokens on a 256-token prefix with W = 32), and the clipped count at the end."""
    P, N, W = 256, 256, 32
    out, lse = _key_sets_via_onehot(BIDIR, P, N, W)
    counts = np.rint(1.0 / out.max(axis=1)).astype(int)
    members = out > 0
    for i in range(N):
        pos = P + i
        want = 2 * W + 1 if i <= 223 else 288 - i
        assert counts[i] == want == members[i].sum()
        assert abs(lse[i] - np.log(want)) < 1e-12
        idx = np.nonzero(members[i])[0]
        assert idx[0] == pos - W and idx[-1] == min(P + N - 1, pos + W)
        np.testing.assert_allclose(out[i, idx], 1.0 / want, rtol=1e-12)


def test_window_cover_causal():
    """P-A3: a causal query at position q >= W sees W+1 keys (the W before it and itself);
    earlier ones see q+1."""
    P, N, W = 8, 40, 5
    out, lse = _key_sets_via_onehot(CAUSAL, P, N, W)
    for i in range(N):
        pos = P + i
        want = W + 1 if pos >= W else pos + 1
        members = np.nonzero(out[i] > 0)[0]
        assert len(members) == want
        assert members[-1] == pos and members[0] == pos - want + 1


def test_window_zero_is_self_and_huge_window_is_global():
    """P-A4: W = 0 returns the token's own value row exactly; W >= P+N equals global."""
    P, N, hq, hkv, D = 6, 9, 4, 2, 8
    q = _rand((N, hq, D), 11)
    k = _rand((P + N, hkv, D), 12)
    v = _rand((P + N, hkv, D), 13)
    for mode in (CAUSAL, BIDIR):
        out, lse = attn_mixed([Seq(0, N, 0, P, mode)], 0, q, k, v, hq, hkv)
        for i in range(N):
            for h in range(hq):
                assert np.array_equal(out[i, h], v[P + i, h // 2])
        wide, _ = attn_mixed([Seq(0, N, 0, P, mode)], P + N + 3, q, k, v, hq, hkv)
        glob, _ = attn_mixed([Seq(0, N, 0, P, mode)], -1, q, k, v, hq, hkv)
        assert np.array_equal(wide, glob)


@pytest.mark.parametrize("W", [-1, 3])
@pytest.mark.parametrize("mode", [CAUSAL, BIDIR])
def test_gqa_equals_repeated_mha(W, mode):
    """P-A5: repeating each KV head G times and running MHA gives the same result."""
    P, N, hq, hkv, D = 5, 7, 8, 2, 4
    q = _rand((N, hq, D), 14)
    k = _rand((P + N, hkv, D), 15)
    v = _rand((P + N, hkv, D), 16)
    a, la = attn_mixed([Seq(0, N, 0, P, mode)], W, q, k, v, hq, hkv)
    b, lb = attn_mixed([Seq(0, N, 0, P, mode)], W, q, _expand_kv(k, 4), _expand_kv(v, 4), hq, hq)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_batch_independence():
    """P-A6: a request's output in a mixed batch equals running it alone."""
    spec = [(0, 6, CAUSAL), (7, 3, CAUSAL), (4, 5, BIDIR), (11, 4, BIDIR)]
    seqs = pack_seqs(spec)
    hq, hkv, D = 4, 2, 8
    tq = sum(n for _, n, _ in spec)
    tk = sum(p + n for p, n, _ in spec)
    q = _rand((tq, hq, D), 17)
    k = _rand((tk, hkv, D), 18)
    v = _rand((tk, hkv, D), 19)
    for W in (-1, 2):
        out, lse = attn_mixed(seqs, W, q, k, v, hq, hkv)
        for s in seqs:
            qs = slice(s.q_start, s.q_start + s.num_q)
            ks = slice(s.kv_start, s.kv_start + s.prefix_len + s.num_q)
            alone, lal = attn_mixed([Seq(0, s.num_q, 0, s.prefix_len, s.mode)], W, q[qs], k[ks], v[ks], hq, hkv)
            assert np.array_equal(out[qs], alone) and np.array_equal(lse[qs], lal)


def test_key_range_contains_self_and_row_subset():
    """Every key set contains the query's own position; computing a row subset gives
    the same rows as the full computation."""
    for mode, P, N, W in itertools.product((CAUSAL, BIDIR), (0, 3), (1, 4), (-1, 0, 2)):
        for i in range(N):
            lo, hi = key_range(mode, P, N, W, i)
            assert lo <= P + i <= hi
    seqs = pack_seqs([(3, 5, BIDIR)])
    q = _rand((5, 2, 4), 20)
    k = _rand((8, 1, 4), 21)
    v = _rand((8, 1, 4), 22)
    full, _ = attn_mixed(seqs, 1, q, k, v, 2, 1)
    part, _ = attn_mixed(seqs, 1, q, k, v, 2, 1, rows=[1, 4])
    assert np.array_equal(part[[1, 4]], full[[1, 4]]) and np.isnan(part[0]).all()

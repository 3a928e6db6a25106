"""GPU parity of the FP8 (OCP E4M3) K/V cache through the C ABI: dg_attn_mixed with
kv_fp8 = 1 and dg_kv_write into FP8 pools.

Bar:
- every E4M3 code widens exactly: attention over one key returns v_scale times the
  decoded V row, bit for bit (a power-of-two v_scale keeps the product exact), on the
  register-staged kernel (head_dim 64) and on the LDS-DMA kernel over codes (256);
- with unit scales, FP8 attention equals bf16 attention on the decoded values bit for
  bit at head_dim 64/128 (the same register-staged kernel after the tile is staged; at
  256 the codes run on their own kernel, whose contraction order differs);
- against the oracle on the dequantized inputs: max-relative error per row <= 2e-2
  and lse within 1e-3, the bf16 path's bar (contiguous and paged, head_dim 64/128/256,
  grouped heads, windows, both modes, split-KV chunks);
- dg_kv_write into FP8 pools: every code equal to the oracle's (round to nearest,
  ties to even, saturation at 448), from bf16 and fp32 rows, at a power-of-two scale
  and at a scale whose reciprocal is inexact.
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from oracle.fp8 import attn_mixed_fp8, attn_mixed_paged_fp8, kv_write_fp8, quantize, e4m3_decode
from workloads import pack_seqs, Seq, CAUSAL, BIDIR, normal
from tests.gpu_util import DEV, dev, host, max_rel_rows, say

pytestmark = pytest.mark.gpu


def codes_dev(c: np.ndarray, fp8_dtype: bool = True) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(c, dtype=np.uint8)).to(DEV)
    return t.view(torch.float8_e4m3fn) if fp8_dtype else t


_CODES = {}


def _fp8_kv(seed, shape, scale):
    """Seeded normal K or V rows as E4M3 codes at `scale` (values up to ~4.5 sigma
    land near the top of the format at scale 1/64); memoised, as the large ones take
    seconds to quantize."""
    key = (seed, tuple(shape), scale)
    if key not in _CODES:
        _CODES[key] = quantize(normal(seed, shape), scale)
    return _CODES[key]


@pytest.mark.parametrize("D", [64, 256])
def test_every_code_widens_exactly(D):
    # V rows hold all 254 non-NaN codes (the two NaN codes replaced by +-1); at head_dim
    # 256 (the LDS-DMA kernel over codes) each of the 4 rows is the code list rotated by
    # 64, so every code passes through 4 different dims (lanes and fragments)
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x38, 0xB8
    v = codes.reshape(4, 1, D) if D == 64 else np.stack([np.roll(codes, 64 * r) for r in range(4)]).reshape(4, 1, D)
    k = np.full_like(v, 0x38)
    q = normal(401 + D, (4, 1, D), bf16=True)
    seqs = [Seq(i, 1, i, 0, BIDIR) for i in range(4)]
    for vs in (1.0, 0.125):
        out = torch.empty(4, 1, D, device=DEV, dtype=torch.bfloat16)
        lse = torch.empty(4, 1, device=DEV)
        dg.dg_attn_mixed(dev(q, True), codes_dev(k), codes_dev(v), out, seqs, -1, 1, 1, lse=lse,
                         k_scale=0.5, v_scale=vs)
        torch.cuda.synchronize()
        want = e4m3_decode(v) * vs
        assert np.array_equal(host(out).astype(np.float64), want), vs
        wl = (q.astype(np.float64) * 0.5).sum(axis=-1) / np.sqrt(D)
        assert np.abs(host(lse) - wl).max() < 1e-5


@pytest.mark.parametrize("D", [64, 128])
def test_unit_scales_equal_bf16_on_decoded_values(D):
    spec = [(300, 77, CAUSAL), (0, 45, BIDIR), (1000, 64, BIDIR)]
    hq, hkv = 8, 2
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q = normal(411, (T, hq, D), bf16=True)
    kc, vc = _fp8_kv(412, (S, hkv, D), 1 / 64), _fp8_kv(413, (S, hkv, D), 1 / 64)
    for window in (-1, 100):
        o8 = torch.empty(T, hq, D, device=DEV, dtype=torch.bfloat16)
        ob = torch.empty_like(o8)
        l8 = torch.empty(T, hq, device=DEV)
        lb = torch.empty_like(l8)
        dg.dg_attn_mixed(dev(q, True), codes_dev(kc), codes_dev(vc, False), o8, seqs, window, hq, hkv, lse=l8)
        dg.dg_attn_mixed(dev(q, True), dev(e4m3_decode(kc), True), dev(e4m3_decode(vc), True), ob, seqs, window,
                         hq, hkv, lse=lb)
        torch.cuda.synchronize()
        assert torch.equal(o8.view(torch.int16), ob.view(torch.int16)), window
        assert torch.equal(l8.view(torch.int32), lb.view(torch.int32)), window


CASES = [
    # label, spec, window, hq, hkv, D, kv_chunk, k_scale, v_scale
    ("d64 G=2 mixed W=16", [(100, 40, CAUSAL), (37, 64, BIDIR)], 16, 4, 2, 64, 0, 0.05, 0.02),
    ("d128 G=4 ragged global", [(300, 77, CAUSAL), (0, 45, BIDIR)], -1, 8, 2, 128, 0, 1 / 64, 1 / 32),
    ("d256 canvas 256 prefix 4096", [(4096, 256, BIDIR)], -1, 16, 8, 256, 0, 1 / 64, 1 / 64),
    ("d256 mixed W=512 forced chunks", [(0, 300, CAUSAL), (1000, 256, BIDIR), (5000, 64, CAUSAL)], 512, 16, 8,
     256, 256, 0.013, 0.021),
    # degenerate requests: no queries, a single token with no cache, W = 0 (itself only)
    ("d128 edges: empty, one-token, W=0", [(50, 0, BIDIR), (0, 1, CAUSAL), (63, 1, BIDIR), (70, 30, CAUSAL)], 0,
     8, 8, 128, 0, 0.5, 0.25),
    ("d64 edges: empty, one-token, global", [(50, 0, BIDIR), (0, 1, BIDIR), (0, 1, CAUSAL), (129, 65, BIDIR)], -1,
     2, 1, 64, 64, 0.07, 0.09),
    # head_dim 256 on the LDS-DMA kernel over codes: chunks of 1 to 7 sub-tiles with ragged
    # last sub-tiles (the ring's repeated rows), one-token and empty requests, a window
    ("d256 short chunks, ragged tails", [(37, 29, CAUSAL), (100, 61, BIDIR), (0, 33, BIDIR), (200, 1, BIDIR),
                                         (10, 0, CAUSAL)], -1, 8, 2, 256, 64, 0.02, 0.03),
    ("d256 W=40 chunks of 192 keys", [(300, 70, CAUSAL), (5, 130, BIDIR)], 40, 16, 8, 256, 192, 0.011, 0.017),
    ("d256 G=8 one q tile, long prefix", [(3000, 16, BIDIR)], -1, 16, 2, 256, 0, 1 / 64, 1 / 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_attention_against_oracle(case):
    label, spec, window, hq, hkv, D, chunk, ks, vs = case
    say(f"[fp8 attn] {label}")
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q = normal(421, (T, hq, D), bf16=True)
    kc, vc = _fp8_kv(422, (S, hkv, D), ks), _fp8_kv(423, (S, hkv, D), vs)
    out = torch.full((T, hq, D), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((T, hq), float("nan"), device=DEV)
    dg.dg_attn_mixed(dev(q, True), codes_dev(kc), codes_dev(vc), out, seqs, window, hq, hkv, lse=lse,
                     kv_chunk=chunk, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    # every row at the small sizes, sampled rows at the canvas-over-4096 size
    rows = None if T * S * hq < 1e7 else np.random.default_rng(424).choice(T, 24, replace=False)
    want, wlse = attn_mixed_fp8(seqs, window, q, kc, vc, ks, vs, hq, hkv, rows=rows)
    got, glse = host(out), host(lse)
    if rows is not None:
        got, glse, want, wlse = got[rows], glse[rows], want[rows], wlse[rows]
    err = max_rel_rows(got, want)
    lerr = float(np.abs(glse - wlse).max())
    say(f"  max-rel {err:.3e}  lse abs {lerr:.3e}")
    assert err <= 2e-2 and lerr <= 1e-3


# The 64-rows-per-wave kernel over codes at small shapes: with the planner's threshold
# lowered to 16 sub-tiles per work group (test hook) these requests run on it.
WIDE_CASES = [
    # label, spec, window, hq, hkv, kv_chunk, k_scale, v_scale
    ("wide bidir G=2", [(2048, 200, BIDIR)], -1, 4, 2, 1024, 1 / 64, 1 / 64),
    ("wide causal W=300 G=2", [(2048, 200, CAUSAL)], 300, 4, 2, 1024, 0.013, 0.021),
    ("wide G=8 ragged, two requests", [(2048, 100, BIDIR), (1500, 77, CAUSAL)], -1, 16, 2, 1024, 1 / 64, 1 / 32),
    ("wide G=16 W=600 causal", [(2048, 37, CAUSAL)], 600, 32, 2, 1024, 0.02, 0.03),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_fp8_wide_kernel_against_oracle(case):
    label, spec, window, hq, hkv, chunk, ks, vs = case
    say(f"[fp8 wide] {label}")
    D = 256
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q = normal(431, (T, hq, D), bf16=True)
    kc, vc = _fp8_kv(432, (S, hkv, D), ks), _fp8_kv(433, (S, hkv, D), vs)
    out = torch.full((T, hq, D), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((T, hq), float("nan"), device=DEV)
    with dg.wide_min_sub(16):
        dg.dg_attn_mixed(dev(q, True), codes_dev(kc), codes_dev(vc), out, seqs, window, hq, hkv, lse=lse,
                         kv_chunk=chunk, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
    want, wlse = attn_mixed_fp8(seqs, window, q, kc, vc, ks, vs, hq, hkv)
    err = max_rel_rows(host(out), want)
    lerr = float(np.abs(host(lse) - wlse).max())
    say(f"  max-rel {err:.3e}  lse abs {lerr:.3e}")
    assert err <= 2e-2 and lerr <= 1e-3


@pytest.mark.parametrize("wide", [False, True])
def test_fp8_score_jump_recomputes(wide):
    """Keys after the first 32 score far above the first ones (about 2^92 in log2 units):
    both head_dim-256 kernels over codes fix each row's reference from its first scores,
    have to recompute the chunk, and still match the oracle."""
    P, N, H, D, ks, vs = 2048, 64, 2, 256, 1 / 64, 1 / 64
    rng = np.random.default_rng(93)
    q = 0.5 + 0.05 * rng.standard_normal((N, H, D))
    k = 0.25 + 0.05 * rng.standard_normal((P + N, H, D))
    k[:32] *= -1.0
    v = rng.standard_normal((P + N, H, D))
    q = q.astype(np.float32)
    kc, vc = quantize(k, ks), quantize(v, vs)
    seqs = pack_seqs([(P, N, BIDIR)])
    qd = dev(q, True)
    want, wlse = attn_mixed_fp8(seqs, -1, host(qd).astype(np.float64), kc, vc, ks, vs, H, H, scale=1.0)
    for chunk in (4096, 1024):
        out = torch.full((N, H, D), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((N, H), float("nan"), device=DEV)
        with dg.wide_min_sub(16 if wide else 1 << 30):
            dg.dg_attn_mixed(qd, codes_dev(kc), codes_dev(vc), out, seqs, -1, H, H, lse=lse, scale=1.0,
                             kv_chunk=chunk, k_scale=ks, v_scale=vs)
            torch.cuda.synchronize()
        err = max_rel_rows(host(out), want)
        lerr = float(np.abs(host(lse) - wlse).max())
        say(f"[fp8 score jump] wide={wide} chunk={chunk}: max-rel {err:.3e}  lse abs {lerr:.3e}")
        assert err <= 2e-2 and lerr <= 1e-3


@pytest.mark.parametrize("window", [-1, 512])
def test_fp8_mixed_four_request_batch_sampled(window):
    """The four-request mixed batch at its full size (a 2048-token causal prefill, a causal
    commit after 8192 tokens, denoise canvases after 1024 and 16384), over an FP8 cache,
    in the launch configuration the per-call timings use; sampled rows of every request."""
    spec = [(0, 2048, CAUSAL), (8192, 256, CAUSAL), (1024, 256, BIDIR), (16384, 256, BIDIR)]
    hq, hkv, D, sc = 16, 8, 256, 1.0 / 64
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    S = sum(p + n for p, n, _ in spec)
    q = normal(461, (T, hq, D), bf16=True)
    kc, vc = _fp8_kv(462, (S, hkv, D), sc), _fp8_kv(463, (S, hkv, D), sc)
    out = torch.empty(T, hq, D, device=DEV, dtype=torch.bfloat16)
    lse = torch.empty(T, hq, device=DEV)
    say(f"[fp8 4-request batch] W={window}")
    dg.dg_attn_mixed(dev(q, True), codes_dev(kc), codes_dev(vc), out, seqs, window, hq, hkv, lse=lse, k_scale=sc,
                     v_scale=sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(464)
    rows = np.concatenate([s.q_start + np.concatenate([[0, s.num_q - 1], rng.choice(s.num_q, 6, replace=False)])
                           for s in seqs])
    want, wlse = attn_mixed_fp8(seqs, window, q, kc, vc, sc, sc, hq, hkv, rows=rows)
    err = max_rel_rows(host(out)[rows], want[rows])
    lerr = float(np.abs(host(lse)[rows] - wlse[rows]).max())
    say(f"  max-rel {err:.3e}  lse abs {lerr:.3e}")
    assert err <= 2e-2 and lerr <= 1e-3


def test_fp8_paged_attention_against_oracle():
    B, hq, hkv, D = 64, 16, 8, 256
    spec = [(130, 64, BIDIR), (0, 70, CAUSAL), (200, 19, BIDIR)]
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    nbs = [-(-(p + n) // B) for p, n, _ in spec]
    nblk = sum(nbs) + 3
    table = np.random.default_rng(431).permutation(nblk)[:sum(nbs)].astype(np.int32)
    pseqs, start = [], 0
    for s, nb in zip(seqs, nbs):
        pseqs.append(Seq(s.q_start, s.num_q, start, s.prefix_len, s.mode))
        start += nb
    kc, vc = _fp8_kv(432, (nblk * B, hkv, D), 0.02), _fp8_kv(433, (nblk * B, hkv, D), 0.03)
    q = normal(434, (T, hq, D), bf16=True)
    tt = torch.from_numpy(table).to(DEV)
    for window in (-1, 40):
        out = torch.empty(T, hq, D, device=DEV, dtype=torch.bfloat16)
        lse = torch.empty(T, hq, device=DEV)
        dg.dg_attn_mixed(dev(q, True), codes_dev(kc), codes_dev(vc), out, pseqs, window, hq, hkv, lse=lse,
                         block_table=tt, block_size=B, k_scale=0.02, v_scale=0.03)
        torch.cuda.synchronize()
        want, wlse = attn_mixed_paged_fp8(pseqs, window, q, kc, vc, 0.02, 0.03, table, B, hq, hkv)
        err = max_rel_rows(host(out), want)
        lerr = float(np.abs(host(lse) - wlse).max())
        say(f"[fp8 paged] W={window}: max-rel {err:.3e}  lse abs {lerr:.3e}")
        assert err <= 2e-2 and lerr <= 1e-3


def test_fp8_paged_wide_kernel_against_oracle():
    """Paged FP8 pools on the 64-rows-per-wave kernel over codes (threshold hook, chunks of
    1024 keys): shuffled 64-row blocks, a bidirectional and a causal request, global and
    windowed."""
    B, hq, hkv, D, ks, vs = 64, 8, 2, 256, 0.02, 0.03
    spec = [(2048, 64, BIDIR), (1500, 70, CAUSAL)]
    seqs = pack_seqs(spec)
    T = sum(n for _, n, _ in spec)
    nbs = [-(-(p + n) // B) for p, n, _ in spec]
    nblk = sum(nbs) + 5
    table = np.random.default_rng(435).permutation(nblk)[:sum(nbs)].astype(np.int32)
    pseqs, start = [], 0
    for s, nb in zip(seqs, nbs):
        pseqs.append(Seq(s.q_start, s.num_q, start, s.prefix_len, s.mode))
        start += nb
    kc, vc = _fp8_kv(436, (nblk * B, hkv, D), ks), _fp8_kv(437, (nblk * B, hkv, D), vs)
    q = normal(438, (T, hq, D), bf16=True)
    tt = torch.from_numpy(table).to(DEV)
    for window in (-1, 300):
        out = torch.empty(T, hq, D, device=DEV, dtype=torch.bfloat16)
        lse = torch.empty(T, hq, device=DEV)
        with dg.wide_min_sub(16):
            dg.dg_attn_mixed(dev(q, True), codes_dev(kc), codes_dev(vc), out, pseqs, window, hq, hkv, lse=lse,
                             kv_chunk=1024, block_table=tt, block_size=B, k_scale=ks, v_scale=vs)
            torch.cuda.synchronize()
        want, wlse = attn_mixed_paged_fp8(pseqs, window, q, kc, vc, ks, vs, table, B, hq, hkv)
        err = max_rel_rows(host(out), want)
        lerr = float(np.abs(host(lse) - wlse).max())
        say(f"[fp8 paged wide] W={window}: max-rel {err:.3e}  lse abs {lerr:.3e}")
        assert err <= 2e-2 and lerr <= 1e-3


def _special_values():
    """Ties between neighbouring E4M3 values, saturation, the subnormal range, signed zeros."""
    pos = e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    extra = np.array([0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e4, -1e4, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -12,
                      -(2.0 ** -9), 0.0009765625 * 1.5])
    return np.concatenate([mids, -mids, pos, -pos, extra])


@pytest.mark.parametrize("bf16,scale", [(True, 1.0), (False, 1.0), (True, 0.37), (False, 0.0123)])
def test_kv_write_fp8_codes_match_oracle(bf16, scale):
    B, hkv, D = 16, 2, 64
    nblocks = 40
    sp = _special_values()
    n_new = 96
    k_new = normal(441, (n_new, hkv, D), std=2.0, bf16=bf16).astype(np.float32)
    v_new = normal(442, (n_new, hkv, D), std=1000.0, bf16=bf16).astype(np.float32)  # many saturate at 448
    flat = k_new.reshape(-1)
    flat[:sp.size] = sp * scale  # ties and special values land exactly at scale 1 (and bf16-exact)
    if bf16:
        k_new = torch.from_numpy(k_new).to(torch.bfloat16).float().numpy()
    table = np.random.default_rng(443).permutation(nblocks).astype(np.int32)
    seqs = [(0, 60, 0, 5), (60, 36, 20, 0)]
    kp = np.zeros((nblocks * B, hkv, D), np.uint8)
    vp = np.zeros_like(kp)
    say(f"[fp8 kv_write] bf16={bf16} scale={scale}")
    want_k, want_v = kv_write_fp8(kp, vp, k_new, v_new, seqs, table, B, scale, 2 * scale)
    kpt, vpt = codes_dev(kp), codes_dev(vp, False)
    dg.dg_kv_write(dev(k_new, bf16), dev(v_new, bf16), kpt, vpt, seqs, torch.from_numpy(table).to(DEV), B,
                   k_scale=scale, v_scale=2 * scale)
    torch.cuda.synchronize()
    got_k, got_v = host(kpt.view(torch.uint8)), host(vpt)
    bad = np.flatnonzero(got_k.reshape(-1) != want_k.reshape(-1))
    assert bad.size == 0, (bad[:8], got_k.reshape(-1)[bad[:8]], want_k.reshape(-1)[bad[:8]])
    assert np.array_equal(got_v, want_v)
    assert (want_v == 0x7E).any() and (want_v == 0xFE).any()  # saturation was exercised


def test_fp8_prefill_and_draft_then_attention_against_oracle():
    """A prompt and a canvas draft quantized into FP8 pools by dg_kv_write, then paged
    FP8 attention of the canvas, against the oracle's own writes and attention."""
    B, hq, hkv, D, P, N = 64, 16, 8, 256, 1000, 256
    nb = -(-(P + N) // B)
    table = np.random.default_rng(451).permutation(nb + 2)[:nb].astype(np.int32)
    ks, vs = 0.011, 0.017
    pk, pv = normal(452, (P, hkv, D), bf16=True), normal(453, (P, hkv, D), bf16=True)
    dk, dv = normal(454, (N, hkv, D), bf16=True), normal(455, (N, hkv, D), bf16=True)
    q = normal(456, (N, hq, D), bf16=True)
    kp = np.zeros(((nb + 2) * B, hkv, D), np.uint8)
    vp = np.zeros_like(kp)
    kpt, vpt, tt = codes_dev(kp), codes_dev(vp), torch.from_numpy(table).to(DEV)
    dg.dg_kv_write(dev(pk, True), dev(pv, True), kpt, vpt, [(0, P, 0, 0)], tt, B, k_scale=ks, v_scale=vs)
    dg.dg_kv_write(dev(dk, True), dev(dv, True), kpt, vpt, [(0, N, 0, P)], tt, B, k_scale=ks, v_scale=vs)
    out = torch.empty(N, hq, D, device=DEV, dtype=torch.bfloat16)
    seqs = [Seq(0, N, 0, P, BIDIR)]
    dg.dg_attn_mixed(dev(q, True), kpt, vpt, out, seqs, -1, hq, hkv, block_table=tt, block_size=B,
                     k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kp, vp = kv_write_fp8(kp, vp, pk, pv, [(0, P, 0, 0)], table, B, ks, vs)
    kp, vp = kv_write_fp8(kp, vp, dk, dv, [(0, N, 0, P)], table, B, ks, vs)
    assert np.array_equal(host(kpt.view(torch.uint8)), kp) and np.array_equal(host(vpt.view(torch.uint8)), vp)
    rows = np.random.default_rng(457).choice(N, 32, replace=False)
    want, _ = attn_mixed_paged_fp8(seqs, -1, q, kp, vp, ks, vs, table, B, hq, hkv, rows=rows)
    err = max_rel_rows(host(out)[rows], want[rows])
    say(f"[fp8 prefill+draft] max-rel {err:.3e}")
    assert err <= 2e-2

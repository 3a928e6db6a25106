"""GPU parity of dg_attn_mixed against the CPU oracle, through the C ABI.

Bar: max-relative error per (token, head) output row <= 2e-2 (bf16 inputs, fp32
accumulation; fp32 inputs are checked against the same bar and expected far
inside it), lse within 1e-3 absolute. Full-size configurations are checked on
sampled query rows that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import block_denoising_step_amd as dg
from oracle.attn import attn_mixed as ref_attn
from workloads import attn_case, pack_seqs, Seq, CAUSAL, BIDIR, normal, round_to_bf16
from tests.gpu_util import DEV, dev, host, max_rel_rows, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _gpu(case_seqs, window, q, k, v, hq, hkv, bf16, kv_chunk=0, out_fill=np.nan, scale=0.0):
    qt, kt, vt = dev(q, bf16), dev(k, bf16), dev(v, bf16)
    out = torch.full(qt.shape, out_fill, device=DEV, dtype=qt.dtype)
    lse = torch.full(qt.shape[:2], np.nan, device=DEV, dtype=torch.float32)
    dg.dg_attn_mixed(qt, kt, vt, out, case_seqs, window, hq, hkv, lse=lse, kv_chunk=kv_chunk, scale=scale)
    torch.cuda.synchronize()
    return host(out), host(lse)


def _compare(seqs, window, q, k, v, hq, hkv, bf16, rows=None, kv_chunk=0, label="", scale=0.0):
    say(f"[attn] {label}: W={window} rows={'all' if rows is None else len(rows)} chunk={kv_chunk}")
    out, lse = _gpu(seqs, window, q, k, v, hq, hkv, bf16, kv_chunk, scale=scale)
    want, wlse = ref_attn(seqs, window, q, k, v, hq, hkv, scale=scale or None, rows=rows)
    sel = np.arange(q.shape[0]) if rows is None else np.array(rows)
    err = max_rel_rows(out[sel], want[sel])
    lerr = float(np.abs(lse[sel] - wlse[sel]).max())
    say(f"  max-rel {err:.3e}  lse abs {lerr:.3e}")
    assert err <= TOL and lerr <= 1e-3, (label, err, lerr)
    # rows of no request are untouched (still NaN)
    covered = np.zeros(q.shape[0], bool)
    for s in seqs:
        covered[s.q_start:s.q_start + s.num_q] = True
    assert np.isnan(out[~covered]).all()
    return err, out


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
@pytest.mark.parametrize("window", [32, -1])
def test_fp32_canvas256_prefix256_heads4_d64(mode, window):
    c = attn_case(1).with_mode(mode).with_window(window)
    q, k, v = c.tensors()
    err, _ = _compare(c.seqs, window, q, k, v, c.num_q_heads, c.num_kv_heads, False, label=f"fp32 canvas 256 prefix 256 mode={mode}")
    assert err < 1e-4


def test_bf16_canvas256_prefix4096_all_rows():
    c = attn_case(2)
    q, k, v = c.tensors()
    _compare(c.seqs, -1, q, k, v, 16, 8, True, label="bf16 bidir global canvas 256 prefix 4096")


@pytest.mark.parametrize("mode", [BIDIR, CAUSAL])
def test_bf16_window512_prefix32768_sampled(mode):
    c = attn_case(3).with_mode(mode)
    q, k, v = c.tensors()
    # every q-tile edge: 64 tokens per 128-row tile at G = 2
    rows = [0, 1, 63, 64, 100, 127, 128, 191, 192, 200, 254, 255]
    _compare(c.seqs, 512, q, k, v, 16, 8, True, rows=rows, label=f"bf16 W=512 prefix 32768 mode={mode}")


@pytest.mark.parametrize("window", [-1, 512])
def test_bf16_mixed_four_request_batch_sampled(window):
    c = attn_case(4)
    q, k, v = c.tensors()
    rows = []
    for s in c.seqs:
        rows += [s.q_start, s.q_start + 1, s.q_start + s.num_q // 2, s.q_start + s.num_q - 1]
        # the q-tile edges of both kernels (64 or 128 tokens per tile at G = 2)
        rows += [s.q_start + i for i in range(63, s.num_q - 1, 64)] + [s.q_start + i for i in range(64, s.num_q, 64)]
    rows += [700, 1500, 2047]
    _compare(c.seqs, window, q, k, v, 16, 8, True, rows=sorted(set(rows)), label=f"bf16 mixed 4-request batch W={window}")


def test_bf16_prefixes_to_262144_sampled():
    c = attn_case(5)
    q, k, v = c.tensors()
    rows = []
    for s in c.seqs:
        # first and last rows and the q-tile edges of both kernels (64 or 128 tokens per tile)
        rows += [s.q_start + i for i in (0, 63, 64, 127, 128, 129, 191, 192, s.num_q - 1)]
    _compare(c.seqs, -1, q, k, v, 16, 8, True, rows=rows, label="bf16 prefixes 262144/131072/65536/4096")


@pytest.mark.parametrize("D,bf16", [(64, True), (128, True), (256, True), (64, False), (128, False)])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (16, 2), (16, 1), (32, 1)])
def test_shapes_ragged_and_split(D, bf16, hq, hkv):
    """Ragged token counts, empty prefix, empty request, forced key splits, every
    supported head_dim and group size, both modes, windows."""
    spec = [(0, 37, CAUSAL), (70, 0, BIDIR), (130, 45, BIDIR), (5, 200, CAUSAL)]
    seqs = pack_seqs(spec)
    tq = sum(n for _, n, _ in spec)
    tk = sum(p + n for p, n, _ in spec)
    seed = 1000 + D + hq
    q = normal(seed, (tq, hq, D), bf16=bf16)
    k = normal(seed + 1, (tk, hkv, D), bf16=bf16)
    v = normal(seed + 2, (tk, hkv, D), bf16=bf16)
    for window, chunk in ((-1, 0), (-1, 64), (17, 0), (0, 0), (40, 128), (9, 64)):
        _compare(seqs, window, q, k, v, hq, hkv, bf16, kv_chunk=chunk,
                 label=f"D={D} bf16={bf16} G={hq // hkv}")


@pytest.mark.parametrize("chunk", [0, 64, 128, 192])
def test_short_chunks_ring_edges(chunk):
    """The 128-row kernel issues one ring stage per sub-tile whatever the chunk's length
    (stages past its end repeat its last sub-tile, clamped to the request's keys), so every
    length from one sub-tile up, with ragged last sub-tiles, is checked: key counts 1, 20,
    32, 33, 64, 65, 100, 129 and 200 (one to seven 32-key sub-tiles), split into chunks of
    64, 128 or 192 keys, in one batch, against the oracle."""
    spec = [(0, 1, BIDIR), (10, 10, BIDIR), (0, 32, CAUSAL), (20, 13, BIDIR), (40, 24, CAUSAL),
            (60, 5, BIDIR), (90, 10, BIDIR), (100, 29, CAUSAL), (150, 50, BIDIR)]
    seqs = pack_seqs(spec)
    tq = sum(n for _, n, _ in spec)
    tk = sum(p + n for p, n, _ in spec)
    q = normal(7100 + chunk, (tq, 16, 256), bf16=True)
    k = normal(7101 + chunk, (tk, 8, 256), bf16=True)
    v = normal(7102 + chunk, (tk, 8, 256), bf16=True)
    for window in (-1, 24):
        _compare(seqs, window, q, k, v, 16, 8, True, kv_chunk=chunk, label=f"short chunks chunk={chunk} W={window}")


def test_batch_independence_bit_exact():
    """A request's output does not depend on the rest of the batch (work split per request)."""
    c = attn_case(4)
    q, k, v = c.tensors()
    _, full = _compare(c.seqs, 512, q, k, v, 16, 8, True, rows=[c.seqs[2].q_start], label="batch")
    for s in c.seqs[1:3]:
        qs = slice(s.q_start, s.q_start + s.num_q)
        ks = slice(s.kv_start, s.kv_start + s.prefix_len + s.num_q)
        alone, _ = _gpu([Seq(0, s.num_q, 0, s.prefix_len, s.mode)], 512, q[qs], k[ks], v[ks], 16, 8, True)
        assert np.array_equal(alone, full[qs])


def test_repeat_is_bit_identical():
    c = attn_case(2)
    q, k, v = c.tensors()
    a, la = _gpu(c.seqs, -1, q, k, v, 16, 8, True)
    b, lb = _gpu(c.seqs, -1, q, k, v, 16, 8, True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("D,bf16", [(256, True), (128, True), (128, False)])
def test_score_jump_far_past_first_tile(D, bf16):
    """Keys after the first 32 score far above the first ones (by 2^91 in log2 units at
    head_dim 256): a
    kernel that fixes each row's softmax reference from its first scores has to
    recompute, and the result still matches the oracle."""
    P, N, H = 96, 40, 2
    rng = np.random.default_rng(77 + D)
    q = 0.5 + 0.05 * rng.standard_normal((N, H, D))
    k = 0.25 + 0.05 * rng.standard_normal((P + N, H, D))
    k[:32] *= -1.0
    v = rng.standard_normal((P + N, H, D))
    q, k, v = (x.astype(np.float32) for x in (q, k, v))
    if bf16:
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    seqs = pack_seqs([(P, N, BIDIR)])
    for chunk in (0, 64):
        _compare(seqs, -1, q, k, v, H, H, bf16, kv_chunk=chunk, scale=1.0, label=f"score jump D={D}")


# The 64-rows-per-wave kernel at small shapes: with the planner's threshold lowered to 16
# sub-tiles per work group (test hook), these requests and chunks run on it: masks,
# windows, group sizes, ragged q tiles, 256-row partials and the merge over them.
WIDE_MIN_SUB = 16
WIDE_CASES = [
    # mode, window, G, N, kv_chunk
    (BIDIR, -1, 2, 200, 1024),
    (CAUSAL, -1, 2, 200, 1024),
    (BIDIR, 300, 2, 200, 1024),
    (CAUSAL, 1000, 4, 130, 4096),
    (BIDIR, 700, 1, 64, 2048),
    (BIDIR, -1, 8, 100, 1024),
    (BIDIR, -1, 16, 40, 1024),
    (CAUSAL, 600, 16, 37, 1024),
    (BIDIR, 300, 32, 21, 1024),
    (CAUSAL, -1, 32, 13, 2048),
]


@pytest.mark.parametrize("mode,window,G,N,chunk", WIDE_CASES)
def test_wide_kernel_cases(mode, window, G, N, chunk):
    P, hkv, D = 2048, 2, 256
    hq = G * hkv
    seed = 5000 + 7 * G + N
    q = normal(seed, (N, hq, D), bf16=True)
    k = normal(seed + 1, (P + N, hkv, D), bf16=True)
    v = normal(seed + 2, (P + N, hkv, D), bf16=True)
    seqs = pack_seqs([(P, N, mode)])
    with dg.wide_min_sub(WIDE_MIN_SUB):
        _compare(seqs, window, q, k, v, hq, hkv, True, kv_chunk=chunk, label=f"wide mode={mode} G={G} N={N}")


def test_wide_kernel_score_jump():
    """The reference-overflow recomputation on the 64-rows-per-wave kernel: keys after
    the first 32 score far above the first ones."""
    P, N, H, D = 2048, 64, 2, 256
    rng = np.random.default_rng(91)
    q = 0.5 + 0.05 * rng.standard_normal((N, H, D))
    k = 0.25 + 0.05 * rng.standard_normal((P + N, H, D))
    k[:32] *= -1.0
    v = rng.standard_normal((P + N, H, D))
    q, k, v = (round_to_bf16(x.astype(np.float32)) for x in (q, k, v))
    seqs = pack_seqs([(P, N, BIDIR)])
    with dg.wide_min_sub(WIDE_MIN_SUB):
        for chunk in (4096, 1024):
            _compare(seqs, -1, q, k, v, H, H, True, kv_chunk=chunk, scale=1.0, label=f"wide score jump chunk={chunk}")


# ---- the register-staged kernel at head_dim 256 (bf16) ---------------------------------
# It serves contiguous bf16 head_dim-256 requests whose K/V span passes 2^31 - 1 bytes
# (the LDS-DMA kernels address a request's K/V with 32-bit offsets). The test hook puts
# every request on it, so it is checked at small shapes too.

@pytest.mark.parametrize("hq,hkv", [(16, 8), (8, 2), (32, 1)])
def test_register_staged_bf16_d256(hq, hkv):
    spec = [(0, 37, CAUSAL), (70, 0, BIDIR), (130, 45, BIDIR), (5, 200, CAUSAL), (600, 90, BIDIR)]
    seqs = pack_seqs(spec)
    tq = sum(n for _, n, _ in spec)
    tk = sum(p + n for p, n, _ in spec)
    seed = 3100 + hq
    q = normal(seed, (tq, hq, 256), bf16=True)
    k = normal(seed + 1, (tk, hkv, 256), bf16=True)
    v = normal(seed + 2, (tk, hkv, 256), bf16=True)
    with dg.force_register_staged():
        for window, chunk in ((-1, 0), (-1, 64), (17, 0), (0, 0), (40, 128)):
            _compare(seqs, window, q, k, v, hq, hkv, True, kv_chunk=chunk,
                     label=f"register-staged d256 G={hq // hkv}")
        # per-request planning on this kernel too: a request alone gives the same bits
        full, _ = _gpu(seqs, 40, q, k, v, hq, hkv, True)
        s = seqs[4]
        qs = slice(s.q_start, s.q_start + s.num_q)
        ks = slice(s.kv_start, s.kv_start + s.prefix_len + s.num_q)
        alone, _ = _gpu([Seq(0, s.num_q, 0, s.prefix_len, s.mode)], 40, q[qs], k[ks], v[ks], hq, hkv, True)
        assert np.array_equal(alone, full[qs])


def test_kv_span_past_2gib_runs_per_request():
    """A contiguous request whose K/V span passes 2^31 - 1 bytes (524,352 keys x 8 heads x
    256 x bf16) runs on the register-staged kernel; the canvas request beside it in the same
    call stays on the LDS-DMA kernels, so its output is bit-identical to running it alone.
    The long request is checked against the oracle on sampled rows. Inputs are seeded
    normals drawn on the device (torch's generator) and copied to the host for the oracle."""
    P0, N0, P1, N1, hq, hkv, D = 524288, 64, 4096, 256, 16, 8, 256
    assert (P0 + N0) * hkv * D * 2 > 2**31 - 1
    seqs = pack_seqs([(P0, N0, BIDIR), (P1, N1, BIDIR)])
    g = torch.Generator(device=DEV)
    g.manual_seed(90210)
    tq, tk = N0 + N1, P0 + N0 + P1 + N1
    qt = torch.randn(tq, hq, D, device=DEV, generator=g).to(torch.bfloat16)
    kt = torch.randn(tk, hkv, D, device=DEV, generator=g).to(torch.bfloat16)
    vt = torch.randn(tk, hkv, D, device=DEV, generator=g).to(torch.bfloat16)
    say(f"[attn] K/V span past 2 GiB: {tk} key rows, {2 * kt.numel() * 2 / 2**30:.2f} GiB of K/V")
    out = torch.full((tq, hq, D), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((tq, hq), float("nan"), device=DEV, dtype=torch.float32)
    dg.dg_attn_mixed(qt, kt, vt, out, seqs, -1, hq, hkv, lse=lse)
    s1 = seqs[1]
    out1 = torch.empty(N1, hq, D, device=DEV, dtype=torch.bfloat16)
    k1 = kt[s1.kv_start:s1.kv_start + P1 + N1]
    v1 = vt[s1.kv_start:s1.kv_start + P1 + N1]
    dg.dg_attn_mixed(qt[N0:], k1, v1, out1, [Seq(0, N1, 0, P1, BIDIR)], -1, hq, hkv)
    torch.cuda.synchronize()
    assert torch.equal(out[N0:].view(torch.int16), out1.view(torch.int16))
    rows = [0, 31, 32, 63]
    q_np, k_np, v_np = host(qt), host(kt[:P0 + N0]), host(vt[:P0 + N0])
    want, wlse = ref_attn(seqs[:1], -1, q_np[:N0], k_np, v_np, hq, hkv, rows=rows)
    got = host(out)
    err = max_rel_rows(got[rows], want[rows])
    lerr = float(np.abs(host(lse)[rows] - wlse[rows]).max())
    say(f"  long request rows {rows}: max-rel {err:.3e}, lse abs {lerr:.3e}")
    assert err <= TOL and lerr <= 1e-3


@pytest.mark.parametrize("D", [128, 256])
def test_max_requests_64(D):
    """DG_MAX_SEQS requests in one call: ragged prefixes and canvases in both modes,
    some empty; every row against the oracle."""
    rng = np.random.default_rng(64 + D)
    spec = [(int(rng.integers(0, 300)), int(rng.integers(0, 40)), int(rng.integers(0, 2))) for _ in range(64)]
    seqs = pack_seqs(spec)
    tq = sum(n for _, n, _ in spec)
    tk = sum(p + n for p, n, _ in spec)
    q = normal(6400 + D, (tq, 8, D), bf16=True)
    k = normal(6401 + D, (tk, 2, D), bf16=True)
    v = normal(6402 + D, (tk, 2, D), bf16=True)
    for window in (-1, 33):
        _compare(seqs, window, q, k, v, 8, 2, True, label=f"64 requests D={D}")

"""Pins of the FP8 (OCP E4M3) oracle: the format against torch's float8_e4m3fn (a library
implementation of the same format), values the OFP8 definition fixes, rounding ties,
saturation, and closed forms of attention over an FP8 cache."""
import numpy as np
import pytest
import torch

from oracle.fp8 import (e4m3_value, e4m3_decode, e4m3_encode, quantize, dequantize, attn_mixed_fp8,
                        attn_mixed_paged_fp8, kv_write_fp8, E4M3_MAX)
from oracle.attn import attn_mixed, CAUSAL, BIDIR


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine, ref = e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_values_fixed_by_the_format():
    assert e4m3_value(0x7E) == 448.0 == E4M3_MAX       # largest finite
    assert e4m3_value(0x08) == 2.0 ** -6                # smallest normal
    assert e4m3_value(0x01) == 2.0 ** -9                # smallest subnormal
    assert e4m3_value(0x07) == 7 * 2.0 ** -9            # largest subnormal
    assert e4m3_value(0x38) == 1.0                      # exponent field 7 = bias
    assert e4m3_value(0x39) == 1.125
    assert e4m3_value(0xC0) == -2.0
    assert np.isnan(e4m3_value(0x7F)) and np.isnan(e4m3_value(0xFF))
    assert e4m3_value(0x80) == 0.0 and np.signbit(e4m3_value(0x80))
    # 254 distinct non-NaN codes, 253 distinct values (+0 and -0), monotone in the code
    pos = e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_matches_torch_on_random_and_tie_values():
    rng = np.random.default_rng(11)
    x = rng.normal(size=30000) * np.exp(rng.uniform(-14, 6.5, size=30000))
    x = x[np.abs(x) <= E4M3_MAX].astype(np.float32)
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), _torch_encode(x))
    # exact midpoints between neighbouring values, both signs: ties go to the even code
    pos = e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    mids = np.concatenate([mids, -mids]).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (np.concatenate([(pos[:-1] + pos[1:]) / 2,
                                                                    -(pos[:-1] + pos[1:]) / 2])))  # exact in fp32
    got = e4m3_encode(mids.astype(np.float64))
    assert np.array_equal(got, _torch_encode(mids))
    assert np.all(got & 1 == 0)


def test_encode_saturates_and_keeps_nan():
    got = e4m3_encode(np.array([448.0, 449.0, 464.0, 480.0, 1e6, -1e30, np.inf, -np.inf, np.nan, -0.0]))
    assert list(got[:8]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert got[8] == 0x7F and got[9] == 0x80


def test_quantize_uses_the_fp32_reciprocal():
    x = np.random.default_rng(12).normal(size=4000).astype(np.float32)
    # power-of-two scales: the product is exact, so the code is the plain encoding of x / s
    for s in (1.0, 0.25, 4.0):
        assert np.array_equal(quantize(x, s), e4m3_encode(x.astype(np.float64) / s))
    # a scale whose reciprocal is inexact: the fp32 product decides
    s = 3.0
    y = (x * (np.float32(1) / np.float32(s))).astype(np.float64)
    assert np.array_equal(quantize(x, s), e4m3_encode(y))
    # error bound of the format: half a step, 2^-4 of the magnitude in the normal range
    d = dequantize(quantize(x, s), s)
    normal = np.abs(x / s) >= 2.0 ** -6
    assert np.all(np.abs(d - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4 * (1 + 1e-6))


def test_attention_over_one_key_returns_the_decoded_value_row():
    rng = np.random.default_rng(13)
    H, D, n = 2, 16, 5
    q = rng.normal(size=(n, H, D))
    kc = rng.integers(0, 256, size=(n, H, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(n, H, D)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38
    vc[(vc & 0x7F) == 0x7F] = 0x38
    seqs = [(i, 1, i, 0, BIDIR) for i in range(n)]
    out, lse = attn_mixed_fp8(seqs, -1, q, kc, vc, 0.5, 2.0, H, H)
    assert np.array_equal(out, e4m3_decode(vc) * 2.0)
    want_lse = np.einsum("nhd,nhd->nh", q, e4m3_decode(kc) * 0.5) / np.sqrt(D)
    assert np.allclose(lse, want_lse, rtol=1e-12, atol=1e-12)


def test_k_scale_moves_into_the_queries():
    rng = np.random.default_rng(14)
    Hq, Hkv, D = 4, 2, 32
    seqs = [(0, 20, 0, 30, CAUSAL), (20, 12, 50, 10, BIDIR)]
    q = rng.normal(size=(32, Hq, D))
    kc = e4m3_encode(rng.normal(size=(72, Hkv, D)))
    vc = e4m3_encode(rng.normal(size=(72, Hkv, D)))
    a, la = attn_mixed_fp8(seqs, 7, q, kc, vc, 0.125, 1.0, Hq, Hkv)
    b, lb = attn_mixed(seqs, 7, q * 0.125, e4m3_decode(kc), e4m3_decode(vc), Hq, Hkv)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14) and np.allclose(la, lb, rtol=1e-12, atol=1e-12)
    # v_scale scales the output and leaves lse alone
    c, lc = attn_mixed_fp8(seqs, 7, q, kc, vc, 0.125, 8.0, Hq, Hkv)
    assert np.allclose(c, 8.0 * a, rtol=1e-12, atol=1e-14) and np.array_equal(lc, la)


def test_paged_fp8_equals_contiguous_fp8_on_gathered_rows():
    rng = np.random.default_rng(15)
    B, H, D = 4, 1, 8
    kc = e4m3_encode(rng.normal(size=(6 * B, H, D)))
    vc = e4m3_encode(rng.normal(size=(6 * B, H, D)))
    table = np.array([3, 0, 5], np.int32)
    rows = np.concatenate([np.arange(b * B, b * B + B) for b in table])[:11]
    q = rng.normal(size=(3, H, D))
    got, _ = attn_mixed_paged_fp8([(0, 3, 0, 8, CAUSAL)], -1, q, kc, vc, 0.5, 0.5, table, B, H, H)
    want, _ = attn_mixed_fp8([(0, 3, 0, 8, CAUSAL)], -1, q, kc[rows], vc[rows], 0.5, 0.5, H, H)
    assert np.array_equal(got, want)


def test_kv_write_fp8_stores_codes_within_the_format_bound():
    rng = np.random.default_rng(16)
    B, H, D = 4, 2, 8
    kp = np.zeros((8 * B, H, D), np.uint8)
    vp = np.zeros_like(kp)
    kn, vn = rng.normal(size=(6, H, D)).astype(np.float32), rng.normal(size=(6, H, D)).astype(np.float32)
    table = np.array([7, 2, 4], np.int32)
    k2, v2 = kv_write_fp8(kp, vp, kn, vn, [(0, 6, 0, 3)], table, B, 0.5, 0.25)
    for i in range(6):
        p = 3 + i
        r = table[p // B] * B + p % B
        assert np.array_equal(k2[r], quantize(kn[i], 0.5)) and np.array_equal(v2[r], quantize(vn[i], 0.25))
    written = {table[(3 + i) // B] * B + (3 + i) % B for i in range(6)}
    untouched = [r for r in range(8 * B) if r not in written]
    assert not k2[untouched].any() and not v2[untouched].any()

"""Oracle: an FP8 (OCP E4M3) K/V cache under the mixed-mode attention (float64).

Test infrastructure only (see the package docstring).

What is computed, and where it is stated:
  * the measured model runs in FP8 - [P1] section "성능 및 양자화" and [P3] section
    "Izmjerene performanse" (FP8 quantization with dynamic activations);
  * the element format is E4M3 of the Open Compute Project's 8-bit floating point
    specification (OFP8): a sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent 0 holds the subnormals (m/8) * 2^-6; exponent 15 with mantissa 7 is NaN
    and there are no infinities, so the largest finite magnitude is 448.

Readings taken where the pages leave the variant open:
  * only the K/V cache is stored in FP8; queries, outputs and arithmetic keep the
    call's dtype;
  * one fp32 scale per tensor (k_scale for K, v_scale for V): the stored value is
    code * scale;
  * quantizing x: y = float32(x) * float32(1 / scale) (the reciprocal rounded to fp32
    once), clamped to [-448, 448], then rounded to the nearest E4M3 value, ties to the
    even code (the code whose mantissa bit 0 is clear). NaN stays NaN.
Attention over an FP8 cache is, by definition, the attention of oracle.attn over the
decoded values times the scales.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .attn import attn_mixed
from .kvcache import attn_mixed_paged, kv_write

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The value of one E4M3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# the non-negative finite codes 0..126 in increasing value
_POS = _TABLE[:127]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Values -> E4M3 codes: clamp to +-448, nearest value, ties to the even code.
    Zero keeps its sign; NaN gives 0x7F (or 0xFF with the sign bit)."""
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    nan = np.isnan(y)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)
    # the two codes around a (values _POS[lo] < a <= _POS[hi]), then the nearer one
    hi = np.searchsorted(_POS, a, side="left")  # first code with value >= a; <= 126
    lo = np.maximum(hi - 1, 0)
    dl, dh = a - _POS[lo], _POS[hi] - a
    nearest = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    c = np.where(_POS[hi] == a, hi, nearest)
    c = np.where(nan, 0x7F, c)
    return (c | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Values (bf16 or fp32 inputs, exact in fp32) -> E4M3 codes at a per-tensor scale,
    the fp32 product by the fp32 reciprocal deciding the code."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float32) * inv  # one fp32 rounding
    return e4m3_encode(y.astype(np.float64))


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes -> float64 values times the scale."""
    return e4m3_decode(codes) * float(np.float32(scale))


def attn_mixed_fp8(seqs: Sequence, window: int, q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray,
                   k_scale: float, v_scale: float, num_q_heads: int, num_kv_heads: int,
                   scale: Optional[float] = None, rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Mixed-mode attention with K and V given as E4M3 codes and per-tensor scales."""
    return attn_mixed(seqs, window, q, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), num_q_heads,
                      num_kv_heads, scale, rows)


def attn_mixed_paged_fp8(seqs: Sequence, window: int, q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray,
                         k_scale: float, v_scale: float, table: np.ndarray, block_size: int, num_q_heads: int,
                         num_kv_heads: int, scale: Optional[float] = None, rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """The same over paged pools of codes."""
    return attn_mixed_paged(seqs, window, q, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), table,
                            block_size, num_q_heads, num_kv_heads, scale, rows)


def kv_write_fp8(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, seqs: Sequence,
                 table: np.ndarray, block_size: int, k_scale: float, v_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """New rows quantized, then written into pools of codes as oracle.kvcache.kv_write does."""
    return kv_write(k_pool, v_pool, quantize(k_new, k_scale), quantize(v_new, v_scale), seqs, table, block_size)

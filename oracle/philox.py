"""Oracle: Philox4x64-10 counter-based generator, in plain Python integers.

Test infrastructure only (see the package docstring).

The pages say candidate tokens are drawn at every canvas position and that
positions whose confidence is low are swapped for random tokens ([P1] section
"샘플링 루프와 엔트로피 경계 디노이징"; [P2] section "Diffusion에 스도쿠가 흥미로운
이유", re-noising). They name no generator. Both sides of the build implement
Philox4x64 with 10 rounds as published by Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), each from that definition:

  one round maps the counter (x0, x1, x2, x3) under key (k0, k1) to
      (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))
  with M0 = 0xD2E7470EE14C6C93, M1 = 0xCA5A826395121157; between rounds the key
  is bumped by the Weyl constants (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B).

Draw layout (a reading; the pages are silent): key = (seed, 0), counter =
(step, position, stream, 0). Stream 0 gives the candidate uniform, stream 1 the
re-noise token, stream 2 the initial canvas token.
"""
from __future__ import annotations

from typing import Tuple

MASK64 = (1 << 64) - 1
M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B

STREAM_CANDIDATE, STREAM_RENOISE, STREAM_INIT = 0, 1, 2


def philox4x64_10(counter: Tuple[int, int, int, int], key: Tuple[int, int]) -> Tuple[int, int, int, int]:
    x0, x1, x2, x3 = (c & MASK64 for c in counter)
    k0, k1 = (k & MASK64 for k in key)
    for r in range(10):
        if r > 0:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        p0 = M0 * x0          # exact 128-bit products
        p1 = M1 * x2
        x0, x1, x2, x3 = ((p1 >> 64) ^ x1 ^ k0, p1 & MASK64, (p0 >> 64) ^ x3 ^ k1, p0 & MASK64)
    return x0, x1, x2, x3


def _word0(seed: int, step: int, position: int, stream: int) -> int:
    return philox4x64_10((step, position, stream, 0), (seed, 0))[0]


def uniform24(seed: int, step: int, position: int) -> float:
    """u in [0, 1) with 24 random bits: the top 24 bits of word 0 times 2^-24
    (exact in float32 and float64)."""
    return (_word0(seed, step, position, STREAM_CANDIDATE) >> 40) * 2.0 ** -24


def renoise_token(seed: int, step: int, position: int, vocab: int, stream: int = STREAM_RENOISE) -> int:
    """Uniform token in [0, vocab): top 32 bits of word 0 scaled by vocab, integer-exact."""
    return ((_word0(seed, step, position, stream) >> 32) * vocab) >> 32

"""Seeded synthetic inputs for the block-diffusion denoising step.

This module only draws numbers: it holds none of the step's arithmetic
(no attention, softmax, entropy, acceptance or embedding average). Both the
CPU oracle's tests and the GPU path's tests/bench take their inputs from here,
so that the two sides see the same values while sharing no compute code.

Recipe (the same for every tensor):
  * generator  numpy.random.Generator(PCG64(seed)), seed = 214000 + 100*cfg + tensor_id
    with tensor ids Q=1, K=2, V=3, z=4, sigma=5, E=6, driver-pool=7, request-seeds=8;
  * large tensors are drawn in chunks of CHUNK elements (flat, row-major), chunk j
    from PCG64(seed).jumped(j), so chunks can be drawn on several threads and any
    chunk can be redrawn alone;
  * values are drawn as float32; for bf16 workloads they are rounded to bf16 with
    round-to-nearest-even and kept as float32 arrays holding bf16-representable values;
  * logits follow l[i, v] = sigma_i * z[i, v], z ~ N(0, 1), ln sigma_i ~ U(ln 0.1, ln 10),
    which spreads per-row entropies from near 0 to near ln V.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os as _os
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

CHUNK = 1 << 22
SEED_BASE = 214000
TID_Q, TID_K, TID_V, TID_Z, TID_SIGMA, TID_E, TID_POOL, TID_REQSEED = 1, 2, 3, 4, 5, 6, 7, 8

CAUSAL, BIDIR = 0, 1


def seed_for(cfg: int, tensor_id: int) -> int:
    return SEED_BASE + 100 * cfg + tensor_id


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(_os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = _os.cpu_count() or 1
    return max(1, min(16, n))


def normal(seed: int, shape, std: float = 1.0, bf16: bool = False) -> np.ndarray:
    """N(0, std^2) float32 draws, chunked as the module docstring states."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(j: int) -> None:
        lo, hi = j * CHUNK, min(n, (j + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(seed).jumped(j))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)
        if bf16:
            out[lo:hi] = round_to_bf16(out[lo:hi])

    if nchunks == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def sigmas(seed: int, rows: int) -> np.ndarray:
    """Per-row scales with ln sigma ~ U(ln 0.1, ln 10), float32."""
    g = np.random.Generator(np.random.PCG64(seed))
    return np.exp(g.uniform(np.log(0.1), np.log(10.0), size=rows)).astype(np.float32)


def logits(cfg: int, rows: int, vocab: int, bf16: bool, tid_z: int = TID_Z,
           tid_sigma: int = TID_SIGMA) -> np.ndarray:
    """Rows of sigma_i * z[i, :] (float32, optionally rounded to bf16)."""
    z = normal(seed_for(cfg, tid_z), (rows, vocab))
    s = sigmas(seed_for(cfg, tid_sigma), rows)
    z *= s[:, None]
    if bf16:
        z = round_to_bf16(z)
    return z


def request_seeds(cfg: int, n: int) -> List[int]:
    g = np.random.Generator(np.random.PCG64(seed_for(cfg, TID_REQSEED)))
    return [int(x) for x in g.integers(0, 2**63 - 1, size=n, dtype=np.int64)]


@dataclass
class Seq:
    """One request of an attention call: q rows [q_start, q_start+num_q) of Q and
    key rows [kv_start, kv_start+prefix_len+num_q) of K/V, the first prefix_len
    being the committed cache and the rest this call's tokens."""
    q_start: int
    num_q: int
    kv_start: int
    prefix_len: int
    mode: int


@dataclass
class AttnCase:
    name: str
    seqs: List[Seq]
    window: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    bf16: bool
    cfg: int

    @property
    def total_q(self) -> int:
        return sum(s.num_q for s in self.seqs)

    @property
    def total_kv(self) -> int:
        return sum(s.prefix_len + s.num_q for s in self.seqs)

    def with_window(self, window: int, name: Optional[str] = None) -> "AttnCase":
        return AttnCase(name or self.name, self.seqs, window, self.num_q_heads,
                        self.num_kv_heads, self.head_dim, self.bf16, self.cfg)

    def with_mode(self, mode: int, name: Optional[str] = None) -> "AttnCase":
        seqs = [Seq(s.q_start, s.num_q, s.kv_start, s.prefix_len, mode) for s in self.seqs]
        return AttnCase(name or self.name, seqs, self.window, self.num_q_heads,
                        self.num_kv_heads, self.head_dim, self.bf16, self.cfg)

    def tensors(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        q = normal(seed_for(self.cfg, TID_Q), (self.total_q, self.num_q_heads, self.head_dim), bf16=self.bf16)
        k = normal(seed_for(self.cfg, TID_K), (self.total_kv, self.num_kv_heads, self.head_dim), bf16=self.bf16)
        v = normal(seed_for(self.cfg, TID_V), (self.total_kv, self.num_kv_heads, self.head_dim), bf16=self.bf16)
        return q, k, v


def pack_seqs(spec: List[Tuple[int, int, int]]) -> List[Seq]:
    """spec = [(prefix_len, num_q, mode), ...] -> back-to-back packed requests."""
    seqs, qs, ks = [], 0, 0
    for p, n, m in spec:
        seqs.append(Seq(qs, n, ks, p, m))
        qs += n
        ks += p + n
    return seqs


# ---- the five workloads ---------------------------------------------------------------

def attn_case(cfg: int) -> AttnCase:
    if cfg == 1:
        return AttnCase("fp32 canvas 256 prefix 256 W=32", pack_seqs([(256, 256, BIDIR)]), 32, 4, 4, 64, False, 1)
    if cfg == 2:
        return AttnCase("bf16 canvas 256 prefix 4096 global", pack_seqs([(4096, 256, BIDIR)]), -1, 16, 8, 256, True, 2)
    if cfg == 3:
        return AttnCase("bf16 canvas 256 prefix 32768 W=512", pack_seqs([(32768, 256, BIDIR)]), 512, 16, 8, 256, True, 3)
    if cfg == 4:
        return AttnCase("bf16 mixed 4-request batch",
                        pack_seqs([(0, 2048, CAUSAL), (8192, 256, CAUSAL), (1024, 256, BIDIR), (16384, 256, BIDIR)]),
                        -1, 16, 8, 256, True, 4)
    if cfg == 5:
        return AttnCase("bf16 prefixes 262144/131072/65536/4096",
                        pack_seqs([(262144, 256, BIDIR), (131072, 256, BIDIR), (65536, 256, BIDIR), (4096, 256, BIDIR)]),
                        -1, 16, 8, 256, True, 5)
    raise ValueError(cfg)


@dataclass
class SamplerCase:
    cfg: int
    vocab: int
    bf16: bool
    budget: float
    # rows per request (each request is one canvas of `rows` positions)
    canvases: List[int] = field(default_factory=lambda: [256])
    embed_dim: int = 0

    @property
    def total_rows(self) -> int:
        return sum(self.canvases)


def sampler_case(cfg: int) -> SamplerCase:
    if cfg == 1:
        return SamplerCase(1, 4096, False, 64.0, [256], 256)
    if cfg == 2:
        return SamplerCase(2, 262144, True, 128.0, [256], 2048)
    if cfg == 4:
        return SamplerCase(4, 262144, True, 128.0, [256, 256], 0)
    if cfg == 5:
        return SamplerCase(5, 262144, True, 128.0, [256, 256, 256, 256], 2048)
    raise ValueError(cfg)


def embed_table(cfg: int, vocab: int, dim: int, bf16: bool) -> np.ndarray:
    """Token-embedding table E [vocab, dim] ~ N(0, 0.02^2)."""
    return normal(seed_for(cfg, TID_E), (vocab, dim), std=0.02, bf16=bf16)


# ---- the 48-step denoise-loop driver (stands in for the model's logits) ---------------

POOL_ROWS = 512


def driver_pool(vocab: int, bf16: bool = True, cfg: int = 2) -> np.ndarray:
    """512 sigma-scaled logits rows: rows [0, 256) are each position's settled
    prediction, rows [256, 512) are noise rows used before a position settles."""
    return logits(cfg, POOL_ROWS, vocab, bf16, tid_z=TID_POOL, tid_sigma=TID_SIGMA)


def driver_rows(step: int, canvas: int = 256) -> np.ndarray:
    """Pool row used by each canvas position at a step: position i has settled once
    i < 32*step; before that it reads noise row 256 + (i + 37*step) mod 256."""
    i = np.arange(canvas)
    settled = i < min(canvas, 32 * step)
    return np.where(settled, i, 256 + (i + 37 * step) % 256).astype(np.int64)

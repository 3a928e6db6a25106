"""Oracle: a paged K/V cache (block tables) under the mixed-mode attention (float64).

Test infrastructure only (see the package docstring).

What is computed, and where the pages state it:
  * a request's keys are its committed cache followed by the tokens of this call;
    a block that has converged is committed to the cache and the next canvas starts
    after it, while the canvas itself is redrafted at every denoise step - [P1]
    sections "샘플링 루프와 엔트로피 경계 디노이징" and "ModelState 인터페이스";
  * the cache keeps vLLM's paged layout - [P3] section "Integracija u vLLM
    infrastrukturu" (the model runs inside vLLM's serving stack and its cache).

Reading taken where the pages leave the layout open: the plain block-table layout.
Pools hold blocks of B rows; key position j of a request lives at pool row
table[start + j // B] * B + j % B, where `start` is the request's first entry in a
flat int32 table. Attention over a paged cache is, by definition, the attention of
oracle.attn over the same key rows gathered into request order.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .attn import attn_mixed, _seq_fields


def pool_row(table: np.ndarray, start: int, j: int, block_size: int) -> int:
    """Pool row of key position j of the request whose table starts at `start`."""
    return int(table[start + j // block_size]) * block_size + j % block_size


def gather_rows(pool: np.ndarray, table: np.ndarray, start: int, n: int, block_size: int) -> np.ndarray:
    """Rows of key positions 0..n-1 of one request, in key order."""
    idx = [pool_row(table, start, j, block_size) for j in range(n)]
    return pool[idx]


def attn_mixed_paged(seqs: Sequence, window: int, q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     table: np.ndarray, block_size: int, num_q_heads: int, num_kv_heads: int,
                     scale: Optional[float] = None, rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Mixed-mode attention with each request's keys read through its block table.

    seqs as for oracle.attn.attn_mixed, except that kv_start is the index of the
    request's first table entry. Each request's prefix_len + num_q key rows are
    gathered in key order, then attn_mixed runs on the gathered, contiguous keys.
    """
    ks, vs, flat = [], [], []
    base = 0
    for s in seqs:
        q_start, num_q, kv_start, prefix_len, mode = _seq_fields(s)
        n = prefix_len + num_q
        ks.append(gather_rows(k_pool, table, kv_start, n, block_size))
        vs.append(gather_rows(v_pool, table, kv_start, n, block_size))
        flat.append((q_start, num_q, base, prefix_len, mode))
        base += n
    k = np.concatenate(ks, axis=0) if ks else k_pool[:0]
    v = np.concatenate(vs, axis=0) if vs else v_pool[:0]
    return attn_mixed(flat, window, q, k, v, num_q_heads, num_kv_heads, scale, rows)


def kv_write(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, seqs: Sequence,
             table: np.ndarray, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """New rows into paged pools; returns updated copies of the pools.

    seqs: (src_start, num, table_start, pos) per request. Row src_start + i goes to key
    position pos + i of the request. A table entry outside the pool writes nothing.
    """
    kp, vp = k_pool.copy(), v_pool.copy()
    blocks = k_pool.shape[0] // block_size
    for src_start, num, table_start, pos in seqs:
        for i in range(num):
            p = pos + i
            e = int(table[table_start + p // block_size])
            if e < 0 or e >= blocks:
                continue
            r = e * block_size + p % block_size
            kp[r] = k_new[src_start + i]
            vp[r] = v_new[src_start + i]
    return kp, vp

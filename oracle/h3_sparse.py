"""Plain CPU oracle of block-sparse tile attention (float64).

TEST INFRASTRUCTURE ONLY, like ``h3_block``: only the tests, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP kernels or their host library.

Video sparse attention selects, for every query tile of T rows and every head,
a set of key tiles of T rows and attends only to the keys inside them (tiles of
64 or 128 rows with head dimension 128; only the selected key blocks and their
valid rows are visited; prefix queries stay dense): FastH3 OmniRef (Ref2VA) on
Apple Silicon MLX, "Opt-in M5 attention backend".  The trained selection is not
on the pages; here it is an input:

    for head h and query tile i:  keys(h, i) = union over j in sel(h, i) of rows
                                  [j*T, min((j+1)*T, n))
    o[h, r] = softmax over keys(h, i) of (q[h, r] . k[h, key] / sqrt(d)) v[h, key]
              for every row r of tile i

sel(h, i) is given in CSR form: tile_idx[tile_off[h*nq + i] : tile_off[h*nq + i + 1]],
nq = ceil(n / T).  The order inside a list does not matter; lists hold no
duplicates.  An empty list gives zeros.
"""
from __future__ import annotations

import math

import numpy as np


def selected_keys(tile_off, tile_idx, h: int, i: int, nq: int, tile: int, n: int) -> np.ndarray:
    """Sorted key rows selected for head h, query tile i."""
    sel = np.asarray(tile_idx)[tile_off[h * nq + i]:tile_off[h * nq + i + 1]]
    rows = [np.arange(j * tile, min((j + 1) * tile, n)) for j in sorted(int(s) for s in sel)]
    return np.concatenate(rows) if rows else np.zeros(0, np.int64)


def attention_sparse(q, k, v, tile: int, tile_off, tile_idx) -> np.ndarray:
    """q, k, v [H, N, d] -> o [H, N, d]: each query tile over its selected key tiles."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    H, N, d = q.shape
    nq = -(-N // tile)
    out = np.zeros((H, N, d))
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        for i in range(nq):
            keys = selected_keys(tile_off, tile_idx, h, i, nq, tile, N)
            if len(keys) == 0:
                continue
            r = slice(i * tile, min((i + 1) * tile, N))
            s = (q[h, r] @ k[h, keys].T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[h, r] = p @ v[h, keys]
    return out

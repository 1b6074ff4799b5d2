"""Pins of the block-sparse attention oracle.

Selecting every tile must give full attention; any selection must equal
torch's scaled-dot-product attention with the equivalent boolean key mask
(float64); a 128-row tile is the union of its two 64-row halves; selecting only
the own tile gives per-tile dense attention; the list order is irrelevant and
an empty list gives zeros.  Ragged row counts (n not a multiple of the tile)
are covered throughout.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from joint_video_audio_h3_amd import synth


def _qkv(H, N, d, seed=0):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((H, N, d)) for _ in range(3))


def _csr(lists):
    off = np.cumsum([0] + [len(l) for l in lists]).astype(np.int32)
    idx = np.concatenate([np.asarray(l, np.int32) for l in lists]) if any(len(l) for l in lists) else np.zeros(0, np.int32)
    return off, idx


@pytest.mark.parametrize("tile,N", [(64, 200), (128, 300), (64, 64)])
def test_all_tiles_equal_full_attention(tile, N):
    H, d = 2, 16
    q, k, v = _qkv(H, N, d, 1)
    nq = -(-N // tile)
    off, idx = _csr([list(range(nq))] * (H * nq))
    np.testing.assert_allclose(oracle.attention_sparse(q, k, v, tile, off, idx),
                               oracle.attention(q, k, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tile,N,keep", [(64, 333, 0.3), (128, 700, 0.25)])
def test_matches_torch_sdpa_with_key_mask(tile, N, keep):
    H, d = 3, 32
    q, k, v = _qkv(H, N, d, 2)
    off, idx = synth.make_tile_mask(N, H, tile, keep, dense_rows=70, seed=3)
    got = oracle.attention_sparse(q, k, v, tile, off, idx)
    nq = -(-N // tile)
    mask = np.zeros((H, N, N), bool)
    for h in range(H):
        for i in range(nq):
            keys = oracle.selected_keys(off, idx, h, i, nq, tile, N)
            mask[h, i * tile:(i + 1) * tile, keys] = True
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None],
                                         attn_mask=torch.from_numpy(mask)[None])[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_tile_128_is_union_of_its_64_halves():
    H, N, d = 2, 450, 8
    q, k, v = _qkv(H, N, d, 4)
    off, idx = synth.make_tile_mask(N, H, 128, 0.4, seed=5)
    nq = -(-N // 128)
    halves = []
    for h in range(H):
        for i in range(nq):
            sel = idx[off[h * nq + i]:off[h * nq + i + 1]]
            half = [jj for j in sel for jj in (2 * j, 2 * j + 1) if jj * 64 < N]
            halves += [half, half]          # both 64-row query halves of tile i
    nq64 = -(-N // 64)
    lists = []
    for h in range(H):
        lists += halves[h * 2 * nq: h * 2 * nq + nq64]
    off64, idx64 = _csr(lists)
    np.testing.assert_allclose(oracle.attention_sparse(q, k, v, 64, off64, idx64),
                               oracle.attention_sparse(q, k, v, 128, off, idx), rtol=1e-12, atol=1e-12)


def test_own_tile_only_is_per_tile_attention_and_order_and_empty():
    H, N, d, T = 2, 150, 8, 64
    q, k, v = _qkv(H, N, d, 6)
    nq = -(-N // T)
    off, idx = _csr([[i] for _ in range(H) for i in range(nq)])
    got = oracle.attention_sparse(q, k, v, T, off, idx)
    for i in range(nq):
        r = slice(i * T, min((i + 1) * T, N))
        np.testing.assert_allclose(got[:, r], oracle.attention(q[:, r], k[:, r], v[:, r]), rtol=1e-12)
    lists = [[2, 0], [1], []] * H
    off2, idx2 = _csr(lists)
    off3, idx3 = _csr([sorted(l) for l in lists])
    a2 = oracle.attention_sparse(q, k, v, T, off2, idx2)
    np.testing.assert_allclose(a2, oracle.attention_sparse(q, k, v, T, off3, idx3), rtol=1e-13)
    assert np.all(a2[:, 128:] == 0)           # empty list: zeros


def test_generator_mask_shape():
    N, H, T = 49840, 2, 128
    off, idx = synth.make_tile_mask(N, H, T, 0.125, dense_rows=1280, seed=0)
    nq = -(-N // T)
    counts = np.diff(off)
    assert off[0] == 0 and len(off) == H * nq + 1 and off[-1] == len(idx)
    assert np.all(counts[:10] == nq) and np.all(counts[nq:nq + 10] == nq)       # dense prefix queries
    assert np.all(counts[10:nq] == int(np.ceil(0.125 * nq)))
    for h in range(H):
        for i in (10, 200, nq - 1):
            sel = idx[off[h * nq + i]:off[h * nq + i + 1]]
            assert np.all(np.diff(sel) > 0) and set(range(10)) <= set(sel.tolist()) and i in sel


def test_block_with_every_tile_selected_equals_dense_block():
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    x, tags, pos, table, blocks = synth.make_inputs(wl, seed=7, n_blocks=1)
    nq = -(-wl.n_rows // 64)
    off, idx = synth.make_tile_mask(wl.n_rows, wl.dims.heads, 64, 1.0, seed=1)
    assert len(idx) == wl.dims.heads * nq * nq
    dense = oracle.block_forward(x, tags, pos, table[0], blocks[0], wl.dims)
    sparse = oracle.block_forward(x, tags, pos, table[0], blocks[0], wl.dims, sparse=(64, off, idx))
    np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-12)

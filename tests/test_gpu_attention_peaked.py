"""Attention on sharply peaked softmax rows, dense and block-sparse (GPU).

The flash kernels keep one reference maximum per query and rescale the output
and the running sum only when a half-tile's probabilities grow too large.
These inputs drive that path hard (``synth.make_peaked_qkv``): scores span tens
of log2 units, for most queries the running maximum keeps rising tile after
tile up to the last, partial tile, one query per head has every score of its
first tile at -160 (its maximum is the last key), and another has its maximum
in the first tile with every later score far below it.  Sizes: N = 300 and
1,192 (the ragged last tile masked), both head widths, both sparse tile sizes,
and the N = 49,840 geometry on sampled rows against the float64 oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import TOL_ATTN, dev, host_bf16, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


def _device(q, k, v, n):
    H, _, d = q.shape
    np_ = lib.padded_rows(n)
    pad = lambda a: np.concatenate([a, np.zeros((H, np_ - n, d), np.uint16)], axis=1)  # noqa: E731
    return dev(pad(q)), dev(pad(k)), dev(np.ascontiguousarray(pad(v).transpose(0, 2, 1)))


def _unscaled(q, d):
    """The oracle takes q before the kernels' log2(e)/sqrt(d) pre-scale."""
    return oracle.bf16_to_f64(q) / (np.log2(np.e) / np.sqrt(d))


CASES = [("tiny", synth.TINY_DIMS, 300), ("h3", synth.H3_DIMS, 300), ("h3", synth.H3_DIMS, 1192)]


@pytest.mark.parametrize("name,dims,n", CASES, ids=[f"{c[0]}-N{c[2]}" for c in CASES])
def test_dense_attention_peaked(name, dims, n):
    say("peaked attention dense", name, n)
    d = dims.head_dim
    q, k, v = synth.make_peaked_qkv(dims.heads, n, d, seed=31)
    qd, kd, vtd = _device(q, k, v, n)
    o = torch.full((n, dims.inner), 0x7FC0, dtype=torch.int16, device="cuda")
    lib.attention(dims, qd, kd, vtd, n, o)
    torch.cuda.synchronize()
    got = host_bf16(o)
    assert np.isfinite(got).all()
    ref = oracle.merge_heads(oracle.attention(_unscaled(q, d), oracle.bf16_to_f64(k), oracle.bf16_to_f64(v)))
    assert rel_l2(got, ref) < TOL_ATTN
    for h in range(dims.heads):
        assert rel_l2(got[:, h * d:(h + 1) * d], ref[:, h * d:(h + 1) * d]) < 2 * TOL_ATTN, h
    # the two extreme queries (row 0: first-tile scores at -160, maximum at the
    # last key; row 1: maximum in the first tile), each on its own
    for r in (0, 1):
        assert rel_l2(got[r], ref[r]) < 2 * TOL_ATTN, r


SPARSE = [("tiny", synth.TINY_DIMS, 300, 64), ("tiny", synth.TINY_DIMS, 300, 128),
          ("h3", synth.H3_DIMS, 1192, 64), ("h3", synth.H3_DIMS, 1192, 128)]


@pytest.mark.parametrize("name,dims,n,tile", SPARSE, ids=[f"{c[0]}-N{c[2]}-T{c[3]}" for c in SPARSE])
def test_sparse_attention_peaked(name, dims, n, tile):
    say("peaked attention sparse", name, n, tile)
    d = dims.head_dim
    q, k, v = synth.make_peaked_qkv(dims.heads, n, d, seed=32)
    qd, kd, vtd = _device(q, k, v, n)
    # every list keeps the first tile (dense prefix keys) and the last, partial one
    off, idx = synth.make_tile_mask(n, dims.heads, tile, 0.5, dense_rows=64, seed=32)
    nq = -(-n // tile)
    lists = [sorted(set(idx[off[i]:off[i + 1]].tolist()) | {nq - 1}) for i in range(len(off) - 1)]
    off = np.cumsum([0] + [len(x) for x in lists]).astype(np.int32)
    idx = np.concatenate([np.asarray(x, np.int32) for x in lists])
    o = torch.full((n, dims.inner), 0x7FC0, dtype=torch.int16, device="cuda")
    lib.attention_sparse(dims, qd, kd, vtd, n, tile, dev(off), dev(idx), o)
    torch.cuda.synchronize()
    got = host_bf16(o)
    assert np.isfinite(got).all()
    ref = oracle.merge_heads(oracle.attention_sparse(_unscaled(q, d), oracle.bf16_to_f64(k),
                                                     oracle.bf16_to_f64(v), tile, off, idx))
    assert rel_l2(got, ref) < TOL_ATTN


def _big_case(seed):
    dims = dataclasses.replace(synth.H3_DIMS, heads=8)   # 8 heads: one per XCD, the remapped grid
    n, d = 49840, 128
    q, k, v = synth.make_peaked_qkv(dims.heads, n, d, seed=seed)
    return dims, n, d, q, k, v


def test_dense_attention_peaked_n49840_sampled():
    dims, n, d, q, k, v = _big_case(33)
    say("peaked attention dense", n)
    qd, kd, vtd = _device(q, k, v, n)
    o = torch.empty(n, dims.inner, dtype=torch.int16, device="cuda")
    lib.attention(dims, qd, kd, vtd, n, o)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 2, n - 1, n - 40],
                                     np.random.default_rng(33).integers(0, n, 14)]))
    got = host_bf16(o[torch.from_numpy(rows).cuda()])
    assert np.isfinite(got).all()
    for h in range(dims.heads):
        ref = oracle.attention(_unscaled(q[h:h + 1, rows], d), oracle.bf16_to_f64(k[h:h + 1]),
                               oracle.bf16_to_f64(v[h:h + 1]))[0]
        assert rel_l2(got[:, h * d:(h + 1) * d], ref) < TOL_ATTN, h


def test_sparse_attention_peaked_n49840_tile128_sampled():
    dims, n, d, q, k, v = _big_case(34)
    tile = 128
    say("peaked attention sparse", n, tile)
    qd, kd, vtd = _device(q, k, v, n)
    off, idx = synth.make_tile_mask(n, dims.heads, tile, 0.125, dense_rows=1280, seed=34)
    o = torch.empty(n, dims.inner, dtype=torch.int16, device="cuda")
    lib.attention_sparse(dims, qd, kd, vtd, n, tile, dev(off), dev(idx), o)
    torch.cuda.synchronize()
    nq = -(-n // tile)
    rng = np.random.default_rng(34)
    pairs = [(0, 0), (7, nq - 1), (3, 12)] + [(int(rng.integers(dims.heads)), int(rng.integers(nq))) for _ in range(5)]
    for h, i in pairs:
        rows = np.arange(i * tile, min((i + 1) * tile, n))
        keys = oracle.selected_keys(off, idx, h, i, nq, tile, n)
        ref = oracle.attention(_unscaled(q[h:h + 1, rows], d), oracle.bf16_to_f64(k[h:h + 1, keys]),
                               oracle.bf16_to_f64(v[h:h + 1, keys]))[0]
        got = host_bf16(o[torch.from_numpy(rows).cuda(), h * d:(h + 1) * d])
        assert np.isfinite(got).all()
        assert rel_l2(got, ref) < TOL_ATTN, (h, i)

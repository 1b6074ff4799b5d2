"""Parity of block-sparse tile attention against the float64 oracle (GPU).

Generator masks (fixed budget per query tile, dense prefix queries, prefix keys
kept) with both tile sizes, ragged row counts, shuffled lists, an empty list
and out-of-range indices; a selection of every tile in order must reproduce the
dense kernel bit for bit where the two share their per-wave arithmetic (head_dim
96), and agree with it to rounding at head_dim 128, where the dense kernel runs
48 queries per wave on 16 x 16 x 32 MFMAs; a 2-block sparse forward against the
oracle; and the
N = 49,840 geometry (56 heads, tile 128, an eighth of the key tiles) on sampled
(head, query tile) pairs.
"""
import numpy as np
import pytest
import torch

import oracle
from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import TOL_ATTN, TOL_DEPTH, dev, host_bf16, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


def _inputs(dims, n, seed):
    H, d = dims.heads, dims.head_dim
    np_ = lib.padded_rows(n)
    qs = np.log2(np.e) / np.sqrt(d)
    q = synth.make_activation_bf16(H * n, d, "q", seed, std=qs).reshape(H, n, d)
    k = synth.make_activation_bf16(H * n, d, "k", seed).reshape(H, n, d)
    v = synth.make_activation_bf16(H * n, d, "v", seed).reshape(H, n, d)
    pad = lambda a: np.concatenate([a, np.zeros((H, np_ - n, d), np.uint16)], axis=1)  # noqa: E731
    return q, k, v, dev(pad(q)), dev(pad(k)), dev(np.ascontiguousarray(pad(v).transpose(0, 2, 1)))


def _run(dims, n, tile, off, idx, qd, kd, vtd):
    o = torch.full((n, dims.inner), 0x7FC0, dtype=torch.int16, device="cuda")
    lib.attention_sparse(dims, qd, kd, vtd, n, tile, dev(off), dev(idx), o)
    torch.cuda.synchronize()
    return o


def _ref(dims, q, k, v, tile, off, idx):
    qs = np.log2(np.e) / np.sqrt(dims.head_dim)
    return oracle.merge_heads(oracle.attention_sparse(oracle.bf16_to_f64(q) / qs, oracle.bf16_to_f64(k),
                                                      oracle.bf16_to_f64(v), tile, off, idx))


CASES = [("tiny", synth.TINY_DIMS, 300, 64, 0.3), ("tiny", synth.TINY_DIMS, 333, 128, 0.4),
         ("tiny", synth.TINY_DIMS, 64, 64, 0.5), ("tiny", synth.TINY_DIMS, 40, 64, 1.0),
         ("h3", synth.H3_DIMS, 1, 128, 1.0), ("h3", synth.H3_DIMS, 777, 128, 0.25),
         ("h3", synth.H3_DIMS, 700, 64, 0.2)]


@pytest.mark.parametrize("name,dims,n,tile,keep", CASES, ids=[f"{c[0]}-N{c[2]}-T{c[3]}" for c in CASES])
def test_sparse_attention_matches_oracle(name, dims, n, tile, keep):
    say("sparse attention", name, n, tile, keep)
    q, k, v, qd, kd, vtd = _inputs(dims, n, seed=21)
    off, idx = synth.make_tile_mask(n, dims.heads, tile, keep, dense_rows=min(100, n), seed=21)
    # shuffle every list: the order must not matter
    r = np.random.default_rng(0)
    idx = idx.copy()
    for a, b in zip(off[:-1], off[1:]):
        idx[a:b] = r.permutation(idx[a:b])
    got = host_bf16(_run(dims, n, tile, off, idx, qd, kd, vtd))
    ref = _ref(dims, q, k, v, tile, off, idx)
    assert rel_l2(got, ref) < TOL_ATTN


def test_empty_and_out_of_range_lists():
    dims, n, tile = synth.TINY_DIMS, 200, 64
    say("sparse attention edge lists")
    q, k, v, qd, kd, vtd = _inputs(dims, n, seed=22)
    nq = -(-n // tile)
    lists = [[] if (h, i) == (0, 1) else ([i, nq + 5] if (h, i) == (1, 2) else sorted({0, i}))
             for h in range(dims.heads) for i in range(nq)]
    off = np.cumsum([0] + [len(x) for x in lists]).astype(np.int32)
    idx = np.concatenate([np.asarray(x, np.int32) for x in lists])
    got = host_bf16(_run(dims, n, tile, off, idx, qd, kd, vtd))
    assert np.all(got[64:128, :dims.head_dim] == 0)            # head 0, query tile 1: empty list
    clamped = [[min(j, nq - 1) for j in x] for x in lists]      # index nq + 5 reads the last tile
    off_c = off
    idx_c = np.concatenate([np.asarray(x, np.int32) for x in clamped])
    ref = _ref(dims, q, k, v, tile, off_c, idx_c)
    assert rel_l2(got, ref) < TOL_ATTN


@pytest.mark.parametrize("dims,n,tile", [(synth.TINY_DIMS, 300, 64), (synth.H3_DIMS, 1192, 128)],
                         ids=["tiny-T64", "h3-T128"])
def test_every_tile_in_order_equals_dense_kernel(dims, n, tile):
    say("sparse all tiles == dense", n, tile)
    q, k, v, qd, kd, vtd = _inputs(dims, n, seed=23)
    off, idx = synth.make_tile_mask(n, dims.heads, tile, 1.0, seed=23)
    got = _run(dims, n, tile, off, idx, qd, kd, vtd)
    dense = torch.empty_like(got)
    lib.attention(dims, qd, kd, vtd, n, dense)
    torch.cuda.synchronize()
    if dims.head_dim != 128:
        assert torch.equal(got, dense)
    else:   # same keys, same values, another summation order and probability rounding
        assert rel_l2(host_bf16(got), host_bf16(dense).astype(np.float64)) < TOL_ATTN


def test_sparse_forward_two_blocks_matches_oracle():
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    say("sparse forward", wl.name)
    x, tags, pos, table, blocks = synth.make_inputs(wl, seed=24)
    tile = 64
    nq = -(-wl.n_rows // tile)
    masks = [synth.make_tile_mask(wl.n_rows, wl.dims.heads, tile, 0.4, dense_rows=16, seed=30 + b)
             for b in range(2)]
    # one CSR offset array per block, indexing one shared index array
    offs, idxs, base = [], [], 0
    for off, idx in masks:
        offs.append(off + base)
        idxs.append(idx)
        base += len(idx)
    xd = dev(x)
    ws = lib.alloc_workspace(wl.dims, wl.n_rows)
    lib.dit_forward_sparse(wl.dims, xd, dev(tags), dev(pos), dev(table), [lib.to_device_block(b) for b in blocks],
                           tile, dev(np.concatenate(offs)), dev(np.concatenate(idxs)), ws)
    torch.cuda.synchronize()
    assert all(len(o) == wl.dims.heads * nq + 1 for o in offs)
    ref = oracle.dit_forward(x, tags, pos, table, lambda b: blocks[b], 2, wl.dims,
                             sparse_for_block=lambda b: (tile, masks[b][0], masks[b][1]))
    dense = oracle.dit_forward(x, tags, pos, table, lambda b: blocks[b], 2, wl.dims)
    got = xd.cpu().numpy().astype(np.float64)
    say("sparse forward rel-L2", rel_l2(got, ref), "vs dense", rel_l2(ref, dense))
    assert rel_l2(got, ref) < TOL_DEPTH
    assert rel_l2(got - x, ref - x) < 2 * TOL_DEPTH
    assert rel_l2(ref, dense) > 10 * rel_l2(got, ref)        # the selection matters


def test_fullsize_n49840_tile128_sampled():
    dims = synth.H3_DIMS
    n, tile = 49840, 128
    say("sparse fullsize", n)
    H, d = dims.heads, dims.head_dim
    np_ = lib.padded_rows(n)
    g = torch.Generator(device="cuda")
    g.manual_seed(25)
    qs = float(np.log2(np.e) / np.sqrt(d))
    qd = torch.zeros(H, np_, d, dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros_like(qd)
    vtd = torch.zeros(H, d, np_, dtype=torch.bfloat16, device="cuda")
    qd[:, :n] = (torch.randn(H, n, d, generator=g, device="cuda") * qs).to(torch.bfloat16)
    kd[:, :n] = torch.randn(H, n, d, generator=g, device="cuda").to(torch.bfloat16)
    vtd[:, :, :n] = torch.randn(H, d, n, generator=g, device="cuda").to(torch.bfloat16)
    off, idx = synth.make_tile_mask(n, H, tile, 0.125, dense_rows=1280, seed=25)
    o = torch.empty(n, H * d, dtype=torch.bfloat16, device="cuda")
    lib.attention_sparse(dims, qd, kd, vtd, n, tile, dev(off), dev(idx), o)
    torch.cuda.synchronize()
    nq = -(-n // tile)
    rng = np.random.default_rng(25)
    pairs = [(0, 0), (55, nq - 1), (7, 9), (13, 10)] + [(int(rng.integers(H)), int(rng.integers(nq))) for _ in range(6)]
    for h, i in pairs:
        rows = np.arange(i * tile, min((i + 1) * tile, n))
        keys = oracle.selected_keys(off, idx, h, i, nq, tile, n)
        qh = qd[h, rows].float().cpu().numpy().astype(np.float64) / qs
        kh = kd[h, keys].float().cpu().numpy().astype(np.float64)
        vh = vtd[h][:, keys].float().cpu().numpy().astype(np.float64).T
        ref = oracle.attention(qh[None], kh[None], vh[None])[0]
        got = o[rows, h * d:(h + 1) * d].float().cpu().numpy()
        assert rel_l2(got, ref) < TOL_ATTN, (h, i)

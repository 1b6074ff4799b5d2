"""INT8 group-32 weights on the two GEMM paths of the forward (GPU).

With the full workspace (h3_workspace_size) the forward dequantises each
linear's weights once into the workspace (RNE_bf16(q * s)) and runs the bf16
GEMM on them; with a workspace that lacks only that buffer it runs the kernel
that dequantises in LDS per row tile.  Both form the same bf16 weights
(RNE_bf16(q * s)), but through different GEMM kernels (other wave tiles, so
other MFMA operand roles and fp32 rounding inside the products): each must
match the oracle's INT8 forward within the depth bound, and the two must agree
with each other to the one-block bound.  Row counts: 1,192 (5 row tiles, the
last partial) and 8,449 (34 row tiles, the last holding one row), the latter
on sampled rows.  The dequantised weights themselves are pinned bit for bit:
the first path must reproduce the bf16 block run on the oracle's dequantised
weights exactly.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import TOL_BLOCK, TOL_DEPTH, dev, rel_l2, say

pytestmark = pytest.mark.gpu
INT8 = synth.WORKLOADS["h3_1blk_n1192_int8"].dims


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


def _min_workspace(dims, n, full):
    # the arena without the dequantisation buffer is the bf16 model's
    need = lib.workspace_size(dataclasses.replace(dims, wfmt=synth.WFMT_BF16), n)
    assert need < full.numel()
    return full[:need]


@pytest.mark.parametrize("n,nb", [(1192, 2), (8449, 1)])
def test_int8_forward_on_both_gemm_paths(n, nb):
    say("int8 forward, both GEMM paths:", n, "rows,", nb, "blocks")
    seed = 61
    x = synth.make_x(n, INT8, seed=seed)
    tags = synth.make_tags(n, INT8.n_tags, seed=seed)
    pos = synth.make_positions(n, seed=seed)
    table = synth.make_table(INT8, nb, seed=seed)
    host = [synth.make_block_weights(INT8, b, seed=seed) for b in range(nb)]
    blocks = [lib.to_device_block(h) for h in host]
    full = lib.alloc_workspace(INT8, n)
    xa, xb = dev(x), dev(x)
    lib.dit_forward(INT8, xa, dev(tags), dev(pos), dev(table), blocks, full)
    lib.dit_forward(INT8, xb, dev(tags), dev(pos), dev(table), blocks, _min_workspace(INT8, n, full))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(xa).all()) and bool(torch.isfinite(xb).all())
    got = xa.cpu().numpy().astype(np.float64)
    got_lds = xb.cpu().numpy().astype(np.float64)
    xd = x.astype(np.float64)
    say("int8 paths: rel-L2 between them", rel_l2(got, got_lds), "updates", rel_l2(got - xd, got_lds - xd))
    assert rel_l2(got - xd, got_lds - xd) < TOL_BLOCK
    if n <= 1192:
        ref = oracle.dit_forward(x, tags, pos, table, lambda b: host[b], nb, INT8)
    else:
        rows = np.unique(np.concatenate([np.random.default_rng(7).choice(n, 11, replace=False), [0, n - 1]]))
        ref = oracle.block_forward(x, tags, pos, table[0], host[0], INT8, q_rows=rows)
        xr = x[rows].astype(np.float64)
    for label, g in (("predequant", got), ("lds", got_lds)):
        if n <= 1192:
            say(f"int8 {label} rel-L2 x_out", rel_l2(g, ref), "update", rel_l2(g - xd, ref - xd))
            assert rel_l2(g, ref) < TOL_DEPTH and rel_l2(g - xd, ref - xd) < 2 * TOL_DEPTH
        else:
            say(f"int8 {label} sampled rel-L2 x_out", rel_l2(g[rows], ref), "update", rel_l2(g[rows] - xr, ref - xr))
            assert rel_l2(g[rows], ref) < TOL_BLOCK and rel_l2(g[rows] - xr, ref - xr) < 2 * TOL_BLOCK


def _bf16_block_from_oracle_dequant(host8):
    """The INT8 block's weights as bf16 bits, dequantised by the oracle
    (RNE_bf16(q * s), exact bf16 values, so their top 16 bits are the value)."""
    out = {}
    for k, v in host8.items():
        if k.startswith("w_"):
            wdq = oracle.dequant_int8_g32(v, host8["s_" + k[2:]])
            f = wdq.astype(np.float32)
            assert np.array_equal(f.astype(np.float64), wdq)
            bits = f.view(np.uint32)
            assert not (bits & 0xFFFF).any()
            out[k] = (bits >> 16).astype(np.uint16)
        elif k.startswith("s_"):
            out[k] = None
        else:
            out[k] = v
    return out


@pytest.fixture(scope="module")
def int8_and_dequantised_blocks():
    host8 = synth.make_block_weights(INT8, 0, seed=71)
    return lib.to_device_block(host8), lib.to_device_block(_bf16_block_from_oracle_dequant(host8))


@pytest.mark.parametrize("n", [300, 1192])
def test_predequant_block_is_the_bf16_block_on_oracle_dequantised_weights(n, int8_and_dequantised_blocks):
    """With the full workspace the INT8 block writes each linear's bf16 weights
    into the workspace and runs the bf16 GEMM on them, so it must equal, bit for
    bit, the bf16 block whose weights are the oracle's RNE_bf16(q * s) (a
    wrong element of any of the four dequantised matrices changes the fp32
    products of its output column in every row)."""
    say("int8 predequant block vs bf16 block on oracle-dequantised weights:", n, "rows")
    seed = 71
    bf16 = dataclasses.replace(INT8, wfmt=synth.WFMT_BF16)
    block8, block16 = int8_and_dequantised_blocks
    x = synth.make_x(n, INT8, seed=seed)
    tags = dev(synth.make_tags(n, INT8.n_tags, seed=seed))
    pos = dev(synth.make_positions(n, seed=seed))
    table = dev(synth.make_table(INT8, 1, seed=seed)[0])
    xa, xb = dev(x), dev(x)
    ws8 = lib.alloc_workspace(INT8, n)
    lib.dit_block_forward(INT8, xa, tags, pos, table, block8, ws8)
    ws16 = lib.alloc_workspace(bf16, n)
    lib.dit_block_forward(bf16, xb, tags, pos, table, block16, ws16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(xa).all())
    assert torch.equal(xa, xb)

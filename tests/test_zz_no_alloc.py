"""h3_dit_forward_noalloc: the forward on the library's static scratch array
(GPU), for callers that cannot allocate.

Through the C ABI it must give what h3_dit_forward gives with a caller
workspace on the same inputs (same kernels and launch shapes, so the same
bits), on two calls in a row, the second with fewer rows and blocks (the array
keeps the first call's contents); a forward whose workspace would not fit the
array is refused on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import TOL_DEPTH, dev, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


def _case(dims, n, nb, seed):
    x = synth.make_x(n, dims, seed=seed)
    tags = synth.make_tags(n, dims.n_tags, seed=seed)
    pos = synth.make_positions(n, seed=seed)
    table = synth.make_table(dims, nb, seed=seed)
    blocks = [lib.to_device_block(synth.make_block_weights(dims, b, seed=seed)) for b in range(nb)]
    return x, dev(tags), dev(pos), dev(table), blocks


def _both(dims, n, nb, seed):
    x, tags, pos, table, blocks = _case(dims, n, nb, seed)
    a = dev(x)
    lib.dit_forward_noalloc(dims, a, tags, pos, table, blocks)
    torch.cuda.synchronize()
    b = dev(x)
    ws = lib.alloc_workspace(dims, n)
    lib.dit_forward(dims, b, tags, pos, table, blocks, ws)
    torch.cuda.synchronize()
    return x, a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_forward_matches_workspace_forward_twice():
    dims = synth.H3_DIMS
    say("noalloc: H3 width, 2 blocks, N = 1,192")
    x, got, ref = _both(dims, 1192, 2, seed=81)
    assert np.isfinite(got).all()
    assert rel_l2(got, ref) < TOL_DEPTH
    np.testing.assert_array_equal(got, ref)
    assert np.abs(got - x).max() > 0.1
    say("noalloc: H3 width, 1 block, N = 300 (smaller, after the larger call)")
    x, got, ref = _both(dims, 300, 1, seed=82)
    assert rel_l2(got, ref) < TOL_DEPTH
    np.testing.assert_array_equal(got, ref)
    say("noalloc: tiny model, 2 blocks, N = 77")
    x, got, ref = _both(synth.TINY_DIMS, 77, 2, seed=83)
    np.testing.assert_array_equal(got, ref)


def test_noalloc_forward_refuses_a_workspace_beyond_the_array():
    dims = synth.H3_DIMS
    n = 1793                        # 2,048 padded rows: 140 MB of workspace
    assert lib.workspace_size(dims, n) > (128 << 20)
    say("noalloc: N =", n, "is refused on the host")
    L = lib.load()
    w = (lib.H3BlockWeights * 1)()
    st = L.h3_dit_forward_noalloc(ctypes.byref(lib.make_dims(dims)), 0x10000, 0x10000, 0x10000, 0x10000,
                                  w, 1, n, None)
    assert st == lib.H3_ERR_WORKSPACE
    assert "static scratch" in lib.last_error()

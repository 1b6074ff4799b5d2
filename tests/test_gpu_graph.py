"""The block stack under HIP graph capture (GPU).

The forward allocates nothing, records no memset and never synchronizes the
host (the optional tag check aside), so it can be captured into a graph
(torch.cuda.CUDAGraph, HIP graphs underneath).  Replays must reproduce the
eager forward bit for bit, again and again, with eager launches of the library
in between: for h3_dit_forward with a caller workspace, and for
h3_dit_forward_noalloc, whose scratch array is the point of capturing it.
"""
import os

import numpy as np
import pytest
import torch

from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    if os.environ.get("H3_CHECK") == "1":
        pytest.skip("the tag check synchronizes the host, which graph capture does not allow")
    lib.load()


def _inputs(dims, n, nb, seed):
    x = synth.make_x(n, dims, seed=seed)
    tags = dev(synth.make_tags(n, dims.n_tags, seed=seed))
    pos = dev(synth.make_positions(n, seed=seed))
    table = dev(synth.make_table(dims, nb, seed=seed))
    blocks = [lib.to_device_block(synth.make_block_weights(dims, b, seed=seed)) for b in range(nb)]
    return dev(x), tags, pos, table, blocks


@pytest.mark.parametrize("dims,noalloc", [(synth.H3_DIMS, False), (synth.H3_W8A8_DIMS, False),
                                          (synth.H3_DIMS, True)],
                         ids=["bf16", "w8a8-g896", "bf16-noalloc"])
def test_captured_forward_replays_bit_identical(dims, noalloc):
    n, nb = 1192, 2
    say("graph capture:", "W8A8" if dims.wfmt else "bf16", "noalloc" if noalloc else "workspace", n, nb)
    x0, tags, pos, table, blocks = _inputs(dims, n, nb, seed=91)
    ws = None if noalloc else lib.alloc_workspace(dims, n)

    def forward(x):
        if noalloc:
            lib.dit_forward_noalloc(dims, x, tags, pos, table, blocks)
        else:
            lib.dit_forward(dims, x, tags, pos, table, blocks, ws)

    ref = x0.clone()
    forward(ref)                        # eager (also settles the library's per-device setup)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ref).all()) and not torch.equal(ref, x0)

    xg = x0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward(xg)
    torch.cuda.synchronize()
    for rep in range(3):
        xg.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, ref), f"replay {rep}"
        # eager work of the library between replays (the same scratch or workspace)
        other = x0.clone()
        forward(other)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(other.cpu().numpy(), ref.cpu().numpy())
    del g

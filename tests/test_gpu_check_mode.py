"""The optional device-side tag check (H3_CHECK=1) of the calls that read
modality tags (GPU).

Without the flag, tags outside [0, n_tags) are the caller's error and are not
scanned.  With it, such a tag fails the call before anything is enqueued, so
x is left as it was; valid tags give the same bits as without the check.
"""
import numpy as np
import pytest
import torch

from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


@pytest.fixture(scope="module")
def case():
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    tags, pos = synth.packed_layout(wl)
    x = synth.make_x(wl, wl.dims, seed=71)
    table = synth.make_table(wl.dims, 1, seed=71)
    block = lib.to_device_block(synth.make_block_weights(wl.dims, 0, seed=71))
    ws = lib.alloc_workspace(wl.dims, wl.n_rows)
    return wl, tags, pos, x, table, block, ws


def _forward(case, tags):
    wl, _, pos, x, table, block, ws = case
    xd = dev(x)
    lib.dit_block_forward(wl.dims, xd, dev(tags), dev(pos), dev(table[0]), block, ws)
    torch.cuda.synchronize()
    return xd.cpu().numpy()


def test_check_mode_valid_tags_same_bits(case, monkeypatch):
    say("check mode: valid tags")
    ref = _forward(case, case[1])
    monkeypatch.setenv("H3_CHECK", "1")
    got = _forward(case, case[1])
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("bad", [3, -1])
def test_check_mode_rejects_out_of_range_tag(case, monkeypatch, bad):
    say("check mode: tag", bad)
    wl, tags, pos, x, table, block, ws = case
    monkeypatch.setenv("H3_CHECK", "1")
    t = tags.copy()
    t[wl.n_rows // 2] = bad
    xd = dev(x)
    with pytest.raises(lib.H3Error) as ei:
        lib.dit_block_forward(wl.dims, xd, dev(t), dev(pos), dev(table[0]), block, ws)
    assert ei.value.status == -1   # H3_ERR_INVALID_ARG
    assert "H3_CHECK" in str(ei.value)
    torch.cuda.synchronize()
    assert np.array_equal(xd.cpu().numpy(), x)


def test_check_mode_covers_step_calls(case, monkeypatch):
    say("check mode: step calls")
    wl, tags, pos, x, table, block, ws = case
    monkeypatch.setenv("H3_CHECK", "1")
    t = tags.copy()
    t[0] = wl.dims.n_tags
    h = torch.empty(wl.n_rows, wl.dims.hidden, dtype=torch.int16, device="cuda")
    with pytest.raises(lib.H3Error):
        lib.adaln_modulate(wl.dims, dev(x), dev(t), dev(table[0]), 0, h)


def test_check_mode_velocity_forward_without_blocks_reads_no_tags(monkeypatch):
    """With no block to run the velocity forward reads no tag, so tag may be
    NULL: under H3_CHECK=1 the call still succeeds and matches the run without
    the check bit for bit."""
    dims, io = synth.TINY_DIMS, synth.TINY_IO
    say("check mode: velocity forward, n_blocks = 0, tag NULL")
    wl = synth.Workload("io", dims, 0, 16, 8, 20, (2, 8, 8))
    inp = synth.make_io_inputs(wl, io, seed=72)
    w = {k: (None if v is None else dev(v)) for k, v in synth.make_io_weights(dims, io, seed=72).items()}
    ftab = dev(synth.make_final_table(dims, seed=72))
    d = {k: (dev(v) if len(v) else None) for k, v in inp.items()}
    sg = lib.segments_of(d["text"], d["cond"], d["audio"], d["video"])
    ws = torch.empty(lib.heads_workspace_size(dims, sg), dtype=torch.uint8, device="cuda")

    def run():
        x = torch.empty(wl.n_rows, dims.hidden, dtype=torch.float32, device="cuda")
        va = torch.empty(wl.A, io.audio_patch, dtype=torch.float32, device="cuda")
        vv = torch.empty(128, io.video_patch, dtype=torch.float32, device="cuda")
        lib.velocity_forward(dims, io, w, d["text"], d["cond"], d["audio"], d["video"],
                             None, None, None, [], ftab, x, va, vv, ws)
        torch.cuda.synchronize()
        return va.cpu().numpy(), vv.cpu().numpy()

    ref = run()
    monkeypatch.setenv("H3_CHECK", "1")
    got = run()
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])

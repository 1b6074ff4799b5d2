"""Parity of the steps around the block stack against the float64 oracle (GPU).

Input projections into the packed stream, the final per-modality AdaLN with the
output heads, and the composed velocity forward, all through the C ABI on
generator inputs (never a value produced by the HIP path).  Sizes cover the
small model, the H3 width at one block's shape, ragged segment lengths (one
row, rows not a multiple of 32) and the full-size segment geometry of the
N = 49,840 workload on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import TOL_BF16_OUT, TOL_BLOCK, TOL_DEPTH, dev, rel_l2, say

pytestmark = pytest.mark.gpu

# fp32 projections: fp32 products and sums against float64 (K <= 5120 terms)
TOL_EMBED = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


def _dev_io(w):
    return {k: (None if v is None else dev(v)) for k, v in w.items()}


def _seg_inputs(io, L, C, A, V, seed):
    wl = synth.Workload("io", synth.TINY_DIMS, 0, L, C, A, (1, 1, V))
    return synth.make_io_inputs(wl, io, seed=seed)


def _run_embed(dims, io, inp, w):
    N = sum(len(inp[k]) for k in ("text", "cond", "audio", "video"))
    x = torch.full((N, dims.hidden), float("nan"), dtype=torch.float32, device="cuda")
    d = {k: (dev(v) if len(v) else None) for k, v in inp.items()}
    lib.embed_inputs(dims, io, _dev_io(w), d["text"], d["cond"], d["audio"], d["video"], x)
    torch.cuda.synchronize()
    return x


EMBED_CASES = [
    ("tiny", synth.TINY_DIMS, synth.TINY_IO, (16, 8, 20, 128)),
    ("tiny-ragged", synth.TINY_DIMS, synth.TINY_IO, (1, 0, 33, 97)),
    ("tiny-video-only", synth.TINY_DIMS, synth.TINY_IO, (0, 0, 0, 31)),
    ("h3", synth.H3_DIMS, synth.H3_IO, (128, 40, 40, 1024)),
]


@pytest.mark.parametrize("name,dims,io,seg", EMBED_CASES, ids=[c[0] for c in EMBED_CASES])
def test_embed_inputs(name, dims, io, seg):
    say("embed", name, seg)
    inp = _seg_inputs(io, *seg, seed=5)
    w = synth.make_io_weights(dims, io, seed=5)
    x = _run_embed(dims, io, inp, w).cpu().numpy().astype(np.float64)
    ref = oracle.embed_inputs(inp["text"], inp["cond"], inp["audio"], inp["video"], w)
    assert np.isfinite(x).all(), "a row of the stream was not written"
    assert rel_l2(x, ref) < TOL_EMBED
    scale = np.abs(ref).max()
    assert np.abs(x - ref).max() < 1e-5 * scale


def _run_heads(dims, io, x_host, counts, ftab, w):
    sg = lib.make_segments(counts["text"], counts["cond"], counts["audio"], counts["video"])
    va = torch.empty(counts["audio"], io.audio_patch, dtype=torch.float32, device="cuda") if counts["audio"] else None
    vv = torch.empty(counts["video"], io.video_patch, dtype=torch.float32, device="cuda") if counts["video"] else None
    ws = torch.empty(lib.heads_workspace_size(dims, sg), dtype=torch.uint8, device="cuda")
    lib.final_heads(dims, io, _dev_io(w), sg, dev(x_host), dev(ftab), va, vv, ws)
    torch.cuda.synchronize()
    return (None if va is None else va.cpu().numpy().astype(np.float64),
            None if vv is None else vv.cpu().numpy().astype(np.float64))


HEAD_CASES = [
    ("tiny", synth.TINY_DIMS, synth.TINY_IO, (16, 8, 20, 128)),
    ("tiny-ragged", synth.TINY_DIMS, synth.TINY_IO, (3, 0, 1, 301)),
    ("tiny-audio-only", synth.TINY_DIMS, synth.TINY_IO, (0, 0, 9, 0)),
    ("tiny-no-audio", synth.TINY_DIMS, synth.TINY_IO, (4, 2, 0, 17)),
    ("h3", synth.H3_DIMS, synth.H3_IO, (128, 0, 40, 1024)),
    ("h3-ragged", synth.H3_DIMS, synth.H3_IO, (5, 2, 257, 33)),
]


@pytest.mark.parametrize("name,dims,io,seg", HEAD_CASES, ids=[c[0] for c in HEAD_CASES])
def test_final_heads(name, dims, io, seg):
    say("final_heads", name, seg)
    counts = dict(zip(("text", "cond", "audio", "video"), seg))
    N = sum(seg)
    x = synth.make_x(N, dims, seed=6) * np.float32(2.5) + np.float32(0.7)
    w = synth.make_io_weights(dims, io, seed=6)
    ftab = synth.make_final_table(dims, seed=6)
    va, vv = _run_heads(dims, io, x, counts, ftab, w)
    ra, rv = oracle.final_heads(x, counts, ftab, w, dims.ln_eps)
    for got, ref in ((va, ra), (vv, rv)):
        if got is None:                      # a modality without rows has no velocity
            assert ref.shape[0] == 0
            continue
        assert got.shape == ref.shape
        assert rel_l2(got, ref) < TOL_BF16_OUT
        # per element: the bf16 rounding of h, summed over D terms of the head
        assert np.abs(got - ref).max() < 0.05 * np.abs(ref).max()


def test_velocity_forward_without_blocks_is_embed_then_heads():
    dims, io = synth.TINY_DIMS, synth.TINY_IO
    say("velocity n_blocks=0")
    inp = _seg_inputs(io, 16, 8, 20, 128, seed=8)
    w = synth.make_io_weights(dims, io, seed=8)
    ftab = dev(synth.make_final_table(dims, seed=8))
    d = {k: (dev(v) if len(v) else None) for k, v in inp.items()}
    N = 16 + 8 + 20 + 128
    x = torch.empty(N, dims.hidden, dtype=torch.float32, device="cuda")
    va = torch.empty(20, io.audio_patch, dtype=torch.float32, device="cuda")
    vv = torch.empty(128, io.video_patch, dtype=torch.float32, device="cuda")
    sg = lib.segments_of(d["text"], d["cond"], d["audio"], d["video"])
    ws = torch.empty(lib.heads_workspace_size(dims, sg), dtype=torch.uint8, device="cuda")
    lib.velocity_forward(dims, io, _dev_io(w), d["text"], d["cond"], d["audio"], d["video"],
                         None, None, None, [], ftab, x, va, vv, ws)
    x2 = _run_embed(dims, io, inp, w)
    va2, vv2 = torch.empty_like(va), torch.empty_like(vv)
    lib.final_heads(dims, io, _dev_io(w), sg, x2, ftab, va2, vv2, ws)
    torch.cuda.synchronize()
    assert torch.equal(x, x2) and torch.equal(va, va2) and torch.equal(vv, vv2)


VEL_CASES = [("tiny_2blk", synth.TINY_DIMS, synth.TINY_IO, (16, 8, 20, 128), 2, TOL_DEPTH),
             ("h3_1blk", synth.H3_DIMS, synth.H3_IO, (128, 0, 40, 1024), 1, TOL_BLOCK)]


@pytest.mark.parametrize("name,dims,io,seg,nb,tol", VEL_CASES, ids=[c[0] for c in VEL_CASES])
def test_velocity_forward(name, dims, io, seg, nb, tol):
    say("velocity_forward", name, seg, nb)
    L, C, A, V = seg
    vgrid = {1024: (1, 32, 32), 128: (2, 8, 8)}[V]
    wl = synth.Workload("vel", dims, nb, L, C, A, vgrid)
    tags, pos = synth.packed_layout(wl)
    table = synth.make_table(dims, nb, seed=9)
    blocks_host = [synth.make_block_weights(dims, b, seed=9) for b in range(nb)]
    inp = synth.make_io_inputs(wl, io, seed=9)
    w = synth.make_io_weights(dims, io, seed=9)
    ftab = synth.make_final_table(dims, seed=9)
    d = {k: (dev(v) if len(v) else None) for k, v in inp.items()}
    N = wl.n_rows
    x = torch.empty(N, dims.hidden, dtype=torch.float32, device="cuda")
    va = torch.empty(A, io.audio_patch, dtype=torch.float32, device="cuda")
    vv = torch.empty(V, io.video_patch, dtype=torch.float32, device="cuda")
    ws = lib.alloc_workspace(dims, N)
    lib.velocity_forward(dims, io, _dev_io(w), d["text"], d["cond"], d["audio"], d["video"],
                         dev(tags), dev(pos), dev(table), [lib.to_device_block(b) for b in blocks_host],
                         dev(ftab), x, va, vv, ws)
    torch.cuda.synchronize()
    ra, rv = oracle.velocity_forward(inp["text"], inp["cond"], inp["audio"], inp["video"], w, ftab,
                                     tags, pos, table, lambda b: blocks_host[b], nb, dims)
    ea, ev = rel_l2(va.cpu().numpy(), ra), rel_l2(vv.cpu().numpy(), rv)
    say("velocity rel-L2 audio", ea, "video", ev)
    assert ea < tol and ev < tol


def test_fullsize_segments_n49840_sampled_rows():
    """The N = 49,840 segment geometry (256 text, 1024 condition, 200 audio,
    48,360 video rows) at H3 width: embed and heads as one launch each per
    segment, as the forward runs them; sampled rows against the oracle."""
    dims, io = synth.H3_DIMS, synth.H3_IO
    wl = synth.WORKLOADS["h3_50blk_n49840"]
    say("fullsize io", wl.name)
    inp = synth.make_io_inputs(wl, io, seed=10)
    w = synth.make_io_weights(dims, io, seed=10)
    x = _run_embed(dims, io, inp, w)
    counts = {"text": wl.L, "cond": wl.C, "audio": wl.A, "video": wl.n_rows - wl.L - wl.C - wl.A}
    seg = oracle.segment_rows(counts)
    rng = np.random.default_rng(10)
    xs = x.cpu().numpy().astype(np.float64)
    assert np.isfinite(xs).all()
    for name in ("text", "cond", "audio", "video"):
        rows = np.unique(np.concatenate([[seg[name].start, seg[name].stop - 1],
                                         rng.integers(seg[name].start, seg[name].stop, 24)]))
        local = rows - seg[name].start
        sub = {k: inp[k][:0] for k in ("text", "cond", "audio", "video")}
        sub[name] = inp[name][local]
        ref = oracle.embed_inputs(sub["text"], sub["cond"], sub["audio"], sub["video"], w)
        assert rel_l2(xs[rows], ref) < TOL_EMBED, name
    ftab = synth.make_final_table(dims, seed=10)
    sg = lib.make_segments(counts["text"], counts["cond"], counts["audio"], counts["video"])
    va = torch.empty(counts["audio"], io.audio_patch, dtype=torch.float32, device="cuda")
    vv = torch.empty(counts["video"], io.video_patch, dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.heads_workspace_size(dims, sg), dtype=torch.uint8, device="cuda")
    lib.final_heads(dims, io, _dev_io(w), sg, x, dev(ftab), va, vv, ws)
    torch.cuda.synchronize()
    vah, vvh = va.cpu().numpy(), vv.cpu().numpy()
    for name, got in (("audio", vah), ("video", vvh)):
        local = np.unique(np.concatenate([[0, counts[name] - 1], rng.integers(0, counts[name], 48)]))
        c = {k: 0 for k in counts}
        c[name] = len(local)
        ref = oracle.final_heads(xs[seg[name].start + local], c, ftab, w, dims.ln_eps)
        ref = ref[0] if name == "audio" else ref[1]
        assert rel_l2(got[local], ref) < TOL_BF16_OUT, name

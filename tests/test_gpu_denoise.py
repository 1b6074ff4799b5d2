"""Parity of the GPU denoising loop (h3_denoise) against the oracle's Euler loop.

Each pass of the oracle runs its own velocity forward (inputs, blocks, final
AdaLN and heads) with that pass's tables; the latents step on the video (12)
and audio (3) shifted schedules.  One GPU pass also equals one velocity
forward followed by the Euler update.  With velocity reuse the loop matches
the oracle's reuse loop: 2 over 4 passes (fresh at 0, 2 and 3; pass 1 steps
along the only fresh velocity), 3 over 7 passes (fresh at 0, 3 and 6; passes 4
and 5 extrapolate each modality's velocity in its own sigma through passes 0
and 3), and 5 over 3 passes (first and last only).
"""
import numpy as np
import pytest
import torch

import oracle
from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import TOL_BLOCK, TOL_DEPTH, dev, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


def _case(dims, io, L, C, A, vgrid, nb, steps, seed):
    wl = synth.Workload("den", dims, nb, L, C, A, vgrid)
    tags, pos = synth.packed_layout(wl)
    tables = synth.make_table(dims, nb * steps, seed=seed).reshape(steps, nb, dims.n_tags, 6, dims.hidden)
    finals = np.stack([synth.make_final_table(dims, seed=seed + 100 + i) for i in range(steps)])
    blocks = [synth.make_block_weights(dims, b, seed=seed) for b in range(nb)]
    inp = synth.make_io_inputs(wl, io, seed=seed)
    w = synth.make_io_weights(dims, io, seed=seed)
    return wl, tags, pos, tables, finals, blocks, inp, w


def _gpu(dims, io, wl, tags, pos, tables, finals, blocks, inp, w, sa, sv, reuse=1):
    d = {k: (dev(v) if len(v) else None) for k, v in inp.items()}
    x = torch.empty(wl.n_rows, dims.hidden, dtype=torch.float32, device="cuda")
    ws = lib.alloc_denoise_workspace(dims, io, d["text"], d["cond"], d["audio"], d["video"])
    iw = {k: (None if v is None else dev(v)) for k, v in w.items()}
    lib.denoise(dims, io, iw, d["text"], d["cond"], d["audio"], d["video"], dev(tags), dev(pos),
                dev(np.ascontiguousarray(tables)), [lib.to_device_block(b) for b in blocks],
                dev(np.ascontiguousarray(finals)), sa, sv, x, ws, reuse=reuse)
    torch.cuda.synchronize()
    return d["audio"].cpu().numpy(), d["video"].cpu().numpy()


CASES = [("tiny", synth.TINY_DIMS, synth.TINY_IO, 16, 8, 20, (2, 8, 8), 2, 3, TOL_DEPTH),
         ("h3", synth.H3_DIMS, synth.H3_IO, 128, 0, 40, (1, 32, 32), 1, 2, TOL_BLOCK)]


@pytest.mark.parametrize("name,dims,io,L,C,A,vgrid,nb,steps,tol", CASES, ids=[c[0] for c in CASES])
def test_denoise_matches_oracle(name, dims, io, L, C, A, vgrid, nb, steps, tol):
    say("denoise", name, nb, steps)
    wl, tags, pos, tables, finals, blocks, inp, w = _case(dims, io, L, C, A, vgrid, nb, steps, seed=40)
    sa, sv = lib.sigma_schedule(steps, 3.0), lib.sigma_schedule(steps, 12.0)
    ga, gv = _gpu(dims, io, wl, tags, pos, tables, finals, blocks, inp, w, sa, sv)

    def vel(i, a, v):
        return oracle.velocity_forward(inp["text"], inp["cond"], a.astype(np.float32), v.astype(np.float32),
                                       w, finals[i], tags, pos, tables[i], lambda b: blocks[b], nb, dims)

    ra, rv = oracle.denoise(inp["audio"], inp["video"], np.array(sa), np.array(sv), vel)
    ea, ev = rel_l2(ga, ra), rel_l2(gv, rv)
    da = rel_l2(ga - inp["audio"], ra - inp["audio"])
    dv = rel_l2(gv - inp["video"], rv - inp["video"])
    say("denoise rel-L2 latents audio", ea, "video", ev, "| updates", da, dv)
    assert ea < tol and ev < tol and da < 2 * tol and dv < 2 * tol


def test_one_pass_is_velocity_forward_then_euler():
    dims, io = synth.TINY_DIMS, synth.TINY_IO
    say("denoise one pass")
    wl, tags, pos, tables, finals, blocks, inp, w = _case(dims, io, 16, 8, 20, (2, 8, 8), 2, 1, seed=41)
    sa, sv = lib.sigma_schedule(1, 3.0), lib.sigma_schedule(1, 12.0)
    ga, gv = _gpu(dims, io, wl, tags, pos, tables, finals, blocks, inp, w, sa, sv)
    d = {k: (dev(v) if len(v) else None) for k, v in inp.items()}
    iw = {k: (None if v is None else dev(v)) for k, v in w.items()}
    x = torch.empty(wl.n_rows, dims.hidden, dtype=torch.float32, device="cuda")
    va = torch.empty(wl.A, io.audio_patch, dtype=torch.float32, device="cuda")
    vv = torch.empty(128, io.video_patch, dtype=torch.float32, device="cuda")
    ws = lib.alloc_workspace(dims, wl.n_rows)
    lib.velocity_forward(dims, io, iw, d["text"], d["cond"], d["audio"], d["video"], dev(tags), dev(pos),
                         dev(np.ascontiguousarray(tables[0])), [lib.to_device_block(b) for b in blocks],
                         dev(finals[0]), x, va, vv, ws)
    torch.cuda.synchronize()
    ea = inp["audio"] + np.float32(sa[1] - sa[0]) * va.cpu().numpy()
    ev = inp["video"] + np.float32(sv[1] - sv[0]) * vv.cpu().numpy()
    np.testing.assert_allclose(ga, ea, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(gv, ev, rtol=1e-6, atol=1e-6)


def test_denoise_with_velocity_reuse_matches_oracle():
    dims, io = synth.TINY_DIMS, synth.TINY_IO
    steps, reuse = 4, 2
    say("denoise reuse", reuse, steps)
    wl, tags, pos, tables, finals, blocks, inp, w = _case(dims, io, 16, 8, 20, (2, 8, 8), 2, steps, seed=42)
    sa, sv = lib.sigma_schedule(steps, 3.0), lib.sigma_schedule(steps, 12.0)
    ga, gv = _gpu(dims, io, wl, tags, pos, tables, finals, blocks, inp, w, sa, sv, reuse=reuse)
    calls = []

    def vel(i, a, v):
        calls.append(i)
        return oracle.velocity_forward(inp["text"], inp["cond"], a.astype(np.float32), v.astype(np.float32),
                                       w, finals[i], tags, pos, tables[i], lambda b: blocks[b], 2, dims)

    ra, rv = oracle.denoise(inp["audio"], inp["video"], np.array(sa), np.array(sv), vel, reuse=reuse)
    assert calls == [0, 2, 3]
    ea, ev = rel_l2(ga, ra), rel_l2(gv, rv)
    say("denoise reuse rel-L2 audio", ea, "video", ev)
    assert ea < TOL_DEPTH and ev < TOL_DEPTH
    # reuse changes the result (passes 1 and 2 differ from the fresh loop)
    fa, fv = _gpu(dims, io, wl, tags, pos, tables, finals, blocks, inp, w, sa, sv, reuse=1)
    assert rel_l2(fa, ga) > 10 * ea


def test_reuse_beyond_steps_runs_first_and_last_pass_only():
    dims, io = synth.TINY_DIMS, synth.TINY_IO
    say("denoise reuse 5 over 3")
    wl, tags, pos, tables, finals, blocks, inp, w = _case(dims, io, 16, 8, 20, (2, 8, 8), 2, 3, seed=43)
    sa, sv = lib.sigma_schedule(3, 3.0), lib.sigma_schedule(3, 12.0)
    ga, gv = _gpu(dims, io, wl, tags, pos, tables, finals, blocks, inp, w, sa, sv, reuse=5)
    calls = []

    def vel(i, a, v):
        calls.append(i)
        return oracle.velocity_forward(inp["text"], inp["cond"], a.astype(np.float32), v.astype(np.float32),
                                       w, finals[i], tags, pos, tables[i], lambda b: blocks[b], 2, dims)

    ra, rv = oracle.denoise(inp["audio"], inp["video"], np.array(sa), np.array(sv), vel, reuse=5)
    assert calls == [0, 2]
    assert rel_l2(ga, ra) < TOL_DEPTH and rel_l2(gv, rv) < TOL_DEPTH


def test_denoise_reuse_extrapolates_skipped_velocities(monkeypatch):
    """Reuse 3 over 7 passes: fresh at 0, 3 and 6; passes 1 and 2 step along
    the velocity of pass 0, passes 4 and 5 along the straight line in each
    modality's sigma through the velocities of passes 0 and 3."""
    dims, io = synth.TINY_DIMS, synth.TINY_IO
    steps, reuse = 7, 3
    say("denoise reuse", reuse, steps)
    wl, tags, pos, tables, finals, blocks, inp, w = _case(dims, io, 16, 8, 20, (2, 8, 8), 2, steps, seed=44)
    sa, sv = lib.sigma_schedule(steps, 3.0), lib.sigma_schedule(steps, 12.0)
    ga, gv = _gpu(dims, io, wl, tags, pos, tables, finals, blocks, inp, w, sa, sv, reuse=reuse)
    calls = []

    def vel(i, a, v):
        calls.append(i)
        return oracle.velocity_forward(inp["text"], inp["cond"], a.astype(np.float32), v.astype(np.float32),
                                       w, finals[i], tags, pos, tables[i], lambda b: blocks[b], 2, dims)

    ra, rv = oracle.denoise(inp["audio"], inp["video"], np.array(sa), np.array(sv), vel, reuse=reuse)
    assert calls == [0, 3, 6]
    ea, ev = rel_l2(ga, ra), rel_l2(gv, rv)
    da = rel_l2(ga - inp["audio"], ra - inp["audio"])
    dv = rel_l2(gv - inp["video"], rv - inp["video"])
    say("denoise reuse 3 rel-L2 audio", ea, "video", ev, "| updates", da, dv)
    assert ea < TOL_DEPTH and ev < TOL_DEPTH and da < 2 * TOL_DEPTH and dv < 2 * TOL_DEPTH
    # the extrapolation matters at this size: the oracle with held velocities
    # on passes 4 and 5 lands much farther from the GPU result
    import oracle.h3_sampler as sampler
    monkeypatch.setattr(sampler, "extrapolate", lambda sig, i, j0, v0, j1, v1: v1)
    ha, hv = oracle.denoise(inp["audio"], inp["video"], np.array(sa), np.array(sv), vel, reuse=reuse)
    say("  held instead: rel-L2 audio", rel_l2(ga, ha), "video", rel_l2(gv, hv))
    assert rel_l2(gv - inp["video"], hv - inp["video"]) > 5 * dv

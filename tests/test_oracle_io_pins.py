"""Pins of the CPU oracle's steps around the block stack (no GPU needed).

The packed order [text | conditions | audio | video], the projection each
segment takes, the weight orientation W[out][in], the final per-modality AdaLN
and the composition order are each tied to a closed form, a library routine or
an invariant, so a swapped segment, a transposed weight, a dropped bias or a
wrong (shift, scale) slot fails one of these tests.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from joint_video_audio_h3_amd import synth

TINY = synth.TINY_DIMS
IO = synth.TINY_IO
WL = synth.WORKLOADS["tiny_2blk_n164"]
ONE_BF16 = np.uint16(0x3F80)      # 1.0
HALF_BF16 = np.uint16(0x3F00)     # 0.5


def _counts(inp):
    return {k: len(inp[k]) for k in ("text", "cond", "audio", "video")}


def _inputs(C=5):
    wl = synth.Workload("io_pin", TINY, 0, WL.L, C, WL.A, WL.V)
    return synth.make_io_inputs(wl, IO, seed=3)


def _identity_io_weights():
    """Projections that copy their input into known columns of the stream."""
    D = TINY.hidden
    w = {k: None for k in ("b_text", "b_video", "b_audio", "b_head_audio", "b_head_video")}
    wt = np.zeros((D, IO.text_dim), np.uint16)
    wt[128 + np.arange(IO.text_dim), np.arange(IO.text_dim)] = ONE_BF16   # text -> cols 128..255
    wv = np.zeros((D, IO.video_patch), np.float32)
    wv[np.arange(IO.video_patch), np.arange(IO.video_patch)] = 1.0        # video -> cols 0..95
    wa = np.zeros((D, IO.audio_patch), np.float32)
    wa[96 + np.arange(IO.audio_patch), np.arange(IO.audio_patch)] = 1.0   # audio -> cols 96..127
    w.update(w_text=wt, w_video=wv, w_audio=wa)
    return w


def test_embed_places_segments_in_packed_order_with_their_projection():
    inp = _inputs()
    w = _identity_io_weights()
    w["b_text"] = np.full(TINY.hidden, HALF_BF16, np.uint16)
    w["b_audio"] = np.full(TINY.hidden, -2.0, np.float32)
    x = oracle.embed_inputs(inp["text"], inp["cond"], inp["audio"], inp["video"], w)
    seg = oracle.segment_rows(_counts(inp))
    assert x.shape == (sum(_counts(inp).values()), TINY.hidden)
    assert [seg[s].start for s in oracle.SEGMENTS] == [0, WL.L, WL.L + 5, WL.L + 5 + WL.A]
    text = oracle.bf16_to_f64(inp["text"])
    np.testing.assert_array_equal(x[seg["text"], 128:], text + 0.5)
    np.testing.assert_array_equal(x[seg["text"], :128], 0.5)
    # conditions are video latents: they take the video projection
    np.testing.assert_array_equal(x[seg["cond"], :96], inp["cond"].astype(np.float64))
    np.testing.assert_array_equal(x[seg["cond"], 96:], 0.0)
    np.testing.assert_array_equal(x[seg["audio"], 96:128], inp["audio"].astype(np.float64) - 2.0)
    np.testing.assert_array_equal(x[seg["audio"], :96], -2.0)
    np.testing.assert_array_equal(x[seg["video"], :96], inp["video"].astype(np.float64))
    np.testing.assert_array_equal(x[seg["video"], 96:], 0.0)


def test_embed_matches_torch_linear_fp64():
    inp = _inputs()
    w = synth.make_io_weights(TINY, IO, seed=5)
    x = oracle.embed_inputs(inp["text"], inp["cond"], inp["audio"], inp["video"], w)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    bf = lambda a: t(synth.bf16_bits_to_f32(a).astype(np.float64))  # noqa: E731
    ref = torch.cat([
        F.linear(bf(inp["text"]), bf(w["w_text"]), bf(w["b_text"])),
        F.linear(t(inp["cond"]), t(w["w_video"]), t(w["b_video"])),
        F.linear(t(inp["audio"]), t(w["w_audio"]), t(w["b_audio"])),
        F.linear(t(inp["video"]), t(w["w_video"]), t(w["b_video"])),
    ]).numpy()
    np.testing.assert_allclose(x, ref, rtol=1e-12, atol=1e-12)


def _head_setup(seed=7):
    r = np.random.default_rng(seed)
    counts = {"text": 3, "cond": 2, "audio": 5, "video": 6}
    N = sum(counts.values())
    x = r.standard_normal((N, TINY.hidden)) * 3.0 + 1.5
    w = synth.make_io_weights(TINY, IO, seed=seed)
    return counts, x, w


def test_final_heads_scale_minus_one_gives_shift_through_head():
    counts, x, w = _head_setup()
    tab = synth.make_final_table(TINY, seed=1)
    tab[:, 1, :] = np.uint16(0xBF80)          # scale = -1: LN(x) * 0 + shift
    va, vv = oracle.final_heads(x, counts, tab, w, TINY.ln_eps)
    for m, (v, name, P) in enumerate(((va, "audio", IO.audio_patch), (vv, "video", IO.video_patch))):
        shift = oracle.bf16_to_f64(tab[m, 0])
        want = oracle.bf16_to_f64(w["w_head_" + name]) @ shift + oracle.bf16_to_f64(w["b_head_" + name])
        assert v.shape == (counts[name], P)
        np.testing.assert_allclose(v, np.broadcast_to(want, v.shape), rtol=1e-12, atol=1e-12)


def test_final_heads_normalise_rows_of_known_moments():
    """Rows a + b*e with e = +-1 (mean 0, variance 1) normalise to e; identity
    heads then return e in their columns, plus (1 + scale) and shift."""
    counts = {"text": 1, "cond": 0, "audio": 2, "video": 3}
    D = TINY.hidden
    e = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    rows = [a + b * e for a, b in ((9.0, 0.25), (-4.0, 3.0), (0.5, 7.0), (100.0, 0.5), (2.0, 2.0), (0.0, 1.0))]
    x = np.stack(rows)
    w = {"w_head_audio": np.zeros((IO.audio_patch, D), np.uint16),
         "w_head_video": np.zeros((IO.video_patch, D), np.uint16),
         "b_head_audio": None, "b_head_video": None}
    w["w_head_audio"][np.arange(IO.audio_patch), np.arange(IO.audio_patch)] = ONE_BF16
    w["w_head_video"][np.arange(IO.video_patch), 100 + np.arange(IO.video_patch)] = ONE_BF16
    tab = np.zeros((2, 2, D), np.uint16)
    tab[0, 1] = ONE_BF16                      # audio scale 1 -> factor 2
    tab[1, 0] = HALF_BF16                     # video shift 0.5
    va, vv = oracle.final_heads(x, counts, tab, w, 0.0)
    np.testing.assert_allclose(va, np.broadcast_to(2.0 * e[:IO.audio_patch], va.shape), rtol=1e-12)
    np.testing.assert_allclose(vv, np.broadcast_to(e[100:100 + IO.video_patch] + 0.5, vv.shape), rtol=1e-12)


def test_final_heads_are_row_local_and_segment_local():
    counts, x, w = _head_setup(11)
    tab = synth.make_final_table(TINY, seed=2)
    va, vv = oracle.final_heads(x, counts, tab, w, TINY.ln_eps)
    seg = oracle.segment_rows(counts)
    y = x.copy()
    y[seg["text"]] *= -3.0                    # text and condition rows feed no head
    y[seg["cond"]] += 5.0
    y[seg["video"].start + 2] += 1.0          # one video row changes one velocity row
    wa, wv = oracle.final_heads(y, counts, tab, w, TINY.ln_eps)
    np.testing.assert_array_equal(wa, va)
    changed = np.where(np.any(wv != vv, axis=1))[0]
    assert changed.tolist() == [2]


def test_velocity_forward_composes_embed_blocks_heads():
    """With every gate zero the blocks are the identity, so the depth drops out."""
    wl = synth.Workload("io_pin", TINY, 2, WL.L, 4, WL.A, WL.V)
    inp = synth.make_io_inputs(wl, IO, seed=4)
    w = synth.make_io_weights(TINY, IO, seed=4)
    x, tags, pos, table, blocks = synth.make_inputs(wl, seed=4)
    ftab = synth.make_final_table(TINY, seed=4)
    args = (inp["text"], inp["cond"], inp["audio"], inp["video"], w, ftab, tags, pos)
    counts = _counts(inp)
    direct = oracle.final_heads(oracle.embed_inputs(*args[:5]), counts, ftab, w, TINY.ln_eps)
    zero_gates = table.copy()
    zero_gates[:, :, 2] = 0
    zero_gates[:, :, 5] = 0
    va, vv = oracle.velocity_forward(*args, zero_gates, lambda b: blocks[b], 2, TINY)
    np.testing.assert_allclose(va, direct[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(vv, direct[1], rtol=1e-12, atol=1e-12)
    va2, vv2 = oracle.velocity_forward(*args, table, lambda b: blocks[b], 2, TINY)
    assert np.abs(vv2 - vv).max() > 1e-3     # the real gates do change the velocity

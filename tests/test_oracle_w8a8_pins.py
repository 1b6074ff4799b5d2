"""Pins of the W8A8 oracle (per-row int8 activations x per-row int8 weights).

The quantizer is tied to closed forms (power-of-two scales make every step
exact, so the codes are known in advance, ties included) and to its error
bound; the integer linear to brute force in Python integers; and the wiring
into the block to the bf16 path on activations that lie on the int8 grid,
where quantization is lossless and both paths must agree.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from joint_video_audio_h3_amd import synth

TINY = synth.TINY_DIMS
TINY_W8A8 = dataclasses.replace(TINY, wfmt=synth.WFMT_W8A8)


def test_quantize_rows_closed_forms():
    base = np.array([127.0, -127.0, 1.0, 0.5, 1.5, 2.5, -0.5, 126.5])
    rows = np.stack([base * 4.0, base * 2.0 ** -10, np.zeros(8)])
    q, s = oracle.quantize_rows(rows)
    # scale = amax / 127 = 2^k exactly; codes = rint(value / 2^k), ties to even
    want = np.array([127, -127, 1, 0, 2, 2, 0, 126])
    np.testing.assert_array_equal(q[0], want)
    np.testing.assert_array_equal(q[1], want)
    np.testing.assert_array_equal(q[2], 0)
    assert s.dtype == np.float32 and s.tolist() == [4.0, 2.0 ** -10, 0.0]


def test_quantize_rows_bound_and_full_range():
    r = np.random.default_rng(0)
    a = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        (r.standard_normal((64, 384)) * r.uniform(1e-3, 1e3, (64, 1))).astype(np.float32))).astype(np.float64)
    q, s = oracle.quantize_rows(a)
    assert np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(q.astype(np.float64) * s[:, None].astype(np.float64) - a)
    # half a code step, plus the float32 rounding of the scale and of a * inv
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -16))
    # the sign of every nonzero code follows the value
    nz = q != 0
    assert np.all(np.sign(q[nz]) == np.sign(a[nz]))


def test_linear_w8a8_brute_force_integers():
    r = np.random.default_rng(1)
    R, C, K = 3, 4, 37
    qa = r.integers(-127, 128, (R, K)).astype(np.int8)
    qw = r.integers(-127, 128, (C, K)).astype(np.int8)
    sa = np.array([0.5, 3.0, 2.0 ** -7], np.float32)
    sw_bits = synth.f32_to_bf16_bits(np.array([1.0, 0.25, -2.0, 96.0], np.float32))
    b = np.array([0.0, 1.0, -1.0, 0.5])
    y = oracle.linear_w8a8(qa, sa, qw, sw_bits, b)
    sw = [1.0, 0.25, -2.0, 96.0]
    for i in range(R):
        for j in range(C):
            dot = sum(int(qa[i, k]) * int(qw[j, k]) for k in range(K))
            assert y[i, j] == float(sa[i]) * sw[j] * dot + b[j]


@pytest.mark.parametrize("name,n_out,k", [("qkv", 3 * 384, 256), ("out", 256, 384),
                                          ("fc1", 2 * 768, 256), ("fc2", 256, 768)])
def test_w8a8_linear_equals_float_linear_on_grid(name, n_out, k):
    """Activations s_r * q (q integers, max |q| = 127, s_r a power of two) are bf16
    values the quantizer maps back to themselves, so the W8A8 linear must equal
    the float linear with the dequantized weights."""
    r = np.random.default_rng(2)
    w = synth.make_block_weights(TINY_W8A8, 0, seed=3)
    qa = r.integers(-126, 127, (5, k))
    qa[:, 7] = 127
    act = qa * (2.0 ** r.integers(-12, 4, (5, 1)))
    got = oracle.linear(act, w, name, n_out, TINY_W8A8)
    W = w["w_" + name].astype(np.float64) * oracle.bf16_to_f64(w["s_" + name])[:, None]
    ref = act @ W.T + oracle.bf16_to_f64(w["b_" + name])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_w8a8_block_close_to_dequantized_float_block():
    """The W8A8 block differs from the float block on the dequantized weights
    (rounded to bf16) by activation quantization and that rounding: small, but present."""
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    x, tags, pos, table, _ = synth.make_inputs(wl, seed=4, n_blocks=1)
    w8 = synth.make_block_weights(TINY_W8A8, 0, seed=4)
    wf = dict(w8)
    for n in ("qkv", "out", "fc1", "fc2"):
        W = w8["w_" + n].astype(np.float64) * oracle.bf16_to_f64(w8["s_" + n])[:, None]
        wf["w_" + n] = synth.f32_to_bf16_bits(W.astype(np.float32))
        wf["s_" + n] = None
    y8 = oracle.block_forward(x, tags, pos, table[0], w8, TINY_W8A8)
    yf = oracle.block_forward(x, tags, pos, table[0], wf, TINY)
    d = np.linalg.norm((y8 - x) - (yf - x)) / np.linalg.norm(yf - x)
    assert 1e-4 < d < 3e-2

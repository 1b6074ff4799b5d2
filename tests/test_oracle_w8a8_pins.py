"""Pins of the group-scaled W8A8 oracle (int8 activations and weights, one
scale per group of G elements along K; FC2 optionally per row).

The quantizer is tied to closed forms (power-of-two scales make every step
exact, so the codes are known in advance, ties included) and to its error
bound; the grouped integer linear to brute force in Python integers, to the
per-row form when one group spans K, and to a case that only per-group scales
get right; the wiring into the block to the float path on activations and
weights that lie on their groups' int8 grids, where quantization is lossless
and both must agree (a transposed or shifted scale index fails there).
"""
import dataclasses

import numpy as np
import pytest

import oracle
from joint_video_audio_h3_amd import synth

TINY = synth.TINY_DIMS
TINY_W8A8 = synth.TINY_W8A8_DIMS


def test_accepted_group_sizes_of_the_pages():
    assert oracle.ACCEPTED_GROUPS == (64, 256, 448, 896)
    # every accepted group tiles the H3 widths (hidden, heads*head_dim, ffn)
    for g in oracle.ACCEPTED_GROUPS:
        assert 5376 % g == 0 and 7168 % g == 0 and 14336 % g == 0
    assert [5376 // 896, 7168 // 896, 14336 // 896] == [6, 8, 16]


def test_quantize_groups_closed_forms():
    base = np.array([127.0, -127.0, 1.0, 0.5, 1.5, 2.5, -0.5, 126.5])
    # two groups of 8 per row with different power-of-two scales, and a zero group
    rows = np.stack([np.concatenate([base * 4.0, base * 2.0 ** -10]),
                     np.concatenate([np.zeros(8), base * 2.0 ** 3])])
    q, s = oracle.quantize_groups(rows, 8)
    # scale = amax / 127 = 2^k exactly; codes = rint(value / 2^k), ties to even
    want = np.array([127, -127, 1, 0, 2, 2, 0, 126])
    np.testing.assert_array_equal(q[0], np.concatenate([want, want]))
    np.testing.assert_array_equal(q[1], np.concatenate([np.zeros(8, int), want]))
    assert s.dtype == np.float32 and s.shape == (2, 2)
    assert s.tolist() == [[4.0, 2.0 ** -10], [0.0, 8.0]]


def test_quantize_rows_is_one_group_per_row():
    r = np.random.default_rng(7)
    a = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(r.standard_normal((5, 96)).astype(np.float32)))
    q1, s1 = oracle.quantize_rows(a)
    q2, s2 = oracle.quantize_groups(a, 96)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2[:, 0])


@pytest.mark.parametrize("group", [64, 256, 448, 896])
def test_quantize_groups_bound_and_full_range(group):
    r = np.random.default_rng(group)
    K = 1792
    scale = r.uniform(1e-3, 1e3, (16, K // group)).repeat(group, axis=1)
    a = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        (r.standard_normal((16, K)) * scale).astype(np.float32))).astype(np.float64)
    q, s = oracle.quantize_groups(a, group)
    assert s.shape == (16, K // group)
    qg = q.reshape(16, K // group, group)
    assert np.all(np.abs(qg).max(axis=2) == 127)          # every group uses its full range
    step = np.repeat(s.astype(np.float64), group, axis=1)
    err = np.abs(q.astype(np.float64) * step - a)
    # half a code step, plus the float32 rounding of the scale and of a * inv
    assert np.all(err <= step * (0.5 + 2.0 ** -16))
    nz = q != 0
    assert np.all(np.sign(q[nz]) == np.sign(a[nz]))


def test_linear_grouped_brute_force_integers():
    r = np.random.default_rng(1)
    R, C, G, ng = 3, 4, 5, 3
    K = G * ng
    qa = r.integers(-127, 128, (R, K)).astype(np.int8)
    qw = r.integers(-127, 128, (C, K)).astype(np.int8)
    sa = (2.0 ** r.integers(-8, 4, (R, ng))).astype(np.float32)
    swv = np.array([[1.0, 0.25, -2.0, 96.0], [0.5, 3.0, 1.0, 0.125], [8.0, -1.5, 0.75, 2.0]], np.float32)
    sw_bits = synth.f32_to_bf16_bits(swv)
    b = np.array([0.0, 1.0, -1.0, 0.5])
    y = oracle.linear_w8a8_grouped(qa, sa, qw, sw_bits, b, G)
    for i in range(R):
        for j in range(C):
            tot = 0.0
            for g in range(ng):
                dot = sum(int(qa[i, k]) * int(qw[j, k]) for k in range(g * G, (g + 1) * G))
                tot += float(sa[i, g]) * float(swv[g, j]) * dot
            assert y[i, j] == tot + b[j]


def test_linear_grouped_with_one_group_equals_per_row_form():
    r = np.random.default_rng(2)
    qa = r.integers(-127, 128, (6, 64)).astype(np.int8)
    qw = r.integers(-127, 128, (5, 64)).astype(np.int8)
    sa = r.uniform(0.1, 2.0, 6).astype(np.float32)
    sw = synth.f32_to_bf16_bits(r.uniform(0.1, 2.0, 5).astype(np.float32))
    b = r.standard_normal(5)
    np.testing.assert_array_equal(oracle.linear_w8a8_grouped(qa, sa[:, None], qw, sw[None, :], b, 64),
                                  oracle.linear_w8a8(qa, sa, qw, sw, b))


def test_group_boundary_case_only_group_scales_get_right():
    """A row whose first group is large and second small, both on their own
    group's int8 grid: group-scaled W8A8 reproduces the float product exactly;
    one scale per row flushes the small group to zero."""
    G = 64
    r = np.random.default_rng(3)
    codes = r.integers(-126, 127, (1, 2 * G))
    codes[0, 0] = codes[0, G] = 127
    act = np.concatenate([codes[:, :G] * 2.0 ** 4, codes[:, G:] * 2.0 ** -12], axis=1)
    wq = r.integers(-127, 128, (3, 2 * G)).astype(np.int8)
    wq[:, 0] = wq[:, G] = 127
    w = wq.astype(np.float64) * 2.0 ** -7                       # weights on their group grids
    _, sw_bits = synth.quantize_int8_groups(synth.f32_to_bf16_bits(w.astype(np.float32)), G)
    exact = act @ w.T
    qa, sa = oracle.quantize_groups(act, G)
    got = oracle.linear_w8a8_grouped(qa, sa, wq, sw_bits, None, G)
    np.testing.assert_array_equal(got, exact)
    qr, sr = oracle.quantize_rows(act)
    _, sw_row = synth.quantize_int8_rows(synth.f32_to_bf16_bits(w.astype(np.float32)))
    per_row = oracle.linear_w8a8(qr, sr, wq, sw_row, None)
    small = act[:, G:] @ w[:, G:].T
    assert np.all(qr[:, G:] == 0)                               # the small group vanishes per row
    np.testing.assert_allclose(per_row, exact - small, rtol=1e-12)
    assert np.abs(small).max() > 0


@pytest.mark.parametrize("name,n_out,k", [("qkv", 3 * 384, 256), ("out", 256, 384),
                                          ("fc1", 2 * 768, 256), ("fc2", 256, 768)])
@pytest.mark.parametrize("row_fc2", [0, 1])
def test_w8a8_linear_equals_float_linear_on_grid(name, n_out, k, row_fc2):
    """Activations that are s_(r,g) * q with integer q, max |q| = 127 in every
    group and s a power of two per (row, group) are bf16 values the quantizer
    maps back to themselves, so the W8A8 linear must equal the float linear
    with the dequantized weights W[o, k] = q_w[o, k] * s_w[k // G, o]."""
    dims = dataclasses.replace(TINY_W8A8, w8a8_row_fc2=row_fc2)
    G = dims.w8a8_group
    per_row = name == "fc2" and row_fc2
    r = np.random.default_rng(2)
    w = synth.make_block_weights(dims, 0, seed=3)
    qa = r.integers(-126, 127, (5, k))
    ng = 1 if per_row else k // G
    gk = k // ng
    qa[:, ::gk] = 127
    act = qa * np.repeat(2.0 ** r.integers(-12, 4, (5, ng)), gk, axis=1)
    got = oracle.linear(act, w, name, n_out, dims)
    sw = oracle.bf16_to_f64(w["s_" + name])
    if per_row:
        W = w["w_" + name].astype(np.float64) * sw[:, None]
    else:
        assert sw.shape == (k // G, n_out)
        W = w["w_" + name].astype(np.float64) * np.repeat(sw.T, G, axis=1)
    ref = act @ W.T + oracle.bf16_to_f64(w["b_" + name])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_w8a8_block_close_to_dequantized_float_block():
    """The W8A8 block differs from the float block on the dequantized weights
    (rounded to bf16) by activation quantization and that rounding: small, but present."""
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    x, tags, pos, table, _ = synth.make_inputs(wl, seed=4, n_blocks=1)
    w8 = synth.make_block_weights(TINY_W8A8, 0, seed=4)
    G = TINY_W8A8.w8a8_group
    wf = dict(w8)
    for n in ("qkv", "out", "fc1", "fc2"):
        W = w8["w_" + n].astype(np.float64) * np.repeat(oracle.bf16_to_f64(w8["s_" + n]).T, G, axis=1)
        wf["w_" + n] = synth.f32_to_bf16_bits(W.astype(np.float32))
        wf["s_" + n] = None
    y8 = oracle.block_forward(x, tags, pos, table[0], w8, TINY_W8A8)
    yf = oracle.block_forward(x, tags, pos, table[0], wf, TINY)
    d = np.linalg.norm((y8 - x) - (yf - x)) / np.linalg.norm(yf - x)
    assert 1e-4 < d < 3e-2
    # and per-group scales are closer to the float block than one scale per row of FC2
    dr = dataclasses.replace(TINY_W8A8, w8a8_row_fc2=1)
    wr = synth.make_block_weights(dr, 0, seed=4)
    yr = oracle.block_forward(x, tags, pos, table[0], wr, dr)
    assert np.linalg.norm(yr - y8) > 0

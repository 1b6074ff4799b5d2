"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test ties one oracle function to what the pages or the mathematics fix:
a library routine computing the same definition (torch CPU ops in float64),
a closed form, an invariant the method implies, brute force on tiny inputs, or
a structural statement the pages make.  Together they are chosen so that a
dropped term, a wrong sign or index, or a transposed operand fails one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from joint_video_audio_h3_amd import synth

TINY = synth.TINY_DIMS


def _rng(i=0):
    return np.random.default_rng(1234 + i)


# ------------------------------------------------------------------ attention
def test_attention_matches_torch_sdpa_fp64():
    r = _rng()
    H, N, d = 3, 37, 96
    q, k, v = (r.standard_normal((H, N, d)) for _ in range(3))
    got = oracle.attention(q, k, v, chunk=8)          # several query chunks + ragged tail
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attention_brute_force_python_loops():
    r = _rng(1)
    N, d = 5, 4
    q, k, v = (r.standard_normal((1, N, d)) for _ in range(3))
    got = oracle.attention(q, k, v)
    for i in range(N):
        s = [sum(q[0, i, t] * k[0, j, t] for t in range(d)) / math.sqrt(d) for j in range(N)]
        e = [math.exp(x) for x in s]
        z = sum(e)
        for t in range(d):
            want = sum(e[j] * v[0, j, t] for j in range(N)) / z
            assert abs(got[0, i, t] - want) < 1e-13


def test_attention_special_cases():
    r = _rng(2)
    H, N, d = 2, 9, 8
    v = r.standard_normal((H, N, d))
    # a single row attends only to itself
    one = oracle.attention(r.standard_normal((H, 1, d)), r.standard_normal((H, 1, d)), v[:, :1])
    np.testing.assert_array_equal(one, v[:, :1])
    # q = 0 -> uniform weights -> the mean of v
    out = oracle.attention(np.zeros((H, N, d)), r.standard_normal((H, N, d)), v)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=1, keepdims=True), out.shape),
                               rtol=1e-13, atol=1e-14)
    # one key far closer to the query than the rest -> that key's value
    k = np.zeros((H, N, d))
    k[:, 4, 0] = 200.0
    q = np.zeros((H, N, d))
    q[:, :, 0] = 1.0
    out = oracle.attention(q, k, v)
    np.testing.assert_allclose(out, np.broadcast_to(v[:, 4:5], out.shape), rtol=0, atol=1e-12)


def test_attention_query_subset_equals_full():
    r = _rng(3)
    q, k, v = (r.standard_normal((2, 23, 16)) for _ in range(3))
    full = oracle.attention(q, k, v)
    rows = np.array([0, 5, 22, 7])
    np.testing.assert_allclose(oracle.attention(q, k, v, rows), full[:, rows], rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ norms, activation
def test_layer_norm_matches_torch_and_closed_form():
    r = _rng(4)
    x = 3.0 * r.standard_normal((7, 256)) + 1.5
    got = oracle.layer_norm(x, 1e-6)
    ref = F.layer_norm(torch.from_numpy(x), (256,), eps=1e-6).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    var = x.var(axis=1)
    np.testing.assert_allclose(got.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(got.var(axis=1), var / (var + 1e-6), rtol=1e-12)


def test_adaln_modulate_special_cases():
    r = _rng(5)
    x = r.standard_normal((4, 64))
    sh = r.standard_normal((4, 64))
    # scale = -1 kills the normalised term: output is the shift exactly
    np.testing.assert_array_equal(oracle.adaln_modulate(x, sh, -np.ones((4, 64)), 1e-6), sh)
    # scale = 0, shift = 0 is the plain non-affine layer norm
    np.testing.assert_array_equal(oracle.adaln_modulate(x, 0 * sh, 0 * sh, 1e-6),
                                  oracle.layer_norm(x, 1e-6))


def test_rms_norm_matches_torch():
    r = _rng(6)
    v = r.standard_normal((3, 11, 128)) * 4
    g = 1 + 0.1 * r.standard_normal(128)
    got = oracle.rms_norm(v, g, 1e-6)
    ref = F.rms_norm(torch.from_numpy(v), (128,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_silu_and_swiglu():
    r = _rng(7)
    t = r.standard_normal((5, 12)) * 3
    np.testing.assert_allclose(oracle.silu(t), F.silu(torch.from_numpy(t)).numpy(), rtol=1e-13)
    z = np.concatenate([t, np.zeros_like(t)], axis=1)          # value half zero
    np.testing.assert_array_equal(oracle.swiglu(z, 12), np.zeros_like(t))
    z = np.concatenate([np.zeros_like(t), t], axis=1)          # gate half zero: silu(0) = 0
    np.testing.assert_array_equal(oracle.swiglu(z, 12), np.zeros_like(t))
    # [gate; value] order, not [value; gate]: silu(g)*v differs from g*silu(v)
    g, v = np.full((1, 1), 2.0), np.full((1, 1), -1.0)
    assert oracle.swiglu(np.concatenate([g, v], 1), 1)[0, 0] == pytest.approx(-2.0 / (1 + math.exp(-2.0)))


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("split", [(32, 48, 48), (24, 36, 36)])
def test_rope_norm_preserving_and_identity_at_zero(split):
    d = sum(split)
    r = _rng(8)
    v = r.standard_normal((2, 9, d))
    pos = r.uniform(-300, 300, (9, 3))
    ang = oracle.rope_angles(pos, split, 10000.0)
    out = oracle.apply_rope(v, ang)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-13)
    zero = oracle.apply_rope(v, oracle.rope_angles(np.zeros((9, 3)), split, 10000.0))
    np.testing.assert_array_equal(zero, v)


@pytest.mark.parametrize("split", [(32, 48, 48), (24, 36, 36)])
def test_rope_relative_position_invariance(split):
    d = sum(split)
    r = _rng(9)
    q, k = r.standard_normal((1, 1, d)), r.standard_normal((1, 1, d))
    p, pp = r.uniform(-200, 200, (1, 3)), r.uniform(-200, 200, (1, 3))
    delta = r.uniform(-200, 200, (1, 3))

    def dot(a, b):
        qa = oracle.apply_rope(q, oracle.rope_angles(a, split, 1e4))
        kb = oracle.apply_rope(k, oracle.rope_angles(b, split, 1e4))
        return float((qa * kb).sum())

    assert dot(p, pp) == pytest.approx(dot(p + delta, pp + delta), rel=1e-9, abs=1e-9)


@pytest.mark.parametrize("split", [(32, 48, 48), (24, 36, 36)])
def test_rope_axis_chunks_and_known_frequencies(split):
    """Each axis turns only its own contiguous chunk; pair 0 of a chunk turns by
    exactly the position (frequency 1) and the pair a quarter into the chunk
    turns by position/100 (10000^(-1/2))."""
    d = sum(split)
    offs = np.cumsum([0] + list(split))
    v = np.zeros((1, 1, d))
    v[..., 0::2] = 1.0                       # every pair starts at angle 0
    for axis in range(3):
        pos = np.zeros((1, 3))
        pos[0, axis] = 1.7
        out = oracle.apply_rope(v, oracle.rope_angles(pos, split, 10000.0))[0, 0]
        ang = np.arctan2(out[1::2], out[0::2])
        lo, hi = offs[axis] // 2, offs[axis + 1] // 2
        assert np.all(ang[:lo] == 0) and np.all(ang[hi:] == 0)
        assert ang[lo] == pytest.approx(1.7, rel=1e-14)
        assert ang[lo + split[axis] // 4] == pytest.approx(0.017, rel=1e-12)
        # the rotation of one pair is multiplication by exp(i * angle)
        z = (0.3 - 0.8j) * np.exp(1j * 1.7)
        w = np.zeros((1, 1, d))
        w[..., 2 * lo], w[..., 2 * lo + 1] = 0.3, -0.8
        o = oracle.apply_rope(w, oracle.rope_angles(pos, split, 10000.0))[0, 0]
        assert o[2 * lo] == pytest.approx(z.real, abs=1e-15)
        assert o[2 * lo + 1] == pytest.approx(z.imag, abs=1e-15)


# ------------------------------------------------------------------ QKV interleave
def test_qkv_split_is_per_head_interleave():
    """Rows of qkv_proj are [h0: q,k,v][h1: q,k,v]..., so the projection output
    reshapes to (..., heads, 3, head_dim) (minimax-h3-mlx README, Validation)."""
    r = _rng(10)
    H, d, N = 4, 96, 5
    u = r.standard_normal((N, 3 * H * d))
    q, k, v = oracle.qkv_split(u, H, d)
    u4 = u.reshape(N, H, 3, d)
    np.testing.assert_array_equal(q, u4[:, :, 0].transpose(1, 0, 2))
    np.testing.assert_array_equal(k, u4[:, :, 1].transpose(1, 0, 2))
    np.testing.assert_array_equal(v, u4[:, :, 2].transpose(1, 0, 2))


def test_merge_heads_layout():
    o = np.arange(2 * 3 * 4, dtype=np.float64).reshape(2, 3, 4)
    m = oracle.merge_heads(o)
    assert m.shape == (3, 8)
    np.testing.assert_array_equal(m[1, 4:8], o[1, 1])


# ------------------------------------------------------------------ bf16 / INT8
def test_round_to_bf16_matches_torch():
    r = _rng(11)
    v = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-6, 6, 20000),
                        # exact ties: 1 + 2^-8 * (odd/2) patterns
                        1.0 + (2 * np.arange(1, 200) + 1) * 2.0 ** -9])
    got = oracle.round_to_bf16(v.astype(np.float32).astype(np.float64))
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)


def test_int8_dequant_bounds_and_exactness():
    bits = synth.f32_to_bf16_bits(_rng(12).standard_normal((16, 128)).astype(np.float32) * 0.05)
    q, s_bits = synth.quantize_int8_g32(bits)
    w = oracle.bf16_to_f64(bits)
    s = np.repeat(oracle.bf16_to_f64(s_bits), 32, axis=1)
    wdq = oracle.dequant_int8_g32(q, s_bits)
    # every dequantised weight is a bf16 value
    np.testing.assert_array_equal(oracle.round_to_bf16(wdq), wdq)
    # within half a quantisation step plus half a bf16 ulp of the original
    ulp = np.ldexp(1.0, np.frexp(np.abs(wdq) + 1e-300)[1] - 8)
    assert np.all(np.abs(w - wdq) <= s / 2 + ulp / 2 + 1e-30)
    # on-grid weights come back exactly
    qq = np.arange(-127, 128, dtype=np.int8)[:128].reshape(1, 128)
    sb = synth.f32_to_bf16_bits(np.full((1, 4), 2.0 ** -7, np.float32))
    np.testing.assert_array_equal(oracle.dequant_int8_g32(qq, sb), qq.astype(np.float64) * 2.0 ** -7)


# ------------------------------------------------------------------ modulation table
def test_table_equals_live_projection_bit_exact():
    """The precomputed table drives the block exactly as the live per-row AdaLN
    projection does (minimax-h3-mlx README, AdaLN precompute: verified bit-exact)."""
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    dims = wl.dims
    x, tags, pos, _, weights = synth.make_inputs(wl, seed=3, n_blocks=1)
    r = _rng(13)
    e_dim = 32
    w_ada = synth.f32_to_bf16_bits((r.standard_normal((18 * dims.hidden, e_dim)) / 6).astype(np.float32))
    b_ada = synth.f32_to_bf16_bits((0.1 * r.standard_normal(18 * dims.hidden)).astype(np.float32))
    temb = r.standard_normal((3, e_dim)).astype(np.float32)
    table = oracle.build_mod_table(w_ada, b_ada, temb)
    table_bits = synth.f32_to_bf16_bits(table.astype(np.float32))
    np.testing.assert_array_equal(oracle.bf16_to_f64(table_bits), table)   # table is bf16-exact
    live = oracle.modulation_live(w_ada, b_ada, temb, tags)
    a = oracle.block_forward(x, tags, pos, table_bits, weights[0], dims)
    b = oracle.block_forward(x, tags, pos, None, weights[0], dims, mods=live)
    assert np.array_equal(a, b)
    # and the gather really distinguishes the tags
    assert not np.array_equal(table[0], table[1])


def test_table_gather_order():
    D = 8
    t = np.arange(3 * 6 * D, dtype=np.float32).reshape(3, 6, D)
    bits = synth.f32_to_bf16_bits(t)
    m = oracle.modulation_from_table(bits, np.array([2, 0, 1]))
    np.testing.assert_array_equal(m["gate2"][0], t[2, 5])
    np.testing.assert_array_equal(m["shift1"][1], t[0, 0])
    np.testing.assert_array_equal(m["scale2"][2], t[1, 4])


# ------------------------------------------------------------------ whole block
@pytest.fixture(scope="module")
def tiny_inputs():
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    return wl, synth.make_inputs(wl, seed=0)


def test_block_gates_zero_is_identity(tiny_inputs):
    wl, (x, tags, pos, table, weights) = tiny_inputs
    t = table[0].copy()
    t[:, 2] = 0
    t[:, 5] = 0
    out = oracle.block_forward(x, tags, pos, t, weights[0], wl.dims)
    np.testing.assert_array_equal(out, x.astype(np.float64))


def test_block_permutation_equivariance(tiny_inputs):
    wl, (x, tags, pos, table, weights) = tiny_inputs
    perm = _rng(14).permutation(len(tags))
    a = oracle.block_forward(x, tags, pos, table[0], weights[0], wl.dims)
    b = oracle.block_forward(x[perm], tags[perm], pos[perm], table[0], weights[0], wl.dims)
    np.testing.assert_allclose(b, a[perm], rtol=1e-11, atol=1e-11)


def test_block_global_position_shift_invariance(tiny_inputs):
    wl, (x, tags, pos, table, weights) = tiny_inputs
    p64 = pos.astype(np.float64)          # exact shift: no re-rounding of fractional times
    a = oracle.block_forward(x, tags, p64, table[0], weights[0], wl.dims)
    b = oracle.block_forward(x, tags, p64 + np.array([7.0, -3.0, 11.0]), table[0], weights[0], wl.dims)
    np.testing.assert_allclose(b, a, rtol=1e-10, atol=1e-10)


def test_block_single_row_attention_is_value(tiny_inputs):
    """With one row, attention returns v, so the attention branch is
    gate1 * (v W_out^T + b_out) with v taken from the interleaved projection."""
    wl, (x, tags, pos, table, weights) = tiny_inputs
    dims = wl.dims
    st = oracle.block_steps(x[:1], tags[:1], pos[:1], table[0], weights[0], dims)
    np.testing.assert_array_equal(st["o"], oracle.merge_heads(st["v"]))
    u = st["h"] @ oracle.weight(weights[0], "qkv").T + oracle.bf16_to_f64(weights[0]["b_qkv"])
    v_ref = u.reshape(1, dims.heads, 3, dims.head_dim)[:, :, 2].reshape(1, -1)
    np.testing.assert_allclose(st["o"], v_ref, rtol=0, atol=0)


def test_block_mlp_branch_reduces_to_bias_when_value_half_zero(tiny_inputs):
    wl, (x, tags, pos, table, weights) = tiny_inputs
    dims = wl.dims
    w = dict(weights[0])
    w1 = w["w_fc1"].copy()
    w1[dims.ffn:] = 0
    b1 = w["b_fc1"].copy()
    b1[dims.ffn:] = 0
    w["w_fc1"], w["b_fc1"] = w1, b1
    st = oracle.block_steps(x, tags, pos, table[0], w, dims)
    g2 = oracle.modulation_from_table(table[0], tags)["gate2"]
    np.testing.assert_allclose(st["x_out"] - st["x_mid"], g2 * oracle.bf16_to_f64(w["b_fc2"]),
                               rtol=0, atol=1e-15)


def test_block_query_subset_matches_full(tiny_inputs):
    wl, (x, tags, pos, table, weights) = tiny_inputs
    full = oracle.block_forward(x, tags, pos, table[0], weights[0], wl.dims)
    rows = np.array([0, 17, 40, 163])
    # same values; only the BLAS summation order differs for a different matrix shape
    np.testing.assert_allclose(oracle.block_forward(x, tags, pos, table[0], weights[0], wl.dims, rows),
                               full[rows], rtol=1e-12, atol=1e-12)


def test_block_against_torch_module_composition(tiny_inputs):
    """An independent float64 composition from torch library ops (layer_norm,
    rms_norm, scaled_dot_product_attention, silu, linear), assembled from the
    pages' statements: interleaved QKV reshaped to (heads, 3, d), rotary as a
    complex multiply per pair, fc2(silu(gate) * value)."""
    wl, (x, tags, pos, table, weights) = tiny_inputs
    dims = wl.dims
    w = weights[0]
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    D, H, d, Fd = dims.hidden, dims.heads, dims.head_dim, dims.ffn
    tb = T(oracle.bf16_to_f64(table[0]))[torch.from_numpy(tags.astype(np.int64))]
    xt = T(x)
    lin = lambda v, n: F.linear(v, T(oracle.weight(w, n)), T(oracle.bf16_to_f64(w["b_" + n])))
    h = F.layer_norm(xt, (D,), eps=1e-6) * (1 + tb[:, 1]) + tb[:, 0]
    u = lin(h, "qkv").view(-1, H, 3, d)
    q = F.rms_norm(u[:, :, 0], (d,), weight=T(oracle.bf16_to_f64(w["q_norm"])), eps=1e-6)
    k = F.rms_norm(u[:, :, 1], (d,), weight=T(oracle.bf16_to_f64(w["k_norm"])), eps=1e-6)
    vv = u[:, :, 2]
    # rotary as complex multiply: pair j of chunk a turns by pos_a * 10000^(-2j/d_a)
    angs = []
    for a, da in enumerate(dims.rope_split):
        inv = torch.pow(torch.tensor(10000.0, dtype=torch.float64),
                        -torch.arange(0, da, 2, dtype=torch.float64) / da)
        angs.append(T(pos[:, a:a + 1]) * inv[None])
    rot = torch.polar(torch.ones(1, dtype=torch.float64), torch.cat(angs, 1))[:, None, :]
    cq = torch.view_as_real(torch.view_as_complex(q.reshape(-1, H, d // 2, 2).contiguous()) * rot).reshape(-1, H, d)
    ck = torch.view_as_real(torch.view_as_complex(k.reshape(-1, H, d // 2, 2).contiguous()) * rot).reshape(-1, H, d)
    o = F.scaled_dot_product_attention(cq.transpose(0, 1), ck.transpose(0, 1), vv.transpose(0, 1).contiguous())
    o = o.transpose(0, 1).reshape(-1, H * d)
    x1 = xt + tb[:, 2] * lin(o, "out")
    h2 = F.layer_norm(x1, (D,), eps=1e-6) * (1 + tb[:, 4]) + tb[:, 3]
    z = lin(h2, "fc1")
    ref = x1 + tb[:, 5] * lin(F.silu(z[:, :Fd]) * z[:, Fd:], "fc2")
    got = oracle.block_forward(x, tags, pos, table[0], w, dims)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-10)


def test_dit_forward_gates_zero_depth_identity(tiny_inputs):
    wl, (x, tags, pos, table, weights) = tiny_inputs
    t = table.copy()
    t[:, :, 2] = 0
    t[:, :, 5] = 0
    out = oracle.dit_forward(x, tags, pos, t, lambda b: weights[b], 2, wl.dims)
    np.testing.assert_array_equal(out, x.astype(np.float64))


@pytest.mark.parametrize("live", [0, 1])
def test_dit_forward_runs_each_block_with_its_own_table_and_weights(tiny_inputs, live):
    """With every residual gate of one block zero, that block is the identity
    (bit for bit), so the 2-block forward equals the other block alone, with
    that block's own table slice and weights.  A forward that used block 0's
    table or weights for every block, or the blocks in the wrong order, fails."""
    wl, (x, tags, pos, table, weights) = tiny_inputs
    dead = 1 - live
    t = table.copy()
    t[dead, :, 2] = 0
    t[dead, :, 5] = 0
    out = oracle.dit_forward(x, tags, pos, t, lambda b: weights[b], 2, wl.dims)
    alone = oracle.block_forward(x, tags, pos, table[live], weights[live], wl.dims)
    np.testing.assert_array_equal(out, alone)
    # and the two blocks really differ: the other block alone gives another answer
    other = oracle.block_forward(x, tags, pos, table[dead], weights[dead], wl.dims)
    assert np.abs(other - alone).max() > 1e-2

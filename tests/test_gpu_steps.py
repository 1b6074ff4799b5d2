"""Per-step parity of the HIP kernels against the float64 oracle (GPU).

Every step is fed stand-alone synthetic inputs from the generator (never a
value produced by the HIP path), run through the C ABI, and compared with the
oracle's definition of that step.  Row counts cover several tiles, ragged
tails and the single-row edge case; the H3-width cases use the real shapes.
"""
import numpy as np
import pytest
import torch

import oracle
from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import (TOL_ATTN, TOL_BF16_OUT, TOL_RESID_DELTA, dev, host_bf16, rel_l2,
                            say)

pytestmark = pytest.mark.gpu

CASES = [("tiny", synth.TINY_DIMS, 1), ("tiny", synth.TINY_DIMS, 164), ("tiny", synth.TINY_DIMS, 300),
         ("h3", synth.H3_DIMS, 1192), ("h3", synth.H3_DIMS, 257)]
IDS = [f"{n}-N{r}" for n, _, r in CASES]
INT8_H3 = synth.WORKLOADS["h3_1blk_n1192_int8"].dims
INT8_TINY = synth.Dims(**{**synth.TINY_DIMS.__dict__, "wfmt": synth.WFMT_INT8_G32})


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


_WCACHE = {}


def _weights(dims, seed=0):
    key = (dims, seed)
    if key not in _WCACHE:
        _WCACHE.clear()
        host = synth.make_block_weights(dims, 0, seed)
        _WCACHE[key] = (host, lib.to_device_block(host))
    return _WCACHE[key]


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
def test_rope_table(name, dims, n):
    say("rope_table", name, n)
    pos = synth.make_positions(n, seed=1)
    np_ = lib.padded_rows(n)
    cs = torch.empty(np_, dims.head_dim // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table(dims, dev(pos), n, cs)
    torch.cuda.synchronize()
    ang = oracle.rope_angles(pos, dims.rope_split, dims.rope_theta)
    got = cs.cpu().numpy().astype(np.float64)
    assert np.abs(got[:n, :, 0] - np.cos(ang)).max() < 2e-7
    assert np.abs(got[:n, :, 1] - np.sin(ang)).max() < 2e-7
    assert np.all(got[n:, :, 0] == 1) and np.all(got[n:, :, 1] == 0)


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
@pytest.mark.parametrize("which", [0, 1])
def test_adaln_modulate(name, dims, n, which):
    say("adaln", name, n, which)
    x = synth.make_x(n, dims, seed=2) * np.float32(1.7) + np.float32(0.3)
    tags = synth.make_tags(n, dims.n_tags, seed=2)
    table = synth.make_table(dims, 1, seed=2)[0]
    h = torch.empty(n, dims.hidden, dtype=torch.int16, device="cuda")
    lib.adaln_modulate(dims, dev(x), dev(tags), dev(table), which, h)
    torch.cuda.synchronize()
    m = oracle.modulation_from_table(table, tags)
    sfx = "1" if which == 0 else "2"
    ref = oracle.adaln_modulate(x, m["shift" + sfx], m["scale" + sfx], dims.ln_eps)
    got = host_bf16(h)
    assert rel_l2(got, ref) < TOL_BF16_OUT
    # every element within one bf16 rounding (+ fp32 statistics noise) of the exact value
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)


def _qkv_case(dims, n, seed=3):
    host, devw = _weights(dims)
    h = synth.make_activation_bf16(n, dims.hidden, "h", seed=seed)
    pos = synth.make_positions(n, seed=seed)
    np_ = lib.padded_rows(n)
    H, d = dims.heads, dims.head_dim
    cs = torch.empty(np_, d // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table(dims, dev(pos), n, cs)
    q = torch.full((H, np_, d), 0x7FC0, dtype=torch.int16, device="cuda")   # NaN-filled: pads must be overwritten
    k = torch.full_like(q, 0x7FC0)
    vt = torch.full((H, d, np_), 0x7FC0, dtype=torch.int16, device="cuda")
    lib.qkv_rope(dims, dev(h), devw, cs, n, q, k, vt)
    torch.cuda.synchronize()
    return host, h, pos, host_bf16(q), host_bf16(k), host_bf16(vt)


def _qkv_ref(dims, host, h, pos, rows=None):
    hh = oracle.bf16_to_f64(h) if rows is None else oracle.bf16_to_f64(h[rows])
    p = pos if rows is None else pos[rows]
    u = hh @ oracle.weight(host, "qkv").T + oracle.bias(host, "qkv", 3 * dims.inner)
    q, k, v = oracle.qkv_split(u, dims.heads, dims.head_dim)
    ang = oracle.rope_angles(p, dims.rope_split, dims.rope_theta)
    gq, gk = oracle.bf16_to_f64(host["q_norm"]), oracle.bf16_to_f64(host["k_norm"])
    q = oracle.apply_rope(oracle.rms_norm(q, gq, dims.qk_eps), ang)
    k = oracle.apply_rope(oracle.rms_norm(k, gk, dims.qk_eps), ang)
    return q, k, v


@pytest.mark.parametrize("name,dims,n", CASES + [("tiny8", INT8_TINY, 300), ("h3-int8", INT8_H3, 1192)],
                         ids=IDS + ["tiny-int8-N300", "h3-int8-N1192"])
def test_qkv_rope(name, dims, n):
    say("qkv_rope", name, n)
    host, h, pos, q, k, vt = _qkv_case(dims, n)
    rq, rk, rv = _qkv_ref(dims, host, h, pos)
    qs = np.log2(np.e) / np.sqrt(dims.head_dim)
    assert rel_l2(q[:, :n] / qs, rq) < TOL_BF16_OUT
    assert rel_l2(k[:, :n], rk) < TOL_BF16_OUT
    assert rel_l2(vt[:, :, :n].transpose(0, 2, 1), rv) < TOL_BF16_OUT
    # per head, not just overall
    for hd in range(dims.heads):
        assert rel_l2(k[hd, :n], rk[hd]) < 2 * TOL_BF16_OUT
    assert np.all(q[:, n:] == 0) and np.all(k[:, n:] == 0) and np.all(vt[:, :, n:] == 0)


def _attn_inputs(dims, n, seed=4):
    H, d = dims.heads, dims.head_dim
    np_ = lib.padded_rows(n)
    qs = np.log2(np.e) / np.sqrt(d)
    q = synth.make_activation_bf16(H * n, d, "q", seed, std=qs).reshape(H, n, d)
    k = synth.make_activation_bf16(H * n, d, "k", seed).reshape(H, n, d)
    v = synth.make_activation_bf16(H * n, d, "v", seed).reshape(H, n, d)
    pad = lambda a: np.concatenate([a, np.zeros((H, np_ - n, d), np.uint16)], axis=1)
    return q, k, v, pad(q), pad(k), np.ascontiguousarray(pad(v).transpose(0, 2, 1))


# at head_dim 128 a block takes 384 queries (48 per wavefront) and n_pad is a
# multiple of 256: 383 / 384 / 385 sit at a block edge (385: a second block
# with one query), and at 769 the last block's rows 1,024 .. 1,151 lie past
# n_pad, so those queries read a clamped row and store nothing
@pytest.mark.parametrize("name,dims,n", CASES + [("h3", synth.H3_DIMS, n) for n in (1, 65, 383, 384, 385, 769)],
                         ids=IDS + [f"h3-N{n}" for n in (1, 65, 383, 384, 385, 769)])
def test_attention(name, dims, n):
    say("attention", name, n)
    q, k, v, qp, kp, vtp = _attn_inputs(dims, n)
    o = torch.empty(n, dims.inner, dtype=torch.int16, device="cuda")
    lib.attention(dims, dev(qp), dev(kp), dev(vtp), n, o)
    torch.cuda.synchronize()
    qs = np.log2(np.e) / np.sqrt(dims.head_dim)
    ref = oracle.merge_heads(oracle.attention(oracle.bf16_to_f64(q) / qs, oracle.bf16_to_f64(k),
                                              oracle.bf16_to_f64(v)))
    got = host_bf16(o)
    assert rel_l2(got, ref) < TOL_ATTN
    # every query row on its own (a row the kernel skipped or wrote for another
    # query would fail here even when the whole-matrix error is small)
    per_row = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    assert float(per_row.max()) < 4 * TOL_ATTN
    if n == 1:   # a single row attends only to itself: o = v up to the bf16 store
        np.testing.assert_array_equal(got, oracle.merge_heads(oracle.bf16_to_f64(v)))


def _resid_case(dims, n, which, seed=5):
    host, devw = _weights(dims)
    K = dims.inner if which == "out" else dims.ffn
    a = synth.make_activation_bf16(n, K, "o" if which == "out" else "a", seed,
                                   std=0.3 if which == "out" else 0.5)
    x = synth.make_x(n, dims, seed)
    tags = synth.make_tags(n, dims.n_tags, seed)
    table = synth.make_table(dims, 1, seed)[0]
    xd = dev(x)
    if which == "out":
        lib.out_proj_residual(dims, dev(a), devw, dev(table), dev(tags), xd)
    else:
        lib.mlp_fc2_residual(dims, dev(a), devw, dev(table), dev(tags), xd)
    torch.cuda.synchronize()
    g = oracle.modulation_from_table(table, tags)["gate1" if which == "out" else "gate2"]
    name = "out" if which == "out" else "fc2"
    delta = g * (oracle.bf16_to_f64(a) @ oracle.weight(host, name).T
                 + oracle.bias(host, name, dims.hidden))
    return xd.cpu().numpy().astype(np.float64) - x, delta


@pytest.mark.parametrize("name,dims,n", CASES + [("h3-int8", INT8_H3, 1192)], ids=IDS + ["h3-int8-N1192"])
@pytest.mark.parametrize("which", ["out", "fc2"])
def test_gated_residual(name, dims, n, which):
    say("gated_residual", which, name, n)
    got, ref = _resid_case(dims, n, which)
    assert rel_l2(got, ref) < TOL_RESID_DELTA


@pytest.mark.parametrize("name,dims,n", CASES + [("tiny8", INT8_TINY, 164), ("h3-int8", INT8_H3, 1192)],
                         ids=IDS + ["tiny-int8-N164", "h3-int8-N1192"])
def test_fc1_swiglu(name, dims, n):
    say("fc1_swiglu", name, n)
    host, devw = _weights(dims)
    h2 = synth.make_activation_bf16(n, dims.hidden, "h", seed=6)
    a = torch.empty(n, dims.ffn, dtype=torch.int16, device="cuda")
    lib.mlp_fc1_swiglu(dims, dev(h2), devw, a)
    torch.cuda.synchronize()
    z = oracle.bf16_to_f64(h2) @ oracle.weight(host, "fc1").T + oracle.bias(host, "fc1", 2 * dims.ffn)
    assert rel_l2(host_bf16(a), oracle.swiglu(z, dims.ffn)) < TOL_BF16_OUT

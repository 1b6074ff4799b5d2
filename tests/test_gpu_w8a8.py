"""Parity of the W8A8 trunk (int8 weights and activations) against the oracle (GPU).

* the row quantizer: codes and scales bit for bit on generator bf16 rows;
* the quantizing AdaLN: its codes dequantize to the oracle's h within half a
  code step plus the bf16 rounding of h, and they equal the oracle's quantizer
  on the oracle's bf16 h except where the two h values round apart;
* each int8 GEMM step on activations the oracle quantized: the integer sums are
  exact on both sides, so only fp32 scaling and the bf16 outputs differ;
* the whole W8A8 block and a 2-block depth against the oracle's W8A8 block.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import (TOL_BF16_OUT, TOL_BLOCK, TOL_DEPTH, TOL_RESID_DELTA, dev, host_bf16,
                            rel_l2, say)

pytestmark = pytest.mark.gpu

W8_TINY = dataclasses.replace(synth.TINY_DIMS, wfmt=synth.WFMT_W8A8)
W8_H3 = dataclasses.replace(synth.H3_DIMS, wfmt=synth.WFMT_W8A8)
CASES = [("tiny", W8_TINY, 1), ("tiny", W8_TINY, 164), ("tiny", W8_TINY, 300), ("h3", W8_H3, 1),
         ("h3", W8_H3, 257), ("h3", W8_H3, 1192)]
IDS = [f"{n}-N{r}" for n, _, r in CASES]


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


def _qa_buffer(q, s):
    """W8A8 activation buffer (codes, then fp32 scales at roundup(n*K, 256)) from host arrays."""
    n, K = q.shape
    buf = np.zeros(lib.quantized_bytes(n, K), np.uint8)
    buf[:n * K] = q.reshape(-1).view(np.uint8)
    off = (n * K + 255) // 256 * 256
    buf[off:off + 4 * n] = np.asarray(s, np.float32).view(np.uint8)
    return dev(buf)


def _read_qa(buf, n, K):
    b = buf.cpu().numpy()
    off = (n * K + 255) // 256 * 256
    return b[:n * K].view(np.int8).reshape(n, K), b[off:off + 4 * n].view(np.float32)


@pytest.mark.parametrize("n,K", [(1, 384), (77, 768), (300, 7168), (129, 14336), (5, 5376)])
def test_quantize_rows_bit_exact(n, K):
    say("quantize_rows", n, K)
    a = synth.make_activation_bf16(n, K, "a", seed=11, std=0.7)
    a[0, :] = 0                                        # an all-zero row: codes 0, scale 0
    buf = torch.zeros(lib.quantized_bytes(n, K), dtype=torch.uint8, device="cuda")
    lib.quantize_rows(dev(a), buf)
    torch.cuda.synchronize()
    q, s = _read_qa(buf, n, K)
    rq, rs = oracle.quantize_rows(oracle.bf16_to_f64(a))
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
def test_adaln_quantized(name, dims, n):
    say("adaln w8a8", name, n)
    x = synth.make_x(n, dims, seed=12) * np.float32(1.3) - np.float32(0.2)
    tags = synth.make_tags(n, dims.n_tags, seed=12)
    table = synth.make_table(dims, 1, seed=12)[0]
    buf = torch.zeros(lib.quantized_bytes(n, dims.hidden), dtype=torch.uint8, device="cuda")
    lib.adaln_modulate(dims, dev(x), dev(tags), dev(table), 1, buf)
    torch.cuda.synchronize()
    q, s = _read_qa(buf, n, dims.hidden)
    m = oracle.modulation_from_table(table, tags)
    h = oracle.adaln_modulate(x, m["shift2"], m["scale2"], dims.ln_eps)
    hb = oracle.round_to_bf16(h)
    deq = q.astype(np.float64) * s[:, None]
    assert np.all(np.abs(deq - h) <= s[:, None] * 0.5 * (1 + 2.0 ** -16) + np.abs(h) * 2.0 ** -8 + 1e-6)
    rq, rs = oracle.quantize_rows(hb)
    np.testing.assert_allclose(s, rs, rtol=2.0 ** -7)
    diff = q.astype(np.int32) - rq
    assert np.abs(diff).max() <= 1 and np.mean(diff != 0) < 2e-3


def _oracle_qa(a_bits):
    return oracle.quantize_rows(oracle.bf16_to_f64(a_bits))


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
def test_qkv_rope_w8a8(name, dims, n):
    say("qkv w8a8", name, n)
    host, devw = _weights(dims)
    h = synth.make_activation_bf16(n, dims.hidden, "h", seed=13)
    qh, sh = _oracle_qa(h)
    pos = synth.make_positions(n, seed=13)
    np_ = lib.padded_rows(n)
    H, d = dims.heads, dims.head_dim
    cs = torch.empty(np_, d // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table(dims, dev(pos), n, cs)
    q = torch.full((H, np_, d), 0x7FC0, dtype=torch.int16, device="cuda")
    k = torch.full_like(q, 0x7FC0)
    vt = torch.full((H, d, np_), 0x7FC0, dtype=torch.int16, device="cuda")
    lib.qkv_rope(dims, _qa_buffer(qh, sh), devw, cs, n, q, k, vt)
    torch.cuda.synchronize()
    u = oracle.linear_w8a8(qh, sh, host["w_qkv"], host["s_qkv"], oracle.bias(host, "qkv", 3 * dims.inner))
    rq, rk, rv = oracle.qkv_split(u, H, d)
    ang = oracle.rope_angles(pos, dims.rope_split, dims.rope_theta)
    gq, gk = oracle.bf16_to_f64(host["q_norm"]), oracle.bf16_to_f64(host["k_norm"])
    rq = oracle.apply_rope(oracle.rms_norm(rq, gq, dims.qk_eps), ang)
    rk = oracle.apply_rope(oracle.rms_norm(rk, gk, dims.qk_eps), ang)
    qs = np.log2(np.e) / np.sqrt(d)
    gq_, gk_, gv_ = host_bf16(q), host_bf16(k), host_bf16(vt)
    assert rel_l2(gq_[:, :n] / qs, rq) < TOL_BF16_OUT
    assert rel_l2(gk_[:, :n], rk) < TOL_BF16_OUT
    assert rel_l2(gv_[:, :, :n].transpose(0, 2, 1), rv) < TOL_BF16_OUT
    assert np.all(gq_[:, n:] == 0) and np.all(gk_[:, n:] == 0) and np.all(gv_[:, :, n:] == 0)


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
@pytest.mark.parametrize("which", ["out", "fc2"])
def test_gated_residual_w8a8(name, dims, n, which):
    say("residual w8a8", which, name, n)
    host, devw = _weights(dims)
    K = dims.inner if which == "out" else dims.ffn
    a = synth.make_activation_bf16(n, K, "o" if which == "out" else "a", 14, std=0.4)
    qa, sa = _oracle_qa(a)
    x = synth.make_x(n, dims, 14)
    tags = synth.make_tags(n, dims.n_tags, 14)
    table = synth.make_table(dims, 1, 14)[0]
    xd = dev(x)
    fn = lib.out_proj_residual if which == "out" else lib.mlp_fc2_residual
    fn(dims, _qa_buffer(qa, sa), devw, dev(table), dev(tags), xd)
    torch.cuda.synchronize()
    g = oracle.modulation_from_table(table, tags)["gate1" if which == "out" else "gate2"]
    nm = "out" if which == "out" else "fc2"
    ref = g * oracle.linear_w8a8(qa, sa, host["w_" + nm], host["s_" + nm], oracle.bias(host, nm, dims.hidden))
    assert rel_l2(xd.cpu().numpy().astype(np.float64) - x, ref) < TOL_RESID_DELTA


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
def test_fc1_swiglu_w8a8(name, dims, n):
    say("fc1 w8a8", name, n)
    host, devw = _weights(dims)
    h2 = synth.make_activation_bf16(n, dims.hidden, "h", seed=15)
    qh, sh = _oracle_qa(h2)
    a = torch.empty(n, dims.ffn, dtype=torch.int16, device="cuda")
    lib.mlp_fc1_swiglu(dims, _qa_buffer(qh, sh), devw, a)
    torch.cuda.synchronize()
    z = oracle.linear_w8a8(qh, sh, host["w_fc1"], host["s_fc1"], oracle.bias(host, "fc1", 2 * dims.ffn))
    assert rel_l2(host_bf16(a), oracle.swiglu(z, dims.ffn)) < TOL_BF16_OUT


BLOCK_CASES = [("tiny_2blk_n164", 1, TOL_BLOCK), ("tiny_2blk_n164", 2, TOL_DEPTH), ("h3_1blk_n1192", 1, TOL_BLOCK)]


@pytest.mark.parametrize("wname,nb,tol", BLOCK_CASES, ids=[f"{w}-{b}blk" for w, b, _ in BLOCK_CASES])
def test_w8a8_forward_matches_oracle(wname, nb, tol):
    say("w8a8 forward", wname, nb)
    base = synth.WORKLOADS[wname]
    wl = dataclasses.replace(base, dims=dataclasses.replace(base.dims, wfmt=synth.WFMT_W8A8))
    x, tags, pos, table, blocks = synth.make_inputs(wl, seed=16, n_blocks=nb)
    xd = dev(x)
    ws = lib.alloc_workspace(wl.dims, wl.n_rows)
    lib.dit_forward(wl.dims, xd, dev(tags), dev(pos), dev(table), [lib.to_device_block(b) for b in blocks], ws)
    torch.cuda.synchronize()
    ref = oracle.dit_forward(x, tags, pos, table, lambda b: blocks[b], nb, wl.dims)
    got = xd.cpu().numpy().astype(np.float64)
    e_out, e_delta = rel_l2(got, ref), rel_l2(got - x, ref - x)
    say("w8a8 rel-L2 x_out", e_out, "update", e_delta)
    assert e_out < tol and e_delta < 2 * tol


def test_fullsize_w8a8_block_n6437_sampled_rows():
    """One W8A8 block at N = 6,437 (the 50-block workload's packed layout), in
    the launch configuration of the forward, compared on sampled output rows;
    keys and values use every row (quantization is per row, so the oracle's
    sampled rows see exactly the rows the GPU computed them from)."""
    wl = synth.WORKLOADS["h3_50blk_n6437_w8a8"]
    say("fullsize w8a8 block", wl.n_rows)
    host = synth.make_block_weights(wl.dims, 0, seed=17)
    tags, pos = synth.packed_layout(wl)
    x = synth.make_x(wl, wl.dims, seed=17)
    table = synth.make_table(wl.dims, 1, seed=17)
    xd = dev(x)
    ws = lib.alloc_workspace(wl.dims, wl.n_rows)
    lib.dit_block_forward(wl.dims, xd, dev(tags), dev(pos), dev(table[0]), lib.to_device_block(host), ws)
    torch.cuda.synchronize()
    r = np.random.default_rng(5).choice(wl.n_rows, size=21, replace=False)
    rows = np.unique(np.concatenate([r, [0, wl.n_rows // 2, wl.n_rows - 1]]))
    got = xd.cpu().numpy().astype(np.float64)[rows]
    ref = oracle.block_forward(x, tags, pos, table[0], host, wl.dims, q_rows=rows)
    xr = x[rows].astype(np.float64)
    say("fullsize w8a8 rel-L2", rel_l2(got, ref), rel_l2(got - xr, ref - xr))
    assert rel_l2(got, ref) < TOL_BLOCK
    assert rel_l2(got - xr, ref - xr) < 2 * TOL_BLOCK

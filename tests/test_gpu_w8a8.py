"""Parity of the group-scaled W8A8 trunk (int8 weights and activations, one
scale per group of K elements on both operands) against the oracle (GPU).

* the group quantizer: codes and scales bit for bit on generator bf16 rows, for
  every accepted group size and for one scale per row (FC2's per-row form),
  with all-zero rows and groups, and zero scales on the padded rows;
* each int8 GEMM step on activations the oracle quantized: the integer sums are
  exact on both sides, so only fp32 scaling, folding order and the bf16
  outputs differ;
* the whole W8A8 block and a 2-block depth against the oracle's W8A8 block,
  with the pages' group 896, the other accepted groups, and per-row FC2; one
  W8A8 block at N = 6,437 and at N = 49,840 on sampled output rows.
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

W8_TINY = synth.TINY_W8A8_DIMS                      # group 64 (the tiny widths allow no other)
W8_H3 = synth.H3_W8A8_DIMS                          # group 896
W8_H3_ROWFC2 = dataclasses.replace(W8_H3, w8a8_row_fc2=1)
CASES = [("tiny", W8_TINY, 1), ("tiny", W8_TINY, 164), ("tiny", W8_TINY, 300), ("h3", W8_H3, 1),
         ("h3", W8_H3, 257), ("h3", W8_H3, 1192),
         ("h3-g64", dataclasses.replace(W8_H3, w8a8_group=64), 300),
         ("h3-g256", dataclasses.replace(W8_H3, w8a8_group=256), 300),
         ("h3-g448", dataclasses.replace(W8_H3, w8a8_group=448), 777)]
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


def _group(dims, K, fc2=False):
    return K if (fc2 and dims.w8a8_row_fc2) else dims.w8a8_group


def _qa_buffer(q, s, group):
    """W8A8 activation buffer from host codes [n, K] and scales [n, K/group]:
    codes, then fp32 scales [K/group][n_pad] at roundup(n*K, 256)."""
    n, K = q.shape
    np_ = lib.padded_rows(n)
    buf = np.zeros(lib.quantized_bytes(n, K, group), np.uint8)
    buf[:n * K] = q.reshape(-1).view(np.uint8)
    off = (n * K + 255) // 256 * 256
    st = np.zeros((K // group, np_), np.float32)
    st[:, :n] = np.asarray(s, np.float32).reshape(n, K // group).T
    buf[off:off + st.nbytes] = st.reshape(-1).view(np.uint8)
    return dev(buf)


def _read_qa(buf, n, K, group):
    b = buf.cpu().numpy()
    np_ = lib.padded_rows(n)
    off = (n * K + 255) // 256 * 256
    st = b[off:off + 4 * (K // group) * np_].view(np.float32).reshape(K // group, np_)
    return b[:n * K].view(np.int8).reshape(n, K), st


def _oracle_qa(a_bits, group):
    a = oracle.bf16_to_f64(a_bits)
    if group == a.shape[1]:
        q, s = oracle.quantize_rows(a)
        return q, s[:, None]
    return oracle.quantize_groups(a, group)


@pytest.mark.parametrize("n,K,group", [(1, 384, 64), (77, 768, 64), (300, 7168, 896), (129, 14336, 448),
                                       (5, 5376, 256), (300, 5376, 896), (64, 14336, 64), (3, 7168, 7168),
                                       (77, 14336, 14336)])
def test_quantize_groups_bit_exact(n, K, group):
    say("quantize_groups", n, K, group)
    a = synth.make_activation_bf16(n, K, "a", seed=11, std=0.7)
    a[0, :] = 0                                        # an all-zero row: codes 0, scales 0
    if n > 1:
        a[n - 1, :group] = 0                           # an all-zero first group
    buf = torch.full((lib.quantized_bytes(n, K, group),), 0x55, dtype=torch.uint8, device="cuda")
    lib.quantize_groups(dev(a), group, buf)
    torch.cuda.synchronize()
    q, st = _read_qa(buf, n, K, group)
    rq, rs = _oracle_qa(a, group)
    np.testing.assert_array_equal(st[:, :n].T, rs)
    np.testing.assert_array_equal(st[:, n:], 0)        # padded rows hold 0
    np.testing.assert_array_equal(q, rq)


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
def test_qkv_rope_w8a8(name, dims, n):
    say("qkv w8a8", name, n)
    host, devw = _weights(dims)
    h = synth.make_activation_bf16(n, dims.hidden, "h", seed=13)
    G = _group(dims, dims.hidden)
    qh, sh = _oracle_qa(h, G)
    pos = synth.make_positions(n, seed=13)
    np_ = lib.padded_rows(n)
    H, d = dims.heads, dims.head_dim
    cs = torch.empty(np_, d // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table(dims, dev(pos), n, cs)
    q = torch.full((H, np_, d), 0x7FC0, dtype=torch.int16, device="cuda")
    k = torch.full_like(q, 0x7FC0)
    vt = torch.full((H, d, np_), 0x7FC0, dtype=torch.int16, device="cuda")
    lib.qkv_rope(dims, _qa_buffer(qh, sh, G), devw, cs, n, q, k, vt)
    torch.cuda.synchronize()
    u = oracle.linear_w8a8_grouped(qh, sh, host["w_qkv"], host["s_qkv"], oracle.bias(host, "qkv", 3 * dims.inner), G)
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


@pytest.mark.parametrize("name,dims,n", CASES + [("h3-rowfc2", W8_H3_ROWFC2, 300)],
                         ids=IDS + ["h3-rowfc2-N300"])
@pytest.mark.parametrize("which", ["out", "fc2"])
def test_gated_residual_w8a8(name, dims, n, which):
    say("residual w8a8", which, name, n)
    host, devw = _weights(dims)
    K = dims.inner if which == "out" else dims.ffn
    G = _group(dims, K, which == "fc2")
    a = synth.make_activation_bf16(n, K, "o" if which == "out" else "a", 14, std=0.4)
    qa, sa = _oracle_qa(a, G)
    x = synth.make_x(n, dims, 14)
    tags = synth.make_tags(n, dims.n_tags, 14)
    table = synth.make_table(dims, 1, 14)[0]
    xd = dev(x)
    fn = lib.out_proj_residual if which == "out" else lib.mlp_fc2_residual
    fn(dims, _qa_buffer(qa, sa, G), devw, dev(table), dev(tags), xd)
    torch.cuda.synchronize()
    g = oracle.modulation_from_table(table, tags)["gate1" if which == "out" else "gate2"]
    nm = "out" if which == "out" else "fc2"
    b = oracle.bias(host, nm, dims.hidden)
    if G == K:
        y = oracle.linear_w8a8(qa, sa[:, 0], host["w_" + nm], host["s_" + nm], b)
    else:
        y = oracle.linear_w8a8_grouped(qa, sa, host["w_" + nm], host["s_" + nm], b, G)
    assert rel_l2(xd.cpu().numpy().astype(np.float64) - x, g * y) < TOL_RESID_DELTA


@pytest.mark.parametrize("name,dims,n", CASES, ids=IDS)
def test_fc1_swiglu_w8a8(name, dims, n):
    say("fc1 w8a8", name, n)
    host, devw = _weights(dims)
    h2 = synth.make_activation_bf16(n, dims.hidden, "h", seed=15)
    G = _group(dims, dims.hidden)
    qh, sh = _oracle_qa(h2, G)
    a = torch.empty(n, dims.ffn, dtype=torch.int16, device="cuda")
    lib.mlp_fc1_swiglu(dims, _qa_buffer(qh, sh, G), devw, a)
    torch.cuda.synchronize()
    z = oracle.linear_w8a8_grouped(qh, sh, host["w_fc1"], host["s_fc1"], oracle.bias(host, "fc1", 2 * dims.ffn), G)
    assert rel_l2(host_bf16(a), oracle.swiglu(z, dims.ffn)) < TOL_BF16_OUT


BLOCK_CASES = [("tiny_2blk_n164", W8_TINY, 1, TOL_BLOCK), ("tiny_2blk_n164", W8_TINY, 2, TOL_DEPTH),
               ("h3_1blk_n1192", W8_H3, 1, TOL_BLOCK),
               ("h3_1blk_n1192", dataclasses.replace(W8_H3, w8a8_group=448), 1, TOL_BLOCK),
               ("h3_1blk_n1192", W8_H3_ROWFC2, 1, TOL_BLOCK)]


@pytest.mark.parametrize("wname,dims,nb,tol", BLOCK_CASES,
                         ids=["tiny-g64-1blk", "tiny-g64-2blk", "h3-g896-1blk", "h3-g448-1blk", "h3-rowfc2-1blk"])
def test_w8a8_forward_matches_oracle(wname, dims, nb, tol):
    say("w8a8 forward", wname, dims.w8a8_group, dims.w8a8_row_fc2, nb)
    wl = dataclasses.replace(synth.WORKLOADS[wname], dims=dims)
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


@pytest.mark.parametrize("wname", ["h3_50blk_n6437_w8a8", "h3_50blk_n49840_w8a8"])
def test_fullsize_w8a8_block_sampled_rows(wname):
    """One W8A8 block at the 50-block workloads' packed layouts (N = 6,437 and
    49,840), in the launch configuration of the forward, compared on sampled
    output rows; keys and values use every row (activations are quantized per
    row and group, so the oracle's sampled rows see exactly the rows the GPU
    computed them from)."""
    wl = synth.WORKLOADS[wname]
    say("fullsize w8a8 block", wl.n_rows)
    host = synth.make_block_weights(wl.dims, 0, seed=17)
    tags, pos = synth.packed_layout(wl)
    x = synth.make_x(wl, wl.dims, seed=17)
    table = synth.make_table(wl.dims, 1, seed=17)
    xd = dev(x)
    ws = lib.alloc_workspace(wl.dims, wl.n_rows)
    lib.dit_block_forward(wl.dims, xd, dev(tags), dev(pos), dev(table[0]), lib.to_device_block(host), ws)
    torch.cuda.synchronize()
    del ws
    r = np.random.default_rng(5).choice(wl.n_rows, size=21 if wl.n_rows < 10000 else 13, replace=False)
    rows = np.unique(np.concatenate([r, [0, wl.n_rows // 2, wl.n_rows - 1]]))
    got = xd.cpu().numpy().astype(np.float64)[rows]
    say("fullsize w8a8 block: oracle on", len(rows), "rows")
    ref = oracle.block_forward(x, tags, pos, table[0], host, wl.dims, q_rows=rows)
    xr = x[rows].astype(np.float64)
    say("fullsize w8a8 rel-L2", rel_l2(got, ref), rel_l2(got - xr, ref - xr))
    assert rel_l2(got, ref) < TOL_BLOCK
    assert rel_l2(got - xr, ref - xr) < 2 * TOL_BLOCK


def test_per_row_fc2_split_launch_n7461():
    """At 7,461 rows FC2's gated-residual GEMM runs as two launches (rows
    [0, 6144) in 256-wide tiles, the rest in 128-wide ones); with the per-row
    W8A8 form the second launch's int8 codes and row scales start at row 6,144.
    Sampled rows either side of the split against the oracle."""
    n, dims = 7461, W8_H3_ROWFC2
    say("residual w8a8 per-row fc2, split launch", n)
    host, devw = _weights(dims, seed=21)
    K = dims.ffn
    a = synth.make_activation_bf16(n, K, "a", 21, std=0.4)
    qa, sa = _oracle_qa(a, K)
    x = synth.make_x(n, dims, 21)
    tags = synth.make_tags(n, dims.n_tags, 21)
    table = synth.make_table(dims, 1, 21)[0]
    xd = dev(x)
    lib.mlp_fc2_residual(dims, _qa_buffer(qa, sa, K), devw, dev(table), dev(tags), xd)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(21).choice(n, 20, replace=False),
                                     [0, 6143, 6144, 6145, n - 1]]))
    g = oracle.modulation_from_table(table, tags[rows])["gate2"]
    y = oracle.linear_w8a8(qa[rows], sa[rows, 0], host["w_fc2"], host["s_fc2"], oracle.bias(host, "fc2", dims.hidden))
    got = xd.cpu().numpy().astype(np.float64)[rows] - x[rows]
    assert rel_l2(got, g * y) < TOL_RESID_DELTA

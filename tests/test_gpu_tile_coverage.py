"""Every output element of the GEMM steps is written (GPU).

The GEMM maps block ids to tiles in two regions: whole groups of row tiles,
whose column tiles the eight XCDs walk in step, and the rows past the last
whole group (8 x 8 row tiles when K < 7168, 8 x 4 when K >= 7168).  At these
row counts both regions are present for both group sizes, or only the
remainder: 49,840 (195 row tiles), 16,640 (65) and 8,449 (34, the last holding
one row); at 1,192 (5 row tiles) the gated-residual GEMMs take 128-wide
column tiles, and at 7,461 and 16,640 rows they run as two launches (the
first 24 or 59 row tiles at 256 wide, the rest at 128 wide).  All three weight formats run: bf16 (the direct-to-LDS kernel),
INT8 group-32 (the dequantising kernel, with its own wave layout) and
group-scaled W8A8 (eight 32 x 128 wave tiles, its own K loop; its inputs are
the activations' group-896 int8 codes and scales).  Outputs start as NaN (bf16 and q/k/v^T) and every element must
have been written, or zero (the fp32 residual stream) and every 32 x 32 tile
must hold updates; the values themselves are checked against the oracle on
sampled rows elsewhere.
"""
import pytest
import torch

from joint_video_audio_h3_amd import lib, synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
H3 = synth.H3_DIMS
INT8_H3 = synth.WORKLOADS["h3_1blk_n1192_int8"].dims   # INT8 group-32 weights, own kernel
W8A8_H3 = synth.H3_W8A8_DIMS                            # group-scaled W8A8, own kernel
SIZES = [1192, 7461, 8449, 16640, 49840]
FORMATS = {"bf16": H3, "int8": INT8_H3, "w8a8": W8A8_H3}
BF16_NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.load()


_WEIGHTS = {}


@pytest.fixture(scope="module", params=list(FORMATS))
def fmt(request):
    # one block of each weight format, made once
    if request.param not in _WEIGHTS:
        _WEIGHTS[request.param] = lib.to_device_block(synth.make_block_weights(FORMATS[request.param], 0, seed=31))
    return FORMATS[request.param], _WEIGHTS[request.param]


def _no_nan_bf16(t):
    return not bool(t.view(torch.bfloat16).isnan().any())


def _step_input(dims, t, K):
    """The activation [n, K] as a step takes it: bf16 bits, or (W8A8) its
    group-scaled int8 codes and scales from the library's quantizer."""
    t16 = t.view(torch.int16)
    if dims.wfmt != synth.WFMT_W8A8:
        return t16
    G = K if (K == dims.ffn and dims.w8a8_row_fc2) else dims.w8a8_group
    buf = torch.empty(lib.quantized_bytes(t16.shape[0], K, G), dtype=torch.uint8, device="cuda")
    lib.quantize_groups(t16, G, buf)
    return buf


@pytest.mark.parametrize("n", SIZES)
def test_fc1_writes_every_element(n, fmt):
    H3, devw = fmt
    say("tile coverage fc1", n, H3.wfmt)
    h2 = synth.make_device_activation(n, H3.hidden, seed=32)
    a = torch.full((n, H3.ffn), BF16_NAN, dtype=torch.int16, device="cuda")
    lib.mlp_fc1_swiglu(H3, _step_input(H3, h2, H3.hidden), devw, a)
    torch.cuda.synchronize()
    assert _no_nan_bf16(a)


@pytest.mark.parametrize("n", SIZES)
def test_qkv_writes_every_element(n, fmt):
    H3, devw = fmt
    say("tile coverage qkv", n, H3.wfmt)
    h = synth.make_device_activation(n, H3.hidden, seed=33)
    pos = torch.from_numpy(synth.make_positions(n, seed=33)).cuda()
    np_ = lib.padded_rows(n)
    cs = torch.empty(np_, H3.head_dim // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table(H3, pos, n, cs)
    q = torch.full((H3.heads, np_, H3.head_dim), BF16_NAN, dtype=torch.int16, device="cuda")
    k = torch.full_like(q, BF16_NAN)
    vt = torch.full((H3.heads, H3.head_dim, np_), BF16_NAN, dtype=torch.int16, device="cuda")
    lib.qkv_rope(H3, _step_input(H3, h, H3.hidden), devw, cs, n, q, k, vt)
    torch.cuda.synchronize()
    assert _no_nan_bf16(q) and _no_nan_bf16(k) and _no_nan_bf16(vt)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("which", ["out", "fc2"])
def test_residual_updates_every_element(n, which, fmt):
    H3, devw = fmt
    say("tile coverage residual", which, n, H3.wfmt)
    K = H3.inner if which == "out" else H3.ffn
    a = synth.make_device_activation(n, K, seed=34, std=0.3)
    x = torch.zeros(n, H3.hidden, dtype=torch.float32, device="cuda")
    tags = torch.from_numpy(synth.make_tags(n, 3, seed=34)).cuda()
    table = torch.from_numpy(synth.make_table(H3, 1, seed=34)[0].view("int16")).cuda()
    fn = lib.out_proj_residual if which == "out" else lib.mlp_fc2_residual
    fn(H3, _step_input(H3, a, K), devw, table, tags, x)
    torch.cuda.synchronize()
    # x starts at zero, so a block never written stays exactly zero.  A single
    # update can be exactly zero (the fp32 sum landing on -bias: a few of the
    # 268M elements at N = 49,840), so the check is per 32 x 32 MFMA tile.
    assert bool(torch.isfinite(x).all())
    nz = (x != 0).float()
    pad = (-n) % 32
    if pad:
        nz = torch.cat([nz, torch.ones(pad, H3.hidden, device="cuda")])
    per_tile = nz.view(-1, 32, H3.hidden // 32, 32).sum(dim=(1, 3))
    assert int((per_tile == 0).sum()) == 0
    assert float(nz.mean()) > 0.999

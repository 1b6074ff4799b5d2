"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, computes workspace sizes, and rejects bad arguments on the
host before any launch.  No compute entry point is ever called with arguments
that could pass validation while a GPU is present."""
import ctypes
import os
import re

import pytest

from joint_video_audio_h3_amd import lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3dit.h")
FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libh3dit.so not built")
    return lib.load()


def _declared():
    src = open(HEADER).read()
    return re.findall(r"H3DIT_API\s+[\w\s\*]+?\b(h3_\w+)\s*\(", src)


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lib._SIGS), "binding and header disagree"


def test_struct_layouts_match_header():
    assert ctypes.sizeof(lib.H3Dims) == 4 * 14
    assert ctypes.sizeof(lib.H3BlockWeights) == 8 * 14
    assert ctypes.sizeof(lib.H3IoDims) == 4 * 3
    assert ctypes.sizeof(lib.H3Segments) == 8 * 4
    assert ctypes.sizeof(lib.H3IoWeights) == 8 * 10


def test_padded_rows_and_workspace(L):
    assert lib.padded_rows(1) == 256 and lib.padded_rows(256) == 256 and lib.padded_rows(257) == 512
    d = synth.H3_DIMS
    n = 49840
    np_ = lib.padded_rows(n)
    ws = lib.workspace_size(d, n)
    # rope cos/sin + h + q,k,v^T (a aliases them) + o, each rounded up to 256 B
    expect = np_ * 128 * 4 + np_ * 5376 * 2 + 3 * np_ * 7168 * 2 + np_ * 7168 * 2
    assert ws == expect
    assert 3.3e9 < ws < 3.6e9


def test_unfused_workspace_holds_one_gemm_output(L, monkeypatch):
    """H3_UNFUSED=1 adds one fp32 buffer for the widest GEMM output of a block
    (bf16 weights only; other formats ignore the switch)."""
    n = 1192
    np_ = lib.padded_rows(n)
    d = synth.H3_DIMS
    base = lib.workspace_size(d, n)
    base8 = lib.workspace_size(synth.H3_W8A8_DIMS, n)
    monkeypatch.setenv("H3_UNFUSED", "1")
    widest = max(3 * d.heads * d.head_dim, 2 * d.ffn, d.hidden)
    assert lib.workspace_size(d, n) == base + (np_ * widest * 4 + 255) // 256 * 256
    assert lib.workspace_size(synth.H3_W8A8_DIMS, n) == base8


def test_int8_workspace_holds_one_dequantised_linear(L):
    """INT8 weights: the full workspace adds FC1's bf16 weights (the largest
    linear) to the bf16 model's arena; a workspace without that buffer is still
    accepted (the forward then dequantises in LDS), one byte less is not."""
    n = 1192
    d8 = synth.WORKLOADS["h3_1blk_n1192_int8"].dims
    full = lib.workspace_size(d8, n)
    base = lib.workspace_size(synth.H3_DIMS, n)
    assert full - base == (2 * 2 * d8.ffn * d8.hidden + 255) // 256 * 256
    dd = lib.make_dims(d8)
    w = _full_weights()
    for f in ("s_qkv", "s_out", "s_fc1", "s_fc2"):
        setattr(w, f, FAKE)
    assert _block_call(L, dd, w, n=n, ws_bytes=base - 1) == lib.H3_ERR_WORKSPACE
    # the workspace checks pass; the call then stops for want of a device here
    for ws_bytes in (base, full):
        assert _block_call(L, dd, w, n=n, ws_bytes=ws_bytes) == lib.H3_ERR_NO_DEVICE, lib.last_error()


@pytest.mark.parametrize("field,value,code", [
    ("hidden", 300, lib.H3_ERR_UNSUPPORTED),
    ("head_dim", 64, lib.H3_ERR_UNSUPPORTED),
    ("ffn", 100, lib.H3_ERR_UNSUPPORTED),
    ("ffn", 399360, lib.H3_ERR_UNSUPPORTED),   # weight tile offsets past 32 bits
    ("n_tags", 0, lib.H3_ERR_INVALID_ARG),
    ("n_tags", 9, lib.H3_ERR_UNSUPPORTED),
    ("wfmt", 7, lib.H3_ERR_INVALID_ARG),
])
def test_bad_dims_rejected(L, field, value, code):
    d = lib.make_dims(synth.H3_DIMS)
    setattr(d, field, value)
    assert L.h3_workspace_size(ctypes.byref(d), 100) == 0
    st = L.h3_attention(ctypes.byref(d), FAKE, FAKE, FAKE, 100, FAKE, None)
    assert st == code, lib.last_error()
    assert lib.last_error()


def test_int8_needs_inner_multiple_of_128(L):
    """INT8 GEMMs run an even number of 64-wide K stages: heads*head_dim % 128 == 0."""
    d = lib.make_dims(synth.TINY_DIMS)
    d.wfmt = 1
    assert L.h3_workspace_size(ctypes.byref(d), 100) > 0     # 4 x 96 = 384 = 3 x 128
    d.heads = 2                                             # 2 x 96 = 192: a multiple of 64 only
    assert L.h3_workspace_size(ctypes.byref(d), 100) == 0
    assert L.h3_attention(ctypes.byref(d), FAKE, FAKE, FAKE, 100, FAKE, None) == lib.H3_ERR_UNSUPPORTED
    assert "128" in lib.last_error()
    d.wfmt = 0                                              # bf16 weights accept it
    assert L.h3_workspace_size(ctypes.byref(d), 100) > 0


def test_bad_rope_split_rejected(L):
    d = lib.make_dims(synth.H3_DIMS)
    d.rope_split[:] = [32, 48, 46]
    st = L.h3_rope_table(ctypes.byref(d), FAKE, 10, FAKE, None)
    assert st == lib.H3_ERR_INVALID_ARG and "rope_split" in lib.last_error()
    d.rope_split[:] = [33, 47, 48]
    assert L.h3_rope_table(ctypes.byref(d), FAKE, 10, FAKE, None) == lib.H3_ERR_INVALID_ARG


def _block_call(L, d, w, n=100, ws_bytes=None, x=FAKE, ws=FAKE):
    ws_bytes = L.h3_workspace_size(ctypes.byref(d), max(n, 1)) if ws_bytes is None else ws_bytes
    return L.h3_dit_block_forward(ctypes.byref(d), x, FAKE, FAKE, FAKE, ctypes.byref(w), n, ws,
                                  ws_bytes, None)


def _full_weights():
    w = lib.H3BlockWeights()
    for f in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
        setattr(w, f, FAKE)
    return w


def test_argument_errors_before_launch(L):
    d = lib.make_dims(synth.H3_DIMS)
    w = _full_weights()
    assert _block_call(L, d, w, n=0) == lib.H3_ERR_INVALID_ARG
    assert _block_call(L, d, w, x=None) == lib.H3_ERR_INVALID_ARG
    assert "x is NULL" in lib.last_error()
    assert _block_call(L, d, w, x=FAKE + 4) == lib.H3_ERR_INVALID_ARG
    assert "aligned" in lib.last_error()
    assert _block_call(L, d, w, ws_bytes=1024) == lib.H3_ERR_WORKSPACE
    w.w_fc2 = None
    assert _block_call(L, d, w) == lib.H3_ERR_INVALID_ARG and "w_fc2" in lib.last_error()
    # INT8 weights need their scales
    d8 = lib.make_dims(synth.WORKLOADS["h3_1blk_n1192_int8"].dims)
    assert _block_call(L, d8, _full_weights()) == lib.H3_ERR_INVALID_ARG
    assert "s_qkv" in lib.last_error()
    bad_which = L.h3_adaln_modulate(ctypes.byref(d), FAKE, FAKE, FAKE, 2, 10, FAKE, None)
    assert bad_which == lib.H3_ERR_INVALID_ARG
    arr = (lib.H3BlockWeights * 2)(_full_weights(), lib.H3BlockWeights())
    ws = L.h3_workspace_size(ctypes.byref(d), 100)
    st = L.h3_dit_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, arr, 2, 100, FAKE, ws, None)
    assert st == lib.H3_ERR_INVALID_ARG and "block 1" in lib.last_error()
    assert L.h3_dit_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, arr, 0, 100, FAKE, ws, None) \
        == lib.H3_ERR_INVALID_ARG


def _io_weights():
    w = lib.H3IoWeights()
    for f in ("w_text", "w_video", "w_audio", "w_head_audio", "w_head_video"):
        setattr(w, f, FAKE)
    return w


def _embed_call(L, d, io, w, sg, x=FAKE, text=FAKE):
    return L.h3_embed_inputs(ctypes.byref(d), ctypes.byref(io), ctypes.byref(w), ctypes.byref(sg),
                             text, FAKE, FAKE, FAKE, x, None)


def test_io_argument_errors_before_launch(L):
    d = lib.make_dims(synth.H3_DIMS)
    io = lib.make_io_dims(synth.H3_IO)
    sg = lib.make_segments(256, 1024, 200, 48360)
    w = _io_weights()
    assert lib.heads_workspace_size(synth.H3_DIMS, sg) == 48360 * 5376 * 2
    assert _embed_call(L, d, io, w, lib.make_segments(0, 0, 0, 0)) == lib.H3_ERR_INVALID_ARG
    assert _embed_call(L, d, io, w, lib.make_segments(-1, 0, 0, 5)) == lib.H3_ERR_INVALID_ARG
    assert _embed_call(L, d, io, w, sg, x=None) == lib.H3_ERR_INVALID_ARG
    assert "x_packed" in lib.last_error()
    assert _embed_call(L, d, io, w, sg, text=None) == lib.H3_ERR_INVALID_ARG
    assert "text" in lib.last_error()
    # a segment with no rows needs no input and no weights
    w2 = _io_weights()
    w2.w_audio = None
    assert _embed_call(L, d, io, w2, sg) == lib.H3_ERR_INVALID_ARG and "w_audio" in lib.last_error()
    for bad in (lib.H3IoDims(5000, 96, 32), lib.H3IoDims(5120, 48, 32), lib.H3IoDims(5120, 96, 160)):
        assert _embed_call(L, d, bad, w, sg) == lib.H3_ERR_UNSUPPORTED, lib.last_error()
    ws = lib.heads_workspace_size(synth.H3_DIMS, sg)
    st = L.h3_final_heads(ctypes.byref(d), ctypes.byref(io), ctypes.byref(w), ctypes.byref(sg),
                          FAKE, FAKE, FAKE, FAKE, FAKE, ws - 256, None)
    assert st == lib.H3_ERR_WORKSPACE
    st = L.h3_final_heads(ctypes.byref(d), ctypes.byref(io), ctypes.byref(w), ctypes.byref(sg),
                          FAKE, None, FAKE, FAKE, FAKE, ws, None)
    assert st == lib.H3_ERR_INVALID_ARG and "final_table" in lib.last_error()
    # the whole path checks its blocks too
    arr = (lib.H3BlockWeights * 1)(lib.H3BlockWeights())
    st = L.h3_velocity_forward(ctypes.byref(d), ctypes.byref(io), ctypes.byref(w), ctypes.byref(sg),
                               FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, arr, 1, FAKE, FAKE, FAKE,
                               FAKE, FAKE, L.h3_workspace_size(ctypes.byref(d), 49840), None)
    assert st == lib.H3_ERR_INVALID_ARG and "block 0" in lib.last_error()
    st = L.h3_velocity_forward(ctypes.byref(d), ctypes.byref(io), ctypes.byref(w), ctypes.byref(sg),
                               FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, arr, -1, FAKE, FAKE, FAKE,
                               FAKE, FAKE, ws, None)
    assert st == lib.H3_ERR_INVALID_ARG


def test_no_device_reported(L):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this case is only meaningful without one")
    d = lib.make_dims(synth.H3_DIMS)
    st = _block_call(L, d, _full_weights())
    assert st == lib.H3_ERR_NO_DEVICE, lib.last_error()


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError, match="no CPU path"):
        saved = lib._lib
        lib._lib = None
        try:
            lib.load(str(tmp_path / "nope.so"))
        finally:
            lib._lib = saved


def test_sigma_schedule_host_function(L):
    import numpy as np

    import oracle
    for steps, shift in ((1, 1.0), (8, 3.0), (40, 12.0), (40, 3.0)):
        np.testing.assert_array_equal(np.array(lib.sigma_schedule(steps, shift)), oracle.schedule(steps, shift))
    buf = (ctypes.c_double * 2)()
    assert L.h3_sigma_schedule(0, 3.0, buf) == lib.H3_ERR_INVALID_ARG
    assert L.h3_sigma_schedule(4, -1.0, buf) == lib.H3_ERR_INVALID_ARG
    assert L.h3_sigma_schedule(4, 3.0, None) == lib.H3_ERR_INVALID_ARG


def test_denoise_argument_errors_before_launch(L):
    d = lib.make_dims(synth.TINY_DIMS)
    io = lib.make_io_dims(synth.TINY_IO)
    sg = lib.make_segments(16, 0, 20, 128)
    w = _io_weights()
    arr = (lib.H3BlockWeights * 1)(_full_weights())
    sig = (ctypes.c_double * 3)(1.0, 0.5, 0.0)
    ws = L.h3_workspace_size(ctypes.byref(d), 164)

    def call(n_steps=2, n_blocks=1, sa=sig, ws_bytes=ws, reuse=1):
        return L.h3_denoise(ctypes.byref(d), ctypes.byref(io), ctypes.byref(w), ctypes.byref(sg),
                            FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, arr, n_blocks, FAKE, sa, sig,
                            n_steps, reuse, FAKE, FAKE, ws_bytes, None)
    assert call(n_steps=0) == lib.H3_ERR_INVALID_ARG
    assert call(reuse=0) == lib.H3_ERR_INVALID_ARG and "reuse" in lib.last_error()
    assert call(n_blocks=0) == lib.H3_ERR_INVALID_ARG
    assert call(sa=None) == lib.H3_ERR_INVALID_ARG and "sigmas" in lib.last_error()
    assert call(ws_bytes=ws - 256) == lib.H3_ERR_WORKSPACE


def test_denoise_workspace_adds_two_velocity_slots_per_modality(L):
    d, io = synth.H3_DIMS, synth.H3_IO
    sg = lib.make_segments(256, 1024, 200, 48360)
    n = 256 + 1024 + 200 + 48360
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    slots = 2 * (up(200 * io.audio_patch * 4) + up(48360 * io.video_patch * 4))
    assert lib.denoise_workspace_size(d, io, sg) == lib.workspace_size(d, n) + slots
    sg_bad = lib.make_segments(-1, 0, 0, 10)
    assert L.h3_denoise_workspace_size(ctypes.byref(lib.make_dims(d)), ctypes.byref(lib.make_io_dims(io)),
                                       ctypes.byref(sg_bad)) == 0


def test_noalloc_forward_refuses_rows_beyond_its_scratch_array(L):
    """The no-allocation forward checks on the host that the workspace fits its
    static 128 MiB array: 1,792 rows at H3 width do, 1,793 (2,048 padded) do not."""
    d = synth.H3_DIMS
    assert lib.workspace_size(d, 1792) <= (128 << 20) < lib.workspace_size(d, 1793)
    w = (lib.H3BlockWeights * 1)()
    st = L.h3_dit_forward_noalloc(ctypes.byref(lib.make_dims(d)), FAKE, FAKE, FAKE, FAKE, w, 1, 1793, None)
    assert st == lib.H3_ERR_WORKSPACE
    assert "static scratch" in lib.last_error()

"""ctypes binding of libh3dit.so (the C ABI declared in include/h3dit.h).

Argument marshalling only: every step of the forward runs in the HIP kernels
behind the C ABI.  torch is used for device memory and streams -- tensors are
passed by ``data_ptr()`` and the current HIP stream by its handle.  There is no
CPU path: if the library is missing, :func:`load` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

from .build import LIB_PATH

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

H3_OK, H3_ERR_INVALID_ARG, H3_ERR_UNSUPPORTED, H3_ERR_WORKSPACE, H3_ERR_HIP, H3_ERR_NO_DEVICE = 0, -1, -2, -3, -4, -5


class H3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"h3dit status {status}: {message}")
        self.status = status


class H3Dims(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("heads", c_i32), ("head_dim", c_i32), ("ffn", c_i32),
                ("n_tags", c_i32), ("rope_split", c_i32 * 3), ("rope_theta", c_f32),
                ("ln_eps", c_f32), ("qk_eps", c_f32), ("wfmt", c_i32), ("w8a8_group", c_i32),
                ("w8a8_row_fc2", c_i32)]


WEIGHT_FIELDS = ["w_qkv", "w_out", "w_fc1", "w_fc2", "s_qkv", "s_out", "s_fc1", "s_fc2",
                 "b_qkv", "b_out", "b_fc1", "b_fc2", "q_norm", "k_norm"]


class H3BlockWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in WEIGHT_FIELDS]


class H3IoDims(ctypes.Structure):
    _fields_ = [("text_dim", c_i32), ("video_patch", c_i32), ("audio_patch", c_i32)]


class H3Segments(ctypes.Structure):
    _fields_ = [("text", c_i64), ("cond", c_i64), ("audio", c_i64), ("video", c_i64)]


IO_WEIGHT_FIELDS = ["w_text", "b_text", "w_video", "b_video", "w_audio", "b_audio",
                    "w_head_audio", "b_head_audio", "w_head_video", "b_head_video"]


class H3IoWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in IO_WEIGHT_FIELDS]


_PD, _PIO, _PW, _PSG = (ctypes.POINTER(H3Dims), ctypes.POINTER(H3IoDims), ctypes.POINTER(H3IoWeights),
                        ctypes.POINTER(H3Segments))

# name -> (restype, argtypes), mirroring include/h3dit.h
_SIGS = {
    "h3_padded_rows": (c_i64, [c_i64]),
    "h3_workspace_size": (c_sz, [ctypes.POINTER(H3Dims), c_i64]),
    "h3_last_error": (ctypes.c_char_p, []),
    "h3_dit_block_forward": (c_i32, [ctypes.POINTER(H3Dims), c_vp, c_vp, c_vp, c_vp,
                                     ctypes.POINTER(H3BlockWeights), c_i64, c_vp, c_sz, c_vp]),
    "h3_dit_forward": (c_i32, [ctypes.POINTER(H3Dims), c_vp, c_vp, c_vp, c_vp,
                               ctypes.POINTER(H3BlockWeights), c_i32, c_i64, c_vp, c_sz, c_vp]),
    "h3_dit_forward_noalloc": (c_i32, [ctypes.POINTER(H3Dims), c_vp, c_vp, c_vp, c_vp,
                                       ctypes.POINTER(H3BlockWeights), c_i32, c_i64, c_vp]),
    "h3_rope_table": (c_i32, [ctypes.POINTER(H3Dims), c_vp, c_i64, c_vp, c_vp]),
    "h3_adaln_modulate": (c_i32, [ctypes.POINTER(H3Dims), c_vp, c_vp, c_vp, c_i32, c_i64, c_vp, c_vp]),
    "h3_qkv_rope": (c_i32, [ctypes.POINTER(H3Dims), c_vp, ctypes.POINTER(H3BlockWeights), c_vp,
                            c_i64, c_vp, c_vp, c_vp, c_vp]),
    "h3_attention": (c_i32, [ctypes.POINTER(H3Dims), c_vp, c_vp, c_vp, c_i64, c_vp, c_vp]),
    "h3_out_proj_residual": (c_i32, [ctypes.POINTER(H3Dims), c_vp, ctypes.POINTER(H3BlockWeights),
                                     c_vp, c_vp, c_i64, c_vp, c_vp]),
    "h3_mlp_fc1_swiglu": (c_i32, [ctypes.POINTER(H3Dims), c_vp, ctypes.POINTER(H3BlockWeights),
                                  c_i64, c_vp, c_vp]),
    "h3_mlp_fc2_residual": (c_i32, [ctypes.POINTER(H3Dims), c_vp, ctypes.POINTER(H3BlockWeights),
                                    c_vp, c_vp, c_i64, c_vp, c_vp]),
    "h3_heads_workspace_size": (c_sz, [_PD, _PSG]),
    "h3_quantized_bytes": (c_sz, [c_i64, c_i32, c_i32]),
    "h3_sigma_schedule": (c_i32, [c_i32, ctypes.c_double, ctypes.POINTER(ctypes.c_double)]),
    "h3_denoise_workspace_size": (c_sz, [_PD, _PIO, _PSG]),
    "h3_denoise": (c_i32, [_PD, _PIO, _PW, _PSG, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                           ctypes.POINTER(H3BlockWeights), c_i32, c_vp,
                           ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), c_i32,
                           c_i32, c_vp, c_vp, c_sz, c_vp]),
    "h3_attention_sparse": (c_i32, [_PD, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "h3_dit_forward_sparse": (c_i32, [_PD, c_vp, c_vp, c_vp, c_vp, ctypes.POINTER(H3BlockWeights), c_i32,
                                      c_i64, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "h3_quantize_groups": (c_i32, [c_vp, c_i64, c_i32, c_i32, c_vp, c_vp]),
    "h3_embed_inputs": (c_i32, [_PD, _PIO, _PW, _PSG, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "h3_final_heads": (c_i32, [_PD, _PIO, _PW, _PSG, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "h3_velocity_forward": (c_i32, [_PD, _PIO, _PW, _PSG, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    ctypes.POINTER(H3BlockWeights), c_i32, c_vp, c_vp, c_vp, c_vp,
                                    c_vp, c_sz, c_vp]),
}

_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (no fallback: raises if it has not been built).

    ``path`` defaults to the in-tree build, or to ``$H3DIT_LIB`` when that is
    set (the host-sanitizer build of the same sources, for the CPU ABI tests)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("H3DIT_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(the H3 forward has no CPU path)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def last_error() -> str:
    return load().h3_last_error().decode()


def _check(status: int):
    if status != H3_OK:
        raise H3Error(status, last_error())


def make_dims(d) -> H3Dims:
    """H3Dims from any object with the h3_dims field names (e.g. synth.Dims)."""
    s = H3Dims()
    s.hidden, s.heads, s.head_dim, s.ffn, s.n_tags = d.hidden, d.heads, d.head_dim, d.ffn, d.n_tags
    s.rope_split[:] = list(d.rope_split)
    s.rope_theta, s.ln_eps, s.qk_eps, s.wfmt = d.rope_theta, d.ln_eps, d.qk_eps, d.wfmt
    s.w8a8_group = getattr(d, "w8a8_group", 0)
    s.w8a8_row_fc2 = getattr(d, "w8a8_row_fc2", 0)
    return s


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_weights(block: Dict) -> H3BlockWeights:
    """H3BlockWeights from a dict of device tensors (missing / None = NULL)."""
    w = H3BlockWeights()
    for n in WEIGHT_FIELDS:
        setattr(w, n, _ptr(block.get(n)))
    return w


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream) if isinstance(stream, int) else stream.cuda_stream


def padded_rows(n: int) -> int:
    return load().h3_padded_rows(n)


def workspace_size(dims, n_rows: int) -> int:
    sz = load().h3_workspace_size(ctypes.byref(make_dims(dims)), n_rows)
    if sz == 0:
        raise H3Error(H3_ERR_INVALID_ARG, last_error())
    return sz


def alloc_workspace(dims, n_rows: int, device="cuda"):
    import torch
    return torch.empty(workspace_size(dims, n_rows), dtype=torch.uint8, device=device)


def dit_block_forward(dims, x, tag, positions, mod_table, block: Dict, workspace, stream=None):
    d = make_dims(dims)
    w = make_weights(block)
    _check(load().h3_dit_block_forward(ctypes.byref(d), x.data_ptr(), tag.data_ptr(),
                                       positions.data_ptr(), mod_table.data_ptr(), ctypes.byref(w),
                                       x.shape[0], workspace.data_ptr(), workspace.numel(),
                                       _stream(stream)))


def dit_forward(dims, x, tag, positions, mod_table, blocks: Sequence[Dict], workspace, stream=None):
    d = make_dims(dims)
    arr = (H3BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    _check(load().h3_dit_forward(ctypes.byref(d), x.data_ptr(), tag.data_ptr(), positions.data_ptr(),
                                 mod_table.data_ptr(), arr, len(blocks), x.shape[0],
                                 workspace.data_ptr(), workspace.numel(), _stream(stream)))


def dit_forward_noalloc(dims, x, tag, positions, mod_table, blocks: Sequence[Dict], stream=None):
    """h3_dit_forward on the library's static scratch array (no workspace argument)."""
    d = make_dims(dims)
    arr = (H3BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    _check(load().h3_dit_forward_noalloc(ctypes.byref(d), x.data_ptr(), tag.data_ptr(), positions.data_ptr(),
                                         mod_table.data_ptr(), arr, len(blocks), x.shape[0],
                                         _stream(stream)))


def rope_table(dims, positions, n_rows, cs, stream=None):
    _check(load().h3_rope_table(ctypes.byref(make_dims(dims)), positions.data_ptr(), n_rows,
                                cs.data_ptr(), _stream(stream)))


def adaln_modulate(dims, x, tag, mod_table, which, h, stream=None):
    _check(load().h3_adaln_modulate(ctypes.byref(make_dims(dims)), x.data_ptr(), tag.data_ptr(),
                                    mod_table.data_ptr(), which, x.shape[0], h.data_ptr(),
                                    _stream(stream)))


def qkv_rope(dims, h, block, cs, n_rows, q, k, vt, stream=None):
    w = make_weights(block)
    _check(load().h3_qkv_rope(ctypes.byref(make_dims(dims)), h.data_ptr(), ctypes.byref(w),
                              cs.data_ptr(), n_rows, q.data_ptr(), k.data_ptr(), vt.data_ptr(),
                              _stream(stream)))


def attention(dims, q, k, vt, n_rows, o, stream=None):
    _check(load().h3_attention(ctypes.byref(make_dims(dims)), q.data_ptr(), k.data_ptr(),
                               vt.data_ptr(), n_rows, o.data_ptr(), _stream(stream)))


def out_proj_residual(dims, o, block, mod_table, tag, x, stream=None):
    w = make_weights(block)
    _check(load().h3_out_proj_residual(ctypes.byref(make_dims(dims)), o.data_ptr(), ctypes.byref(w),
                                       mod_table.data_ptr(), tag.data_ptr(), x.shape[0],
                                       x.data_ptr(), _stream(stream)))


def mlp_fc1_swiglu(dims, h2, block, a, stream=None):
    """a [n, F] <- SwiGLU(h2 W_fc1^T + b).  The row count is a's (h2 may be a
    flat W8A8 activation buffer)."""
    w = make_weights(block)
    _check(load().h3_mlp_fc1_swiglu(ctypes.byref(make_dims(dims)), h2.data_ptr(), ctypes.byref(w),
                                    a.shape[0], a.data_ptr(), _stream(stream)))


def mlp_fc2_residual(dims, a, block, mod_table, tag, x, stream=None):
    w = make_weights(block)
    _check(load().h3_mlp_fc2_residual(ctypes.byref(make_dims(dims)), a.data_ptr(), ctypes.byref(w),
                                      mod_table.data_ptr(), tag.data_ptr(), x.shape[0],
                                      x.data_ptr(), _stream(stream)))


def _need_int32(*ts):
    import torch
    for t in ts:
        if t.dtype != torch.int32:
            raise TypeError(f"tile_off / tile_idx must be int32 device tensors, got {t.dtype}")


def attention_sparse(dims, q, k, vt, n_rows, tile, tile_off, tile_idx, o, stream=None):
    """Block-sparse attention: CSR key-tile lists (int32 device tensors) per (head, query tile)."""
    _need_int32(tile_off, tile_idx)
    _check(load().h3_attention_sparse(ctypes.byref(make_dims(dims)), q.data_ptr(), k.data_ptr(),
                                      vt.data_ptr(), n_rows, tile, tile_off.data_ptr(),
                                      tile_idx.data_ptr(), o.data_ptr(), _stream(stream)))


def dit_forward_sparse(dims, x, tag, positions, mod_table, blocks: Sequence[Dict], tile, tile_off,
                       tile_idx, workspace, stream=None):
    """h3_dit_forward with block-sparse attention; tile_off holds one CSR offset array per block."""
    _need_int32(tile_off, tile_idx)
    d = make_dims(dims)
    arr = (H3BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    _check(load().h3_dit_forward_sparse(ctypes.byref(d), x.data_ptr(), tag.data_ptr(),
                                        positions.data_ptr(), mod_table.data_ptr(), arr, len(blocks),
                                        x.shape[0], tile, tile_off.data_ptr(), tile_idx.data_ptr(),
                                        workspace.data_ptr(), workspace.numel(), _stream(stream)))


def sigma_schedule(n_steps: int, shift: float):
    """Host list of n_steps + 1 sigmas (h3_sigma_schedule)."""
    buf = (ctypes.c_double * (n_steps + 1))()
    _check(load().h3_sigma_schedule(n_steps, shift, buf))
    return list(buf)


def denoise_workspace_size(dims, io, segments: "H3Segments") -> int:
    sz = load().h3_denoise_workspace_size(ctypes.byref(make_dims(dims)), ctypes.byref(make_io_dims(io)),
                                          ctypes.byref(segments))
    if sz == 0:
        raise H3Error(H3_ERR_INVALID_ARG, last_error())
    return sz


def alloc_denoise_workspace(dims, io, text, cond, audio, video, device="cuda"):
    import torch
    sg = segments_of(text, cond, audio, video)
    return torch.empty(denoise_workspace_size(dims, io, sg), dtype=torch.uint8, device=device)


def denoise(dims, io, io_w: Dict, text, cond, audio, video, tag, positions, mod_tables,
            blocks: Sequence[Dict], final_tables, sigmas_audio, sigmas_video, x, workspace,
            stream=None, reuse: int = 1):
    """len(sigmas) - 1 Euler passes; audio / video latents updated in place.
    reuse r: fresh velocities at passes i % r == 0 and the last; a skipped pass
    extrapolates each modality's last two fresh velocities in its own sigma.
    ``workspace``: alloc_denoise_workspace()."""
    sg = segments_of(text, cond, audio, video)
    w = make_io_weights(io_w)
    arr = (H3BlockWeights * len(blocks))(*[make_weights(b) for b in blocks])
    n_steps = len(sigmas_video) - 1
    if len(sigmas_audio) != n_steps + 1:
        raise ValueError("audio and video schedules must have the same number of passes")
    sa = (ctypes.c_double * len(sigmas_audio))(*sigmas_audio)
    sv = (ctypes.c_double * len(sigmas_video))(*sigmas_video)
    _check(load().h3_denoise(
        ctypes.byref(make_dims(dims)), ctypes.byref(make_io_dims(io)), ctypes.byref(w), ctypes.byref(sg),
        _ptr(text), _ptr(cond), _ptr(audio), _ptr(video), tag.data_ptr(), positions.data_ptr(),
        mod_tables.data_ptr(), arr, len(blocks), final_tables.data_ptr(), sa, sv, n_steps, int(reuse),
        x.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def quantized_bytes(n_rows: int, width: int, group: int) -> int:
    return load().h3_quantized_bytes(n_rows, width, group)


def quantize_groups(x, group: int, out, stream=None):
    """W8A8 activation buffer ``out`` (uint8, quantized_bytes) <- int8 codes of bf16 x
    [n, K] with one scale per row and group of ``group`` elements (group = K: per row)."""
    _check(load().h3_quantize_groups(x.data_ptr(), x.shape[0], x.shape[1], group, out.data_ptr(),
                                     _stream(stream)))


def make_io_dims(io) -> H3IoDims:
    s = H3IoDims()
    s.text_dim, s.video_patch, s.audio_patch = io.text_dim, io.video_patch, io.audio_patch
    return s


def make_segments(text: int, cond: int, audio: int, video: int) -> H3Segments:
    s = H3Segments()
    s.text, s.cond, s.audio, s.video = int(text), int(cond), int(audio), int(video)
    return s


def make_io_weights(w: Dict) -> H3IoWeights:
    out = H3IoWeights()
    for n in IO_WEIGHT_FIELDS:
        setattr(out, n, _ptr(w.get(n)))
    return out


def heads_workspace_size(dims, segments: H3Segments) -> int:
    sz = load().h3_heads_workspace_size(ctypes.byref(make_dims(dims)), ctypes.byref(segments))
    if sz == 0:
        raise H3Error(H3_ERR_INVALID_ARG, last_error())
    return sz


def _rows(t) -> int:
    return 0 if t is None else int(t.shape[0])


def segments_of(text, cond, audio, video) -> H3Segments:
    return make_segments(_rows(text), _rows(cond), _rows(audio), _rows(video))


def embed_inputs(dims, io, io_w: Dict, text, cond, audio, video, x, stream=None):
    """x fp32 [N, D] <- the packed [text | cond | audio | video] rows."""
    sg = segments_of(text, cond, audio, video)
    w = make_io_weights(io_w)
    _check(load().h3_embed_inputs(ctypes.byref(make_dims(dims)), ctypes.byref(make_io_dims(io)),
                                  ctypes.byref(w), ctypes.byref(sg), _ptr(text), _ptr(cond),
                                  _ptr(audio), _ptr(video), x.data_ptr(), _stream(stream)))


def final_heads(dims, io, io_w: Dict, segments: H3Segments, x, final_table, vel_audio, vel_video,
                workspace, stream=None):
    w = make_io_weights(io_w)
    _check(load().h3_final_heads(ctypes.byref(make_dims(dims)), ctypes.byref(make_io_dims(io)),
                                 ctypes.byref(w), ctypes.byref(segments), x.data_ptr(),
                                 final_table.data_ptr(), _ptr(vel_audio), _ptr(vel_video),
                                 workspace.data_ptr(), workspace.numel(), _stream(stream)))


def velocity_forward(dims, io, io_w: Dict, text, cond, audio, video, tag, positions, mod_table,
                     blocks: Sequence[Dict], final_table, x, vel_audio, vel_video, workspace,
                     stream=None):
    """Inputs -> packed stream x -> len(blocks) blocks -> (vel_audio, vel_video)."""
    sg = segments_of(text, cond, audio, video)
    w = make_io_weights(io_w)
    arr = (H3BlockWeights * max(len(blocks), 1))(*[make_weights(b) for b in blocks])
    _check(load().h3_velocity_forward(
        ctypes.byref(make_dims(dims)), ctypes.byref(make_io_dims(io)), ctypes.byref(w),
        ctypes.byref(sg), _ptr(text), _ptr(cond), _ptr(audio), _ptr(video), _ptr(tag),
        _ptr(positions), _ptr(mod_table), arr, len(blocks), final_table.data_ptr(), x.data_ptr(),
        _ptr(vel_audio), _ptr(vel_video), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def to_device_block(block: Dict, device="cuda") -> Dict:
    """Host weight dict (numpy: uint16 bf16 bits / int8 / None) -> device tensors."""
    import numpy as np
    import torch
    out = {}
    for k, v in block.items():
        if v is None:
            out[k] = None
        elif v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).to(device)
        else:
            out[k] = torch.from_numpy(v).to(device)
    return out

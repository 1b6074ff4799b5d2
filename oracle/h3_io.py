"""Plain CPU oracle of the steps around the H3 block stack (float64).

TEST INFRASTRUCTURE ONLY, like ``h3_block``: only the tests, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP kernels or their host library.

One velocity forward turns a denoising step's inputs into the model's velocity:

 1. The packed residual stream is [text L | conditions C | audio A | video V]
    (minimax-h3-mlx README, "Architecture").  Its rows are made by:
    * text rows: the text encoder's hidden state (width 5120, read unnormalised
      after its 50th layer) through the DiT's condition projection
      (minimax-h3-mlx README, "Encoder truncation");
    * audio rows: audio latent patches (32 channels) through the audio patch
      projection; video rows: video latent patches (96 channels) through the
      video patch projection (minimax-h3-mlx README, "Architecture": two input
      patch projections; H3-metal digest, "Specialized projection kernels":
      96 -> 5376 and 32 -> 5376 with float32 weights, inputs and accumulation);
    * condition rows (keyframes, i.e. video latents): the video patch
      projection, since only two patch projections exist.
 2. The blocks (``h3_block.dit_forward``).
 3. The audio and video slices of the stream each go through a final AdaLN with
    their own (shift, scale) and a narrow output head back to patch width
    (minimax-h3-mlx README, "Architecture": two output heads; H3-metal digest,
    "Exact DiT fusions": final audio/video AdaLN on the stream's slices, and
    "Specialized projection kernels": heads on bf16 weights converted once
    from the released float32 ones).

Readings where the pages are silent: every projection is one linear layer
y = u W^T + b (PyTorch layout W[out][in]), biases optional; the final AdaLN has
the blocks' form LN(x) * (1 + scale) + shift with the same epsilon, and its
(shift, scale) pairs come precomputed per timestep like the block table, as a
table [2][2][D] ordered (audio, video) x (shift, scale).  Text and condition
rows get no velocity.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .h3_block import bf16_to_f64, layer_norm

SEGMENTS = ("text", "cond", "audio", "video")


def _linear(u: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """u W^T + b in float64; W [out, in]."""
    y = np.asarray(u, np.float64) @ np.asarray(w, np.float64).T
    return y if b is None else y + np.asarray(b, np.float64)


def _f64(a, bf16: bool) -> Optional[np.ndarray]:
    if a is None:
        return None
    return bf16_to_f64(a) if bf16 else np.asarray(a, np.float32).astype(np.float64)


def segment_rows(counts: Dict[str, int]) -> Dict[str, slice]:
    """Row range of each segment in the packed order text | cond | audio | video."""
    out, r = {}, 0
    for s in SEGMENTS:
        n = int(counts.get(s, 0))
        out[s] = slice(r, r + n)
        r += n
    return out


def embed_inputs(text_bits, cond, audio, video, io_w: Dict) -> np.ndarray:
    """Packed stream x [L+C+A+V, D] from the four inputs (step 1).

    text_bits: bf16 bits [L, text_dim]; cond, video: fp32 [C|V, video_patch];
    audio: fp32 [A, audio_patch].  io_w holds w_text/b_text (bf16 bits),
    w_video/b_video and w_audio/b_audio (fp32).
    """
    wt, bt = _f64(io_w["w_text"], True), _f64(io_w.get("b_text"), True)
    wv, bv = _f64(io_w["w_video"], False), _f64(io_w.get("b_video"), False)
    wa, ba = _f64(io_w["w_audio"], False), _f64(io_w.get("b_audio"), False)
    parts = [
        _linear(bf16_to_f64(text_bits), wt, bt),
        _linear(_f64(cond, False), wv, bv),
        _linear(_f64(audio, False), wa, ba),
        _linear(_f64(video, False), wv, bv),
    ]
    return np.concatenate(parts, axis=0)


def final_heads(x, counts: Dict[str, int], final_table_bits, io_w: Dict, eps: float):
    """Velocities (audio [A, audio_patch], video [V, video_patch]) from the stream (step 3).

    final_table_bits: bf16 bits [2, 2, D], (audio, video) x (shift, scale).
    Heads: w_head_audio / w_head_video bf16 bits [patch, D], biases bf16 or None.
    """
    x = np.asarray(x, np.float64)
    seg = segment_rows(counts)
    tab = bf16_to_f64(final_table_bits)
    out = []
    for m, name in enumerate(("audio", "video")):
        shift, scale = tab[m, 0], tab[m, 1]
        h = layer_norm(x[seg[name]], eps) * (1.0 + scale) + shift
        out.append(_linear(h, bf16_to_f64(io_w["w_head_" + name]),
                           _f64(io_w.get("b_head_" + name), True)))
    return out[0], out[1]


def velocity_forward(text_bits, cond, audio, video, io_w, final_table_bits,
                     tags, pos, table, weights_for_block, n_blocks: int, dims):
    """Inputs -> packed stream -> n_blocks blocks -> (audio, video) velocities."""
    from .h3_block import dit_forward

    counts = {"text": len(text_bits), "cond": len(cond), "audio": len(audio), "video": len(video)}
    x = embed_inputs(text_bits, cond, audio, video, io_w)
    if n_blocks:
        x = dit_forward(x, tags, pos, table, weights_for_block, n_blocks, dims)
    return final_heads(x, counts, final_table_bits, io_w, dims.ln_eps)

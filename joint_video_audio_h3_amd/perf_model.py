"""Algorithmic work of the H3 DiT block forward: FLOPs and bytes per unit.

Counts are the method's own work (what any correct implementation must do),
not what a particular kernel happens to move:

* linear layers, per row per block: 2 * D * (3*Di + Di + 2*F + F) FLOP
  = 2*D*(4*Di + 3*F); at H3 width 770.70 MFLOP.
* attention, per block: 4 * N^2 * Di FLOP (q k^T and p v, full unmasked
  attention over all N rows; softmax not counted).
* AdaLN norm-modulate, per call: read x fp32 [N, D] and write h bf16 [N, D]
  = 6 * N * D bytes (the [T, 6, D] table is negligible and L2-resident).
* around the block stack (once per forward): the text projection
  2 * L * text_dim * D FLOP (bf16); each patch projection 2 * rows * P * D
  FLOP (fp32) moving 4 * rows * (P + D) bytes; each output head a final AdaLN
  (6 * rows * D bytes) and 2 * rows * D * P FLOP (bf16).

The page "minimax-h3-mlx README", section "Performance", states the linear
layers are about 42% of the work at 37,966 packed rows and about 20% at
109,318 rows; this model reproduces both (a CPU test checks it).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class BlockWork:
    linear_flop: float
    attn_flop: float
    qkv_flop: float
    out_flop: float
    fc1_flop: float
    fc2_flop: float
    norm_bytes: float          # one AdaLN call
    weight_bytes_bf16: float

    @property
    def total_flop(self) -> float:
        return self.linear_flop + self.attn_flop


def block_work(n: int, hidden: int, inner: int, ffn: int) -> BlockWork:
    D, Di, F = hidden, inner, ffn
    qkv = 2.0 * n * D * 3 * Di
    out = 2.0 * n * Di * D
    fc1 = 2.0 * n * D * 2 * F
    fc2 = 2.0 * n * F * D
    return BlockWork(
        linear_flop=qkv + out + fc1 + fc2,
        attn_flop=4.0 * n * n * Di,
        qkv_flop=qkv, out_flop=out, fc1_flop=fc1, fc2_flop=fc2,
        norm_bytes=6.0 * n * D,
        weight_bytes_bf16=2.0 * D * (3 * Di + Di + 2 * F + F),
    )


def forward_flop(n: int, n_blocks: int, hidden: int, inner: int, ffn: int) -> float:
    return n_blocks * block_work(n, hidden, inner, ffn).total_flop


@dataclass(frozen=True)
class IoWork:
    text_flop: float
    patch_flop: float          # condition + audio + video projections
    video_patch_flop: float
    video_patch_bytes: float
    head_flop: float           # audio + video heads
    head_norm_bytes: float     # the two final AdaLN calls


def io_work(L: int, C: int, A: int, V: int, hidden: int, text_dim: int, video_patch: int,
            audio_patch: int) -> IoWork:
    D = hidden
    return IoWork(
        text_flop=2.0 * L * text_dim * D,
        patch_flop=2.0 * D * ((C + V) * video_patch + A * audio_patch),
        video_patch_flop=2.0 * V * video_patch * D,
        video_patch_bytes=4.0 * V * (video_patch + D),
        head_flop=2.0 * D * (A * audio_patch + V * video_patch),
        head_norm_bytes=6.0 * (A + V) * D,
    )


# MI355X published peaks (dense; AMD product specification)
PEAK_BF16_TFLOPS = 2500.0
PEAK_INT8_TOPS = 5000.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

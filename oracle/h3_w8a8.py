"""Plain CPU oracle of the W8A8 trunk linears (int8 weights and activations).

TEST INFRASTRUCTURE ONLY, like ``h3_block``: only the tests, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP kernels or their host library.

The 200 trunk linears (QKV, out-projection, FC1, FC2 of the 50 blocks) can run
as W8A8: int8 weights and int8 activations with scales, the product
accumulated exactly in integers (mlx-h3 README, "Generate": an opt-in backend
runs the 200 main DiT trunk linears as group-scaled W8A8, group sizes 64 to
896 along K).

Reading taken here: one scale per activation row and one per weight output row,
i.e. the group spans the whole K; symmetric codes in [-127, 127].  Each
linear's input is the activation the bf16 path would store (h after AdaLN, o
after attention, a after SwiGLU, each rounded to bf16), quantized per row:

    amax = max_k |a[r, k]|,  inv = 127 / amax,  q[r, k] = clamp(rint(a[r, k] * inv), -127, 127),
    s_a[r] = amax / 127     (every operation in IEEE float32, rint = half to even;
                             amax = 0 gives q = 0 and s_a = 0)

The codes are an integer decision, so the oracle takes it in float32, the
precision the GPU takes it in.  The linear is then

    y[r, c] = s_a[r] * s_w[c] * sum_k q[r, k] * q_w[c, k] + b[c]

with s_w the bf16 scale of weight row c.  The integer sum is exact here: float64
matmul of integers below 2^53 in magnitude (|sum| <= K * 127^2 < 2^28) has no
rounding.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .h3_block import bf16_to_f64


def quantize_rows(a) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8 codes and float32 scales of a [R, K] (float32-exact values)."""
    a32 = np.asarray(a, np.float64).astype(np.float32)
    assert np.array_equal(a32.astype(np.float64), np.asarray(a, np.float64)), "inputs must be fp32 values"
    amax = np.abs(a32).max(axis=1)                                   # exact
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    inv = (np.float32(127) / safe).astype(np.float32)                # one IEEE fp32 division
    t = (a32 * inv[:, None]).astype(np.float32)                      # one IEEE fp32 product
    q = np.clip(np.rint(t), -127, 127)
    q = np.where(nz[:, None], q, 0).astype(np.int8)
    s = np.where(nz, (safe / np.float32(127)).astype(np.float32), np.float32(0)).astype(np.float32)
    return q, s


def linear_w8a8(q_a, s_a, q_w, s_w_bits, b: Optional[np.ndarray]) -> np.ndarray:
    """y = s_a[r] * s_w[c] * (q_a q_w^T)[r, c] + b[c] in float64 (integer sum exact)."""
    acc = np.asarray(q_a, np.int8).astype(np.float64) @ np.asarray(q_w, np.int8).astype(np.float64).T
    y = acc * np.asarray(s_a, np.float32).astype(np.float64)[:, None] * bf16_to_f64(s_w_bits)[None, :]
    return y if b is None else y + b

"""Plain CPU oracle of the W8A8 trunk linears (int8 weights and activations).

TEST INFRASTRUCTURE ONLY, like ``h3_block``: only the tests, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP kernels or their host library.

The 200 trunk linears (QKV, out-projection, FC1, FC2 of the 50 blocks) can run
as group-scaled W8A8: int8 weights and int8 activations, each with one scale
per group of G consecutive elements along K, G one of 64, 256, 448 or 896
(mlx-h3 README, "Generate": the opt-in backend replaces the 200 main DiT trunk
linears with group-scaled W8A8, accepted group sizes 64, 256, 448 and 896, 896
in the example).  With groups g = [g*G, (g+1)*G) of K:

    y[r, c] = b[c] + sum_g  s_a[r, g] * s_w[c, g] * sum_{k in g} q_a[r, k] * q_w[c, k]

Readings where the page is silent:
* symmetric codes in [-127, 127]; each activation group is quantized from its
  own absolute maximum:
      amax = max_{k in g} |a[r, k]|,  inv = 127 / amax,
      q[r, k] = clamp(rint(a[r, k] * inv), -127, 127),  s_a[r, g] = amax / 127
  (rint = half to even; amax = 0 gives q = 0 and s_a = 0).  The page fixes no
  precision for this integer decision, so it is taken in IEEE float32 (the
  precision of the GPU kernels), on both sides, so the codes can be compared.
* the activation quantized is the bf16 tensor the model carries between its
  steps (h after AdaLN, o after attention, a after SwiGLU): the pages' runtime
  holds the DiT's activations in bf16.
* weight scales are bf16, one per (output row, group), from the same symmetric
  rule applied to the bf16 weight draw (the input generator does this).

FC2 has a second form (H3-metal digest, "4. Choose a speed/quality preset": an
option uses one activation scale per FC2 row and a single full-width product,
less conservative numerically than grouped int8): one scale per activation row
and one per weight output row, i.e. the group spans the whole K
(``quantize_rows`` and ``linear_w8a8``).

The integer sums are exact here: float64 matmul of integers with
|sum| <= K * 127^2 < 2^28 has no rounding.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .h3_block import bf16_to_f64

ACCEPTED_GROUPS = (64, 256, 448, 896)


def _fp32_codes(a32: np.ndarray, amax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Codes of a32 [..., G] and scales for its absolute maxima amax [...] (float32 steps)."""
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    inv = (np.float32(127) / safe).astype(np.float32)               # one IEEE fp32 division
    t = (a32 * inv[..., None]).astype(np.float32)                   # one IEEE fp32 product
    q = np.clip(np.rint(t), -127, 127)
    q = np.where(nz[..., None], q, 0).astype(np.int8)
    s = np.where(nz, (safe / np.float32(127)).astype(np.float32), np.float32(0)).astype(np.float32)
    return q, s


def _as_fp32(a) -> np.ndarray:
    a32 = np.asarray(a, np.float64).astype(np.float32)
    assert np.array_equal(a32.astype(np.float64), np.asarray(a, np.float64)), "inputs must be fp32 values"
    return a32


def quantize_groups(a, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 codes of a [R, K] per group of ``group`` consecutive K
    elements: (q int8 [R, K], s float32 [R, K / group])."""
    a32 = _as_fp32(a)
    R, K = a32.shape
    assert K % group == 0, (K, group)
    g = a32.reshape(R, K // group, group)
    q, s = _fp32_codes(g, np.abs(g).max(axis=2))
    return q.reshape(R, K), s


def quantize_rows(a) -> Tuple[np.ndarray, np.ndarray]:
    """One group per row (FC2's per-row form): (q int8 [R, K], s float32 [R])."""
    q, s = quantize_groups(a, np.asarray(a).shape[1])
    return q, s[:, 0]


def linear_w8a8_grouped(q_a, s_a, q_w, s_w_bits, b: Optional[np.ndarray], group: int) -> np.ndarray:
    """y = b + sum_g s_a[:, g] s_w[g, :] (q_a[:, g] q_w[:, g]^T) in float64.

    q_a int8 [R, K], s_a float32 [R, K/G]; q_w int8 [C, K], s_w_bits bf16 bits
    [K/G, C] (group-major: the scales of one group for every output row are
    contiguous)."""
    qa = np.asarray(q_a, np.int8).astype(np.float64)
    qw = np.asarray(q_w, np.int8).astype(np.float64)
    sa = np.asarray(s_a, np.float32).astype(np.float64)
    sw = bf16_to_f64(s_w_bits)
    R, K = qa.shape
    ng = K // group
    assert K % group == 0 and sa.shape == (R, ng) and sw.shape == (ng, qw.shape[0])
    y = np.zeros((R, qw.shape[0]))
    for g in range(ng):
        ks = slice(g * group, (g + 1) * group)
        y += (qa[:, ks] @ qw[:, ks].T) * sa[:, g][:, None] * sw[g][None, :]
    return y if b is None else y + b


def linear_w8a8(q_a, s_a, q_w, s_w_bits, b: Optional[np.ndarray]) -> np.ndarray:
    """FC2's per-row form: y = s_a[r] * s_w[c] * (q_a q_w^T)[r, c] + b[c] (s_w bf16 [C])."""
    acc = np.asarray(q_a, np.int8).astype(np.float64) @ np.asarray(q_w, np.int8).astype(np.float64).T
    y = acc * np.asarray(s_a, np.float32).astype(np.float64)[:, None] * bf16_to_f64(s_w_bits)[None, :]
    return y if b is None else y + b

"""Plain, slow CPU oracle of the MiniMax-H3 DiT block forward (float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the tests, the smoke check of ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` use it.  It shares no code with the HIP
kernels, their headers or their host library, and it does not import the
input generator: it takes the generator's arrays as plain numpy inputs.

Every floating-point step runs in float64 on values decoded exactly from the
inputs (bf16 bit patterns, int8 codes, fp32 activations).  Nothing is blocked,
fused or reordered beyond what each definition states; attention is split over
query rows only to bound memory, which changes no value.

What the block computes, per row r with modality tag m = tag[r] (sources are
page titles and sections):

 1. (shift1, scale1, gate1, shift2, scale2, gate2) = table[m, 0..5]
    -- minimax-h3-mlx README, "AdaLN precompute" (per-timestep modulation table,
    18 x D = 3 tags x 6 vectors) and "AdaLN: measure, do not reason" (the six
    tensors: x*(1+scale)+shift for the norms, x + gate*f(x) for the branches).
 2. h = LN(x) * (1 + scale1) + shift1;  LN without affine, biased variance.
 3. u = h W_qkv^T + b_qkv, rows interleaved per head [q, k, v]
    -- minimax-h3-mlx README, "Validation".
 4. q, k <- RMSNorm over head_dim (gain gamma_q / gamma_k), before RoPE
    -- H3-metal digest, "Checkpoint layout and media pipeline" (fused
    QK-normalisation/RoPE kernel on the interleaved QKV layout).
 5. q, k <- 3-D rotary embedding over (t, h, w) chunks of head_dim
    -- minimax-h3-mlx README, "Architecture" (3D MM-RoPE).
 6. o = softmax(q k^T / sqrt(d)) v over all rows, no mask
    -- minimax-h3-mlx README, "Architecture" (full self-attention over the
    packed sequence) and "Performance" (flash-style, never materialised).
 7. x <- x + gate1 * (o W_out^T + b_out)
 8. h2 = LN(x) * (1 + scale2) + shift2
 9. z = h2 W_fc1^T + b_fc1;  a = silu(z[:, :F]) * z[:, F:]
    -- minimax-h3-mlx README, "Validation" (fc1 is fused [gate; value]).
10. x <- x + gate2 * (a W_fc2^T + b_fc2)

Readings where the pages are silent: LN and RMSNorm epsilon 1e-6; rotary base
10000, contiguous chunks [t | h | w], adjacent pairs (2j, 2j+1), frequency
theta^(-2j/d_axis); softmax scale 1/sqrt(d); all biases optional (absent = 0),
QK gains optional (absent = 1).  INT8 weight-only layers use
W = bf16(q * s) with s one bf16 scale per 32 consecutive K elements (the GPU
feeds the same dequantised bf16 values to its matrix cores).  W8A8 layers
(int8 weights and activations with one scale per group of K elements) follow
``h3_w8a8``.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence

import numpy as np

MOD_NAMES = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")


# ------------------------------------------------------------------ decoding
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (bf16 is the top half of an fp32 word)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits: write v = m * 2**e with 0.5 <= |m| < 1, round
    m * 2**8 to an integer (half to even) and scale back.  Only normal-range
    values occur here.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def dequant_int8_g32(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """W[o, k] = bf16(q[o, k] * s[o, k // 32]) as float64 (weight-only INT8, group 32)."""
    q = np.asarray(q, dtype=np.int8).astype(np.float64)
    s = bf16_to_f64(s_bits)
    o, k = q.shape
    prod = q.reshape(o, k // 32, 32) * s[:, :, None]
    return round_to_bf16(prod).reshape(o, k)


def weight(w: Dict[str, Optional[np.ndarray]], name: str) -> np.ndarray:
    """Decode linear layer ``name`` ('qkv', 'out', 'fc1', 'fc2') to float64 [out, in]."""
    raw = w["w_" + name]
    if raw.dtype == np.int8:
        return dequant_int8_g32(raw, w["s_" + name])
    return bf16_to_f64(raw)


def bias(w, name: str, n_out: int) -> np.ndarray:
    b = w.get("b_" + name)
    return np.zeros(n_out) if b is None else bf16_to_f64(b)


WFMT_W8A8 = 2   # group-scaled int8 weights and activations (h3_w8a8)


def linear(act: np.ndarray, w, name: str, n_out: int, dims) -> np.ndarray:
    """Trunk linear ``name``: act W^T + b, or its W8A8 form (h3_w8a8) when the
    weights are W8A8: the activation, a bf16 tensor in the model, is quantized
    per group of dims.w8a8_group K elements (FC2 per row when
    dims.w8a8_row_fc2) and multiplied in integers."""
    if getattr(dims, "wfmt", 0) == WFMT_W8A8:
        from .h3_w8a8 import linear_w8a8, linear_w8a8_grouped, quantize_groups, quantize_rows
        a = round_to_bf16(act)
        if name == "fc2" and getattr(dims, "w8a8_row_fc2", 0):
            q, s = quantize_rows(a)
            return linear_w8a8(q, s, w["w_" + name], w["s_" + name], bias(w, name, n_out))
        G = dims.w8a8_group
        q, s = quantize_groups(a, G)
        return linear_w8a8_grouped(q, s, w["w_" + name], w["s_" + name], bias(w, name, n_out), G)
    return act @ weight(w, name).T + bias(w, name, n_out)


# ------------------------------------------------------------------ steps
def modulation_from_table(table_b: np.ndarray, tags: np.ndarray) -> Dict[str, np.ndarray]:
    """Per-row modulation vectors gathered from one block's table [T, 6, D] (step 1)."""
    t = bf16_to_f64(table_b)
    g = t[np.asarray(tags)]                       # [N, 6, D]
    return {name: g[:, i, :] for i, name in enumerate(MOD_NAMES)}


def build_mod_table(w_ada_bits: np.ndarray, b_ada_bits: np.ndarray,
                    temb_by_tag: np.ndarray) -> np.ndarray:
    """Precompute one block's table from its AdaLN projection (step 1's source).

    The projection maps a timestep embedding e to 18*D values = 3 groups x 6
    vectors; group m of the projection of modality m's embedding is table[m].
    The projection's output is bf16, as in the bf16 model.
    minimax-h3-mlx README, "AdaLN precompute".
    """
    W = bf16_to_f64(w_ada_bits)
    b = bf16_to_f64(b_ada_bits)
    T = temb_by_tag.shape[0]
    D = W.shape[0] // (6 * T)
    out = np.empty((T, 6, D))
    for m in range(T):
        full = round_to_bf16(W @ np.asarray(temb_by_tag[m], np.float64) + b)
        out[m] = full.reshape(T, 6, D)[m]
    return out


def modulation_live(w_ada_bits, b_ada_bits, temb_by_tag, tags) -> Dict[str, np.ndarray]:
    """Per-row modulation computed by running the projection for every row.

    Row r takes its own modality's embedding through the full projection and
    keeps chunk tag[r] of the 18*D outputs.  This is the path the table replaces.
    """
    W = bf16_to_f64(w_ada_bits)
    b = bf16_to_f64(b_ada_bits)
    T = temb_by_tag.shape[0]
    D = W.shape[0] // (6 * T)
    N = len(tags)
    mods = np.empty((N, 6, D))
    for r in range(N):
        m = int(tags[r])
        full = round_to_bf16(W @ np.asarray(temb_by_tag[m], np.float64) + b)
        mods[r] = full.reshape(T, 6, D)[m]
    return {name: mods[:, i, :] for i, name in enumerate(MOD_NAMES)}


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(biased var + eps) over the last axis, no affine."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    c = x - mu
    var = (c * c).mean(axis=-1, keepdims=True)
    return c / np.sqrt(var + eps)


def adaln_modulate(x, shift, scale, eps: float) -> np.ndarray:
    """Steps 2 and 8: LN(x) * (1 + scale) + shift."""
    return layer_norm(x, eps) * (1.0 + scale) + shift


def qkv_split(u: np.ndarray, heads: int, head_dim: int):
    """Split the fused projection output [N, 3*H*d] into q, k, v [H, N, d].

    Columns of head h are [q | k | v] at 3*d*h + (0, d, 2d) (per-head interleave).
    """
    N = u.shape[0]
    q = np.empty((heads, N, head_dim))
    k = np.empty_like(q)
    v = np.empty_like(q)
    for h in range(heads):
        base = 3 * head_dim * h
        q[h] = u[:, base:base + head_dim]
        k[h] = u[:, base + head_dim:base + 2 * head_dim]
        v[h] = u[:, base + 2 * head_dim:base + 3 * head_dim]
    return q, k, v


def rms_norm(v: np.ndarray, gamma: Optional[np.ndarray], eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * gamma over the last axis (step 4)."""
    v = np.asarray(v, np.float64)
    r = v / np.sqrt((v * v).mean(axis=-1, keepdims=True) + eps)
    return r if gamma is None else r * gamma


def rope_angles(pos: np.ndarray, split: Sequence[int], theta: float) -> np.ndarray:
    """Rotation angle of every channel pair: [N, d/2] (step 5).

    Pair j of axis chunk a (width d_a) turns by pos[:, a] * theta**(-2j/d_a).
    """
    pos = np.asarray(pos, np.float64)
    cols = []
    for a, d_a in enumerate(split):
        j = np.arange(d_a // 2, dtype=np.float64)
        freq = theta ** (-2.0 * j / d_a)
        cols.append(pos[:, a:a + 1] * freq[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(v: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (2j, 2j+1) of v [..., N, d] by ang [N, d/2]."""
    v = np.asarray(v, np.float64)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              q_rows: Optional[np.ndarray] = None, chunk: int = 512) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v per head over all key rows (step 6).

    q, k, v: [H, N, d].  Returns [H, R, d] for the query rows ``q_rows``
    (default all).  Query rows are processed ``chunk`` at a time.
    """
    H, N, d = k.shape
    rows = np.arange(q.shape[1]) if q_rows is None else np.asarray(q_rows)
    out = np.empty((H, len(rows), d))
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        for c0 in range(0, len(rows), chunk):
            r = rows[c0:c0 + chunk]
            s = (q[h, r] @ k[h].T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[h, c0:c0 + chunk] = p @ v[h]
    return out


def merge_heads(o: np.ndarray) -> np.ndarray:
    """[H, N, d] -> [N, H*d], head h in columns [h*d, (h+1)*d)."""
    H, N, d = o.shape
    return np.ascontiguousarray(o.transpose(1, 0, 2)).reshape(N, H * d)


def silu(t: np.ndarray) -> np.ndarray:
    return t / (1.0 + np.exp(-t))


def swiglu(z: np.ndarray, ffn: int) -> np.ndarray:
    """Step 9's activation: silu(gate) * value with z = [gate | value]."""
    return silu(z[:, :ffn]) * z[:, ffn:]


# ------------------------------------------------------------------ block
def block_steps(x, tags, pos, table_b, w, dims, q_rows=None, mods=None,
                sparse=None) -> Dict[str, np.ndarray]:
    """Run one block and return every intermediate (float64).

    ``q_rows`` restricts the row-local steps after attention (and attention's
    query side) to a subset of rows; keys and values always use every row.
    ``mods`` replaces the table gather with given per-row modulation vectors.
    ``sparse`` = (tile, tile_off, tile_idx) makes step 6 block-sparse
    (``h3_sparse.attention_sparse``) instead of full.
    """
    D, H, d, F = dims.hidden, dims.heads, dims.head_dim, dims.ffn
    x = np.asarray(x, np.float64)
    N = x.shape[0]
    rows = np.arange(N) if q_rows is None else np.asarray(q_rows)
    m = modulation_from_table(table_b, tags) if mods is None else mods
    out: Dict[str, np.ndarray] = {}
    h = adaln_modulate(x, m["shift1"], m["scale1"], dims.ln_eps)
    out["h"] = h
    u = linear(h, w, "qkv", 3 * H * d, dims)
    q, k, v = qkv_split(u, H, d)
    gq = None if w.get("q_norm") is None else bf16_to_f64(w["q_norm"])
    gk = None if w.get("k_norm") is None else bf16_to_f64(w["k_norm"])
    ang = rope_angles(pos, dims.rope_split, dims.rope_theta)
    q = apply_rope(rms_norm(q, gq, dims.qk_eps), ang)
    k = apply_rope(rms_norm(k, gk, dims.qk_eps), ang)
    out["q"], out["k"], out["v"] = q, k, v
    if sparse is not None:
        from .h3_sparse import attention_sparse
        assert q_rows is None, "block-sparse attention runs over every query row"
        o = merge_heads(attention_sparse(q, k, v, *sparse))
    else:
        o = merge_heads(attention(q, k, v, rows))
    out["o"] = o
    xr = x[rows] + m["gate1"][rows] * linear(o, w, "out", D, dims)
    out["x_mid"] = xr
    h2 = adaln_modulate(xr, m["shift2"][rows], m["scale2"][rows], dims.ln_eps)
    out["h2"] = h2
    z = linear(h2, w, "fc1", 2 * F, dims)
    a = swiglu(z, F)
    out["a"] = a
    out["x_out"] = xr + m["gate2"][rows] * linear(a, w, "fc2", D, dims)
    return out


def block_forward(x, tags, pos, table_b, w, dims, q_rows=None, mods=None, sparse=None) -> np.ndarray:
    """One H3 DiT block: x [N, D] -> x_out [N, D] (or [R, D] for ``q_rows``)."""
    return block_steps(x, tags, pos, table_b, w, dims, q_rows, mods, sparse)["x_out"]


def dit_forward(x, tags, pos, table, weights_for_block: Callable[[int], dict],
                n_blocks: int, dims, sparse_for_block: Optional[Callable[[int], tuple]] = None) -> np.ndarray:
    """Blocks 0..n_blocks-1 in order over the packed rows (one denoising forward);
    ``sparse_for_block(b)`` gives block b's (tile, tile_off, tile_idx) selection."""
    y = np.asarray(x, np.float64)
    for b in range(n_blocks):
        sp = None if sparse_for_block is None else sparse_for_block(b)
        y = block_forward(y, tags, pos, table[b], weights_for_block(b), dims, sparse=sp)
    return y

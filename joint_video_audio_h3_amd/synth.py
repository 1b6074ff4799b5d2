"""Seeded synthetic inputs for the MiniMax-H3 DiT block forward.

This module only *makes inputs*: the shapes of the packed-sequence workloads,
one independent random stream per tensor, packing of fp32 draws into bf16 bit
patterns, and the INT8 group-32 quantizer that turns a bf16 weight draw into
the (int8 codes, bf16 scales) pair the weight-only path consumes.  No step of
the block (normalisation, projection, rotation, attention, gating) is computed
here, so both the CPU oracle and the GPU path can take these arrays as they are.

Sources for the shapes (page titles and sections; no real checkpoint exists
here, every tensor is a synthetic draw):

* minimax-h3-mlx README, "Architecture": 50 blocks, hidden 5376, 56x128 heads
  (inner 7168), SwiGLU FFN 14336, 3D MM-RoPE; one packed sequence
  [text L | keyframe conditions C | target audio A | target video V]; modality
  enters through a per-row AdaLN tag.
* minimax-h3-mlx README, "AdaLN precompute": the per-block projection is
  [96768, 2688] and 96768 = 18 x 5376, i.e. 3 modality groups x 6 modulation
  vectors of width D per timestep.
* minimax-h3-mlx README, "Validation": the packed (t, h, w) grid is built in
  float64; video and audio share one 40-units-per-second rotary clock.

Readings (stated once, used everywhere):

* tags: 0 = text and condition rows, 1 = audio rows, 2 = video rows.
* positions: a text or audio row at index i is 1-D, i.e. (i, i, i) on the three
  rotary axes; a video latent (f, y, x) sits at (f * 20/3, y, x) -- one latent
  frame is 4 video frames at 24 fps, 1/6 s, i.e. 20/3 units of the 40 u/s clock;
  a condition (reference image) token on a 32-wide grid sits at (0, y, x).  The
  grid is built in float64 and cast to float32 once.
* distributions: x ~ N(0, 1) fp32; W ~ N(0, 1/fan_in) rounded to bf16; biases
  ~ N(0, 1/fan_in) bf16; QK-norm gains ~ 1 + N(0, 0.01) bf16; modulation table
  ~ N(0, 0.1) (variance 0.1) bf16.
* INT8 weight-only: symmetric, groups of 32 along K, one bf16 scale per group:
  s = bf16(max|w_g| / 127) (s = 0 gives q = 0), q = clamp(round-half-even(w/s),
  -127, 127).  W8A8 weights: the same with groups of dims.w8a8_group along K
  and the scales stored group-major [K / group][out] (per output row for FC2
  in its per-row form).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

# tensor ids of the per-tensor streams: SeedSequence([seed, block, tensor_id])
_TID = {
    "x": 0, "w_qkv": 1, "b_qkv": 2, "w_out": 3, "b_out": 4, "w_fc1": 5,
    "b_fc1": 6, "w_fc2": 7, "b_fc2": 8, "q_norm": 9, "k_norm": 10, "table": 11,
    "h": 12, "o": 13, "a": 14, "q": 15, "k": 16, "v": 17, "tags": 18, "pos": 19,
    "text": 20, "cond": 21, "audio_in": 22, "video_in": 23, "w_text": 24, "b_text": 25,
    "w_video": 26, "b_video": 27, "w_audio": 28, "b_audio": 29, "w_head_audio": 30,
    "b_head_audio": 31, "w_head_video": 32, "b_head_video": 33, "final_table": 34,
    "tile_mask": 35,
}
TAG_TEXT, TAG_AUDIO, TAG_VIDEO = 0, 1, 2
WFMT_BF16, WFMT_INT8_G32, WFMT_W8A8 = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    n_tags: int = 3
    rope_split: Tuple[int, int, int] = (32, 48, 48)
    rope_theta: float = 10000.0
    ln_eps: float = 1e-6
    qk_eps: float = 1e-6
    wfmt: int = WFMT_BF16
    w8a8_group: int = 0          # W8A8: K elements per scale group (64, 256, 448 or 896)
    w8a8_row_fc2: int = 0        # W8A8: FC2 with one scale per row instead of per group

    @property
    def inner(self) -> int:
        return self.heads * self.head_dim


H3_DIMS = Dims(hidden=5376, heads=56, head_dim=128, ffn=14336)
TINY_DIMS = Dims(hidden=256, heads=4, head_dim=96, ffn=768, rope_split=(24, 36, 36))
# group-scaled W8A8 trunk, group 896 as in the pages' example (the tiny model's
# widths 256 / 384 / 768 take only the group of 64)
H3_W8A8_DIMS = dataclasses.replace(H3_DIMS, wfmt=WFMT_W8A8, w8a8_group=896)
TINY_W8A8_DIMS = dataclasses.replace(TINY_DIMS, wfmt=WFMT_W8A8, w8a8_group=64)


@dataclasses.dataclass(frozen=True)
class IoDims:
    """Widths of the stream's inputs and outputs around the block stack."""
    text_dim: int = 5120      # text encoder hidden state
    video_patch: int = 96     # 24 latent channels x (1 x 2 x 2) patch
    audio_patch: int = 32     # 32 latent channels


H3_IO = IoDims()
TINY_IO = IoDims(text_dim=128)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    n_blocks: int
    L: int
    C: int
    A: int
    V: Tuple[int, int, int]

    @property
    def n_rows(self) -> int:
        return self.L + self.C + self.A + self.V[0] * self.V[1] * self.V[2]


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_2blk_n164", TINY_DIMS, 2, 16, 0, 20, (2, 8, 8)),
        Workload("h3_1blk_n1192", H3_DIMS, 1, 128, 0, 40, (1, 32, 32)),
        Workload("h3_50blk_n6437", H3_DIMS, 50, 256, 0, 37, (6, 32, 32)),
        Workload("h3_50blk_n7461", H3_DIMS, 50, 256, 1024, 37, (6, 32, 32)),
        Workload("h3_50blk_n49840", H3_DIMS, 50, 256, 1024, 200, (31, 30, 52)),
        Workload("h3_1blk_n1192_int8",
                 dataclasses.replace(H3_DIMS, wfmt=WFMT_INT8_G32), 1, 128, 0, 40, (1, 32, 32)),
        Workload("h3_1blk_n1192_w8a8", H3_W8A8_DIMS, 1, 128, 0, 40, (1, 32, 32)),
        Workload("h3_50blk_n6437_w8a8", H3_W8A8_DIMS, 50, 256, 0, 37, (6, 32, 32)),
        Workload("h3_50blk_n49840_w8a8", H3_W8A8_DIMS, 50, 256, 1024, 200, (31, 30, 52)),
    ]
}


def _rng(seed: int, block: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, block, _TID[name]])))


# ---------------------------------------------------------------- bf16 packing
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1          # finite inputs only: u + 0x8000 stays below 2^32
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def quantize_int8_rows(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric INT8 codes with one bf16 scale per output row (W8A8 FC2 in its
    per-row form).

    ``w_bits`` bf16 [out, in]; returns (q int8 [out, in], s bf16 bits [out]):
    s = bf16(max|w_row| / 127), q = clamp(round-half-even(w / s), -127, 127).
    """
    q, s = quantize_int8_groups(w_bits, w_bits.shape[1])
    return q, s[0]


def quantize_int8_groups(w_bits: np.ndarray, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric INT8 codes with one bf16 scale per output row and group of
    ``group`` consecutive K elements (the group-scaled W8A8 weights).

    ``w_bits`` bf16 [out, in]; returns (q int8 [out, in], s bf16 bits
    [in / group, out]), group-major: s[g, o] = bf16(max|w[o, g]| / 127),
    q = clamp(round-half-even(w / s), -127, 127) (s = 0 gives q = 0).
    """
    out_f, in_f = w_bits.shape
    assert in_f % group == 0
    w = bf16_bits_to_f32(w_bits).astype(np.float64).reshape(out_f, in_f // group, group)
    amax = np.abs(w).max(axis=2)
    s_bits = f32_to_bf16_bits((amax / 127.0).astype(np.float32))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(w / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8).reshape(out_f, in_f)
    return q, np.ascontiguousarray(s_bits.T)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_int8_g32(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric INT8 codes with one bf16 scale per 32 consecutive K elements.

    ``w_bits`` is a bf16 weight [out, in] (bit patterns); returns (q int8
    [out, in], s bf16 bits [out, in/32]).
    """
    out_f, in_f = w_bits.shape
    assert in_f % 32 == 0
    w = bf16_bits_to_f32(w_bits).astype(np.float64).reshape(out_f, in_f // 32, 32)
    amax = np.abs(w).max(axis=2)
    s_bits = f32_to_bf16_bits((amax / 127.0).astype(np.float32))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(w / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8).reshape(out_f, in_f)
    return q, s_bits


# ---------------------------------------------------------------- geometry
def packed_layout(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Modality tags int32 [N] and rotary positions float32 [N, 3] of the packed rows."""
    rows_t, rows_p = [], []
    L, C, A = wl.L, wl.C, wl.A
    f, gh, gw = wl.V
    idx = np.arange(L, dtype=np.float64)
    rows_t.append(np.full(L, TAG_TEXT, np.int32))
    rows_p.append(np.stack([idx, idx, idx], axis=1))
    if C:
        c = np.arange(C)
        rows_t.append(np.full(C, TAG_TEXT, np.int32))
        rows_p.append(np.stack([np.zeros(C), (c // 32).astype(np.float64),
                                (c % 32).astype(np.float64)], axis=1))
    k = np.arange(A, dtype=np.float64)
    rows_t.append(np.full(A, TAG_AUDIO, np.int32))
    rows_p.append(np.stack([k, k, k], axis=1))
    ff, yy, xx = np.meshgrid(np.arange(f), np.arange(gh), np.arange(gw), indexing="ij")
    rows_t.append(np.full(f * gh * gw, TAG_VIDEO, np.int32))
    rows_p.append(np.stack([ff.ravel() * (20.0 / 3.0), yy.ravel().astype(np.float64),
                            xx.ravel().astype(np.float64)], axis=1))
    tags = np.concatenate(rows_t)
    pos = np.concatenate(rows_p).astype(np.float32)
    assert tags.shape[0] == wl.n_rows
    return tags, np.ascontiguousarray(pos)


# ---------------------------------------------------------------- tensors
def make_activation_bf16(n: int, width: int, name: str, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """bf16 bits [n, width] ~ N(0, std^2): stand-alone input of one step ('h', 'o', 'a', ...)."""
    a = _rng(seed, 0, name).standard_normal((n, width), dtype=np.float32)
    return f32_to_bf16_bits(a * np.float32(std))


def make_peaked_qkv(heads: int, n: int, d: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Attention inputs whose softmax is sharply peaked: bf16 bits q, k, v [heads, n, d].

    q is given in the attention kernels' convention (already multiplied by
    log2(e)/sqrt(d)), so q . k is a score in log2 units.  Channel 0 carries a
    key ramp: keys of the first 64 rows sit at -8, the later keys rise linearly
    to +8 at the last row; every query scales that ramp by b ~ U(-1, 4), and the
    other channels are N(0, 1) noise on both sides (a score spread of about 11
    log2 units per query).  So scores span tens of log2 units and, for most
    queries, the running maximum keeps rising tile after tile up to the last
    (possibly partial) tile.  Row 0 of every head is 20 * e_0: its first 64
    scores are -160 and its maximum is the last key; row 1 is -20 * e_0: its
    maximum is in the first tile and the later scores fall to -160.
    """
    r = _rng(seed, 0, "q")
    ramp = np.full(n, -8.0, np.float32)
    if n > 65:
        ramp[64:] = np.linspace(-8.0, 8.0, n - 64, dtype=np.float32)
    k = _rng(seed, 0, "k").standard_normal((heads, n, d), dtype=np.float32)
    k[:, :, 0] = ramp
    q = r.standard_normal((heads, n, d), dtype=np.float32)
    q[:, :, 0] = r.uniform(-1.0, 4.0, (heads, n)).astype(np.float32)
    q[:, 0, :] = 0.0
    q[:, 0, 0] = 20.0
    if n > 1:
        q[:, 1, :] = 0.0
        q[:, 1, 0] = -20.0
    v = _rng(seed, 0, "v").standard_normal((heads, n, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_tags(n: int, n_tags: int = 3, seed: int = 0) -> np.ndarray:
    """Random modality tags int32 [n] (for steps tested away from a packed layout)."""
    return _rng(seed, 0, "tags").integers(0, n_tags, n).astype(np.int32)


def make_positions(n: int, seed: int = 0) -> np.ndarray:
    """Random rotary coordinates float32 [n, 3] in [0, 250), fractional and integral mixed."""
    r = _rng(seed, 0, "pos")
    p = r.uniform(0, 250, (n, 3))
    p[::2] = np.floor(p[::2])
    return p.astype(np.float32)


def make_x(wl_or_n, dims: Dims, seed: int = 0) -> np.ndarray:
    n = wl_or_n.n_rows if isinstance(wl_or_n, Workload) else int(wl_or_n)
    return _rng(seed, 0, "x").standard_normal((n, dims.hidden), dtype=np.float32)


def _normal_bf16(seed, block, name, shape, var) -> np.ndarray:
    a = _rng(seed, block, name).standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(a * np.float32(np.sqrt(var)))


def make_table(dims: Dims, n_blocks: int, seed: int = 0) -> np.ndarray:
    """Modulation table bf16 bits [n_blocks, n_tags, 6, D] ~ N(0, 0.1)."""
    return np.stack([_normal_bf16(seed, b, "table", (dims.n_tags, 6, dims.hidden), 0.1)
                     for b in range(n_blocks)])


def make_block_weights(dims: Dims, block: int, seed: int = 0,
                       biases: bool = True, norms: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Host weights of one block in PyTorch Linear layout W[out][in].

    bf16 layers: ``w_*`` are uint16 bit patterns.  INT8 layers (dims.wfmt == 1):
    ``w_*`` are int8 codes and ``s_*`` are bf16 scale bits [out, in/32]; W8A8
    layers (dims.wfmt == 2): int8 codes and bf16 scale bits [in/G, out] (G =
    dims.w8a8_group; [out] for FC2 when dims.w8a8_row_fc2).  All are derived
    from the same seeded bf16 draw the bf16 build would use.
    Rows of ``w_qkv`` are interleaved per head: [h0: q, k, v][h1: q, k, v]...
    and ``w_fc1`` stacks [gate; value].
    """
    D, Di, F, d = dims.hidden, dims.inner, dims.ffn, dims.head_dim
    shapes = {"qkv": (3 * Di, D), "out": (D, Di), "fc1": (2 * F, D), "fc2": (D, F)}
    w: Dict[str, Optional[np.ndarray]] = {}

    def one(k):
        o, i = shapes[k]
        bits = _normal_bf16(seed, block, "w_" + k, (o, i), 1.0 / i)
        if dims.wfmt == WFMT_INT8_G32:
            return quantize_int8_g32(bits)
        if dims.wfmt == WFMT_W8A8:
            if k == "fc2" and dims.w8a8_row_fc2:
                return quantize_int8_rows(bits)
            return quantize_int8_groups(bits, dims.w8a8_group)
        return bits, None

    # independent streams per tensor: drawing them concurrently changes no value
    with ThreadPoolExecutor(max_workers=4) as ex:
        drawn = dict(zip(shapes, ex.map(one, shapes)))
    for k, (o, i) in shapes.items():
        w["w_" + k], w["s_" + k] = drawn[k]
        w["b_" + k] = _normal_bf16(seed, block, "b_" + k, (o,), 1.0 / i) if biases else None
    if norms:
        for k in ("q_norm", "k_norm"):
            g = 1.0 + 0.1 * _rng(seed, block, k).standard_normal(d, dtype=np.float32)
            w[k] = f32_to_bf16_bits(g)
    else:
        w["q_norm"] = w["k_norm"] = None
    return w


def make_io_weights(dims: Dims, io: IoDims, seed: int = 0, biases: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Weights of the steps around the block stack (host arrays).

    w_text bf16 bits [D, text_dim]; w_video fp32 [D, video_patch]; w_audio fp32
    [D, audio_patch]; output heads bf16 bits [patch, D] (drawn in fp32 and
    rounded once, as the released fp32 heads are converted); biases of the
    same kinds, all ~ N(0, 1/fan_in).
    """
    D = dims.hidden
    w: Dict[str, Optional[np.ndarray]] = {}

    def f32(name, shape, var):
        return (_rng(seed, 0, name).standard_normal(shape, dtype=np.float32)
                * np.float32(np.sqrt(var)))

    w["w_text"] = _normal_bf16(seed, 0, "w_text", (D, io.text_dim), 1.0 / io.text_dim)
    w["w_video"] = f32("w_video", (D, io.video_patch), 1.0 / io.video_patch)
    w["w_audio"] = f32("w_audio", (D, io.audio_patch), 1.0 / io.audio_patch)
    w["w_head_audio"] = _normal_bf16(seed, 0, "w_head_audio", (io.audio_patch, D), 1.0 / D)
    w["w_head_video"] = _normal_bf16(seed, 0, "w_head_video", (io.video_patch, D), 1.0 / D)
    if biases:
        w["b_text"] = _normal_bf16(seed, 0, "b_text", (D,), 1.0 / io.text_dim)
        w["b_video"] = f32("b_video", (D,), 1.0 / io.video_patch)
        w["b_audio"] = f32("b_audio", (D,), 1.0 / io.audio_patch)
        w["b_head_audio"] = _normal_bf16(seed, 0, "b_head_audio", (io.audio_patch,), 1.0 / D)
        w["b_head_video"] = _normal_bf16(seed, 0, "b_head_video", (io.video_patch,), 1.0 / D)
    else:
        for k in ("b_text", "b_video", "b_audio", "b_head_audio", "b_head_video"):
            w[k] = None
    return w


def make_final_table(dims: Dims, seed: int = 0) -> np.ndarray:
    """Final AdaLN table bf16 bits [2, 2, D], (audio, video) x (shift, scale), ~ N(0, 0.1)."""
    return _normal_bf16(seed, 0, "final_table", (2, 2, dims.hidden), 0.1)


def make_io_inputs(wl: Workload, io: IoDims, seed: int = 0) -> Dict[str, np.ndarray]:
    """Per-step inputs of the packed segments: text hidden state bf16 bits
    [L, text_dim] ~ N(0, 1); condition and video latent patches fp32
    [C|V, video_patch] and audio patches fp32 [A, audio_patch], all ~ N(0, 1)
    (the noised latents of rectified flow are unit-variance)."""
    V = wl.V[0] * wl.V[1] * wl.V[2]

    def f32(name, shape):
        return _rng(seed, 0, name).standard_normal(shape, dtype=np.float32)

    return {
        "text": _normal_bf16(seed, 0, "text", (wl.L, io.text_dim), 1.0),
        "cond": f32("cond", (wl.C, io.video_patch)),
        "audio": f32("audio_in", (wl.A, io.audio_patch)),
        "video": f32("video_in", (V, io.video_patch)),
    }


def make_tile_mask(n: int, heads: int, tile: int, keep: float, dense_rows: int = 0,
                   seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Synthetic key-tile selection of block-sparse attention, CSR (tile_off
    int32 [heads*nq + 1], tile_idx int32 [nnz]), nq = ceil(n / tile).

    Query tiles that overlap the first ``dense_rows`` rows (the text and
    condition prefix) select every tile.  Every other query tile selects the
    prefix's key tiles, its own tile, and further distinct tiles at random
    until it holds max(ceil(keep * nq), those) tiles; indices sorted.  (The
    trained selection is not available; this keeps its shape: a fixed budget
    per query tile, dense prefix queries, prefix keys always kept.)
    """
    nq = -(-n // tile)
    budget = min(nq, max(1, int(np.ceil(keep * nq))))
    n_prefix = min(nq, -(-dense_rows // tile)) if dense_rows > 0 else 0
    r = _rng(seed, 0, "tile_mask")
    score = r.random((heads, nq, nq))                 # [head, query tile, key tile]
    score[:, :, :n_prefix] = 2.0                      # prefix keys always kept
    ii = np.arange(nq)
    score[:, ii, ii] = 2.0                            # the own tile always kept
    score[:, :n_prefix, :] = 2.0                      # prefix queries: every tile
    # every non-prefix query tile keeps k = max(prefix tiles + own tile, budget)
    # tiles: those scoring at least its k-th largest score (random scores are
    # distinct; the forced ones score highest)
    k = min(nq, max(n_prefix + 1, budget))
    thr = np.partition(score, nq - k, axis=2)[..., nq - k:nq - k + 1]
    thr[:, :n_prefix] = -1.0                          # prefix queries keep everything
    sel = score >= thr
    counts = sel.sum(axis=2).reshape(-1)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    idx = np.nonzero(sel.reshape(heads * nq, nq))[1].astype(np.int32)   # row-major: sorted per row
    return off, idx


def make_inputs(wl: Workload, seed: int = 0, n_blocks: Optional[int] = None,
                biases: bool = True, norms: bool = True):
    """Everything one forward of ``wl`` needs, on the host (small workloads only)."""
    nb = wl.n_blocks if n_blocks is None else n_blocks
    tags, pos = packed_layout(wl)
    x = make_x(wl, wl.dims, seed)
    table = make_table(wl.dims, nb, seed)
    weights = [make_block_weights(wl.dims, b, seed, biases, norms) for b in range(nb)]
    return x, tags, pos, table, weights


def make_device_rows(wl: Workload, seed: int = 0, device: str = "cuda"):
    """x fp32 [N, D] ~ N(0, 1) drawn on the device, plus the packed tags and positions."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + 1)
    tags, pos = packed_layout(wl)
    x = torch.randn(wl.n_rows, wl.dims.hidden, generator=g, device=device, dtype=torch.float32)
    return x, torch.from_numpy(tags).to(device), torch.from_numpy(pos).to(device)


def make_device_activation(n: int, width: int, seed: int, std: float = 1.0, device: str = "cuda"):
    """bf16 [n, width] ~ N(0, std^2) drawn on the device (large stand-alone step inputs)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + 3)
    return (torch.randn(n, width, generator=g, device=device) * std).to(torch.bfloat16)


def make_device_weights(dims: Dims, n_blocks: int, seed: int = 0, device: str = "cuda"):
    """Modulation table and per-block weights with the host generator's
    distributions, drawn on the device by torch.

    Used where the host generator would take minutes (50 blocks of 5376-wide
    weights = 19.3e9 draws).  The streams differ from the host generator's, so
    inputs made here serve timing and properties that hold for any input;
    parity against the oracle always uses :func:`make_inputs`.
    """
    import torch

    D, Di, F, d = dims.hidden, dims.inner, dims.ffn, dims.head_dim
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + 2)
    table = (torch.randn(n_blocks, dims.n_tags, 6, D, generator=g, device=device)
             * float(np.sqrt(0.1))).to(torch.bfloat16)
    shapes = {"qkv": (3 * Di, D), "out": (D, Di), "fc1": (2 * F, D), "fc2": (D, F)}
    blocks = []
    for b in range(n_blocks):
        g.manual_seed(seed * 1000003 + 7919 * (b + 1))
        wb = {}
        for k, (o, i) in shapes.items():
            w = torch.randn(o, i, generator=g, device=device) * float(1.0 / np.sqrt(i))
            if dims.wfmt == WFMT_INT8_G32:
                wb["w_" + k], wb["s_" + k] = _quantize_int8_g32_torch(w.to(torch.bfloat16))
            elif dims.wfmt == WFMT_W8A8:
                grp = i if (k == "fc2" and dims.w8a8_row_fc2) else dims.w8a8_group
                wq, ws = _quantize_int8_groups_torch(w.to(torch.bfloat16), grp)
                wb["w_" + k], wb["s_" + k] = wq, (ws[0].contiguous() if grp == i else ws)
            else:
                wb["w_" + k], wb["s_" + k] = w.to(torch.bfloat16), None
            del w
            wb["b_" + k] = (torch.randn(o, generator=g, device=device)
                            * float(1.0 / np.sqrt(i))).to(torch.bfloat16)
        for k in ("q_norm", "k_norm"):
            wb[k] = (1.0 + 0.1 * torch.randn(d, generator=g, device=device)).to(torch.bfloat16)
        blocks.append(wb)
    return table, blocks


def _quantize_int8_g32_torch(w_bf16):
    import torch

    o, i = w_bf16.shape
    w = w_bf16.float().view(o, i // 32, 32)
    s = (w.abs().amax(dim=2) / 127.0).to(torch.bfloat16)
    sf = s.float().unsqueeze(-1)
    q = torch.where(sf > 0, torch.round(w / torch.where(sf > 0, sf, torch.ones_like(sf))),
                    torch.zeros_like(w))
    return q.clamp_(-127, 127).to(torch.int8).view(o, i).contiguous(), s.contiguous()


def _quantize_int8_groups_torch(w_bf16, group):
    """Device twin of quantize_int8_groups: (codes [o, i], bf16 scales [i/group, o])."""
    import torch

    o, i = w_bf16.shape
    w = w_bf16.float().view(o, i // group, group)
    s = (w.abs().amax(dim=2) / 127.0).to(torch.bfloat16)
    sf = s.float().unsqueeze(-1)
    q = torch.where(sf > 0, torch.round(w / torch.where(sf > 0, sf, torch.ones_like(sf))),
                    torch.zeros_like(w))
    return q.clamp_(-127, 127).to(torch.int8).view(o, i).contiguous(), s.t().contiguous()

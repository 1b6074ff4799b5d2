"""Conditioning of the group-scaled W8A8 forward, measured on the oracle alone.

Writes (merges into) w8a8_conditioning.json beside this file.  For each case,
two oracle forwards of the H3-width W8A8 model (group 896, 50 blocks) start
from x and from x * (1 + 1e-7 * noise), a perturbation at the level of float32
rounding, and the script records after every block the rel-L2 distance between
the two states and between their updates x_b - x_0.  The bf16-weight model is
traced the same way over its first blocks for comparison.  Any two correct
implementations differ at least at that level (float32 against float64
arithmetic, another summation order, bf16 intermediates), so this distance is
the spread the W8A8 trunk itself puts between correct results: its int8 codes
turn sub-ulp differences of an activation into whole code steps.

Cases (the long GPU depth tests' inputs, seed 50):
  n1192   N = 1,192 (text 128, audio 40, video 1x32x32)    about 30 minutes on 8 cores
  n6437   N = 6,437 (text 256, audio 37, video 6x32x32)    about 3 hours on 8 cores

Run: python tests/golden/w8a8_conditioning.py n1192 [n6437]
It calls only the oracle and the seeded input generator.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from joint_video_audio_h3_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "w8a8_conditioning.json")
CASES = {
    "n1192": ("H3 width, N = 1,192 (L 128, A 40, V 1x32x32), seed 50, eps 1e-7", 128, 40, (1, 32, 32)),
    "n6437": ("H3 width, N = 6,437 (L 256, A 37, V 6x32x32), seed 50, eps 1e-7", 256, 37, (6, 32, 32)),
}


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def trace(dims, n_blocks, L, A, V, seed=50, eps=1e-7):
    wl = synth.Workload("cond", dims, n_blocks, L, 0, A, V)
    tags, pos = synth.packed_layout(wl)
    x = synth.make_x(wl, dims, seed=seed).astype(np.float64)
    table = synth.make_table(dims, n_blocks, seed=seed)
    xp = x * (1.0 + eps * np.random.default_rng(seed).standard_normal(x.shape))
    a, b = x.copy(), xp.copy()
    out = []
    for blk in range(n_blocks):
        w = synth.make_block_weights(dims, blk, seed)
        a = oracle.block_forward(a, tags, pos, table[blk], w, dims)
        b = oracle.block_forward(b, tags, pos, table[blk], w, dims)
        out.append({"block": blk + 1, "x": rel(b, a), "update": rel(b - xp, a - x)})
        print(dims.wfmt, out[-1], flush=True)
    return out


def main(names):
    res = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            res = json.load(f)
    for name in names:
        desc, L, A, V = CASES[name]
        res[name] = {"workload": desc,
                     "w8a8_group896": trace(synth.H3_W8A8_DIMS, 50, L, A, V),
                     "bf16_first_blocks": trace(synth.H3_DIMS, 3, L, A, V)}
        with open(OUT, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main(sys.argv[1:] or ["n1192"])

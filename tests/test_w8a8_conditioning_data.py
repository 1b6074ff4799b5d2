"""The stored conditioning trace of the W8A8 trunk (tests/golden/w8a8_conditioning.json,
written by tests/golden/w8a8_conditioning.py from the oracle alone) is what the long
GPU depth tests take their W8A8 bounds from.  Here (CPU) its first block is
recomputed with the oracle and must match, and the trace must have the shape the
bound assumes: 50 blocks, growing, and far above the bf16 model's spread under the
same perturbation."""
import importlib.util
import json
import os

import numpy as np
import pytest

from joint_video_audio_h3_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
COND = os.path.join(HERE, "golden", "w8a8_conditioning.json")


def _script():
    spec = importlib.util.spec_from_file_location("w8a8_conditioning", os.path.join(HERE, "golden", "w8a8_conditioning.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_stored_trace_shape():
    with open(COND) as f:
        cond = json.load(f)
    assert "n1192" in cond
    for case, t in cond.items():
        w = t["w8a8_group896"]
        assert [r["block"] for r in w] == list(range(1, 51)), case
        xs = np.array([r["x"] for r in w])
        assert np.all(np.diff(xs) > 0), case                      # the spread only grows
        assert 1e-3 < xs[0] < xs[-1] < 0.2, case
        bf = t["bf16_first_blocks"]
        assert len(bf) == 3 and max(r["x"] for r in bf) < 1e-6, case   # bf16: the 1e-7 nudge stays 1e-7
        assert xs[2] > 1e3 * bf[2]["x"], case


@pytest.mark.timeout(600)
def test_first_block_reproduces():
    """Block 1 of the N = 1,192 trace, recomputed from the oracle."""
    mod = _script()
    with open(COND) as f:
        stored = json.load(f)["n1192"]["w8a8_group896"][0]
    _, L, A, V = mod.CASES["n1192"]
    got = mod.trace(synth.H3_W8A8_DIMS, 1, L, A, V)[0]
    assert got["block"] == 1
    np.testing.assert_allclose(got["x"], stored["x"], rtol=0.02)
    np.testing.assert_allclose(got["update"], stored["update"], rtol=0.02)

"""Input generator and work-model checks (no GPU)."""
import json
import os

import numpy as np
import pytest
import torch

from joint_video_audio_h3_amd import perf_model, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def test_bf16_packing_matches_torch_rounding():
    r = np.random.default_rng(0)
    a = (r.standard_normal(50000) * 10.0 ** r.integers(-8, 8, 50000)).astype(np.float32)
    a = np.concatenate([a, np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0])])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(a), ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ref),
                                  torch.from_numpy(a).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_shapes(name):
    wl = synth.WORKLOADS[name]
    tags, pos = synth.packed_layout(wl)
    assert tags.shape == (wl.n_rows,) and pos.shape == (wl.n_rows, 3)
    assert pos.dtype == np.float32 and tags.dtype == np.int32
    counts = np.bincount(tags, minlength=3)
    assert counts[0] == wl.L + wl.C and counts[1] == wl.A
    assert counts[2] == wl.V[0] * wl.V[1] * wl.V[2]
    assert sum(wl.dims.rope_split) == wl.dims.head_dim


def test_named_row_counts():
    n = {k: w.n_rows for k, w in synth.WORKLOADS.items()}
    assert n["tiny_2blk_n164"] == 164
    assert n["h3_1blk_n1192"] == 1192
    assert n["h3_50blk_n6437"] == 6437
    assert n["h3_50blk_n7461"] == 7461
    assert n["h3_50blk_n49840"] == 49840


def test_video_positions_on_shared_clock():
    wl = synth.WORKLOADS["tiny_2blk_n164"]
    tags, pos = synth.packed_layout(wl)
    vid = pos[tags == 2]
    # second latent frame is 4 frames at 24 fps = 1/6 s = 20/3 units of the 40 u/s clock
    assert vid[64, 0] == np.float32(20.0 / 3.0)
    assert vid[1, 2] == 1.0 and vid[8, 1] == 1.0


def test_generator_is_deterministic_and_streams_independent():
    d = synth.TINY_DIMS
    a = synth.make_block_weights(d, 0, seed=5)
    b = synth.make_block_weights(d, 0, seed=5)
    c = synth.make_block_weights(d, 1, seed=5)
    for k in a:
        if a[k] is not None:
            np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["w_qkv"], c["w_qkv"])
    assert a["w_qkv"].shape == (3 * d.inner, d.hidden) and a["w_fc1"].shape == (2 * d.ffn, d.hidden)


def test_int8_quantizer_ranges():
    d = synth.WORKLOADS["h3_1blk_n1192_int8"].dims
    small = synth.Dims(hidden=256, heads=2, head_dim=128, ffn=256, wfmt=synth.WFMT_INT8_G32)
    w = synth.make_block_weights(small, 0, seed=1)
    assert w["w_qkv"].dtype == np.int8 and w["s_qkv"].shape == (3 * 256, 256 // 32)
    assert np.abs(w["w_qkv"].astype(np.int32)).max() == 127
    assert d.wfmt == synth.WFMT_INT8_G32


def test_work_model_reproduces_pages_linear_share():
    g = json.load(open(GOLDEN))["linear_share_of_work"]
    d = synth.H3_DIMS
    for rows, share in zip(g["rows"], g["approx_share"]):
        w = perf_model.block_work(rows, d.hidden, d.inner, d.ffn)
        assert abs(w.linear_flop / w.total_flop - share) < 0.01


def test_work_model_per_row_and_weights():
    d = synth.H3_DIMS
    w = perf_model.block_work(1, d.hidden, d.inner, d.ffn)
    assert w.linear_flop == pytest.approx(770.70e6, rel=1e-4)
    g = json.load(open(GOLDEN))
    # trunk bf16 weights for 50 blocks ~ the ~38 GB bf16 DiT body; int8 + g32 scales ~ 20 GB
    body = 50 * w.weight_bytes_bf16 / 1e9
    assert abs(body - g["dit_body_resident_gb"]["bf16"]) < 1.0
    int8 = 50 * w.weight_bytes_bf16 / 2 * (1 + 2 / 32) / 1e9
    assert abs(int8 - g["dit_body_resident_gb"]["int8"]) < 1.0
    # trunk params below the 20.11B that remain once the AdaLN projections are dropped
    assert 50 * w.weight_bytes_bf16 / 2 / 1e9 < g["params_after_adaln_drop_billion"]["value"]


def test_table_layout_matches_cache_size():
    g = json.load(open(GOLDEN))
    out, _ = g["adaln_proj_shape"]["value"]
    d = synth.H3_DIMS
    assert out == d.n_tags * 6 * d.hidden
    c = g["adaln_cache_77_timesteps"]
    table = synth.make_table(synth.TINY_DIMS, 1)
    assert table.dtype == np.uint16 and table.shape[1:] == (3, 6, 256)
    mb = c["distinct_timesteps"] * g["adaln_proj_shape"]["blocks"] * out * table.itemsize / 1e6
    assert abs(mb - c["megabytes"]) < 1.0

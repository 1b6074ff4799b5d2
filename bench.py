#!/usr/bin/env python3
"""Benchmark of the MiniMax-H3 DiT forward on one MI355X.

A step is one denoising forward: the 50-block DiT over one packed sequence,
inputs and weights resident in HBM, run through the C ABI (h3_dit_forward).
Primary workload: N = 49,840 packed rows (L 256 | C 1024 | A 200 | V 31x30x52);
secondary: N = 6,437 (L 256 | A 37 | V 6x32x32); extra: N = 7,461 (the same
with a 1,024-row reference image, C = 1024).  All use the same 50 blocks of
synthetic bf16 weights (random init, H3 shapes).

Printed: one JSON line with packed tokens/s per forward, the per-step kernel
times (HIP events on the launch stream) with their TFLOP/s and fraction of the
bf16 MFMA peak, the roofline of the dominant kernel, the steps around the block
stack (input projections, output heads) at the same segment geometry, and the
CPU oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from joint_video_audio_h3_amd import perf_model, synth  # noqa: E402

PEAK = perf_model.PEAK_BF16_TFLOPS
HBM = perf_model.PEAK_HBM_GBS
# HBM traffic of the dominant kernels from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE,
# bytes per launch after the copy-kernel calibration (profiles/), with the first
# 16 hex digits of the SHA-256 of the kernel's source file when the counters
# were taken: reported only while that source is unchanged, else None.
TRAFFIC_BYTES = {("h3_50blk_n49840", "attention"): (8.578e9, "0ff5dc2ed7652585")}
KERNEL_SOURCE = {"attention": "attention.hip", "qkv_rope": "gemm.hip", "fc1_swiglu": "gemm.hip",
                 "fc2_resid": "gemm.hip", "out_proj_resid": "gemm.hip"}


def measured_traffic(workload, kernel):
    """Counter-measured bytes per launch, if taken on the current kernel source."""
    import hashlib

    entry = TRAFFIC_BYTES.get((workload, kernel))
    if entry is None:
        return None
    path = os.path.join(ROOT, "joint_video_audio_h3_amd", "csrc", KERNEL_SOURCE[kernel])
    with open(path, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    return entry[0] if sha == entry[1] else None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _time_launches(fn, reps, torch):
    """Average duration (ms) of `fn` over `reps` launches, bracketed by HIP events
    on the current stream (the stream the C ABI launches on)."""
    fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def step_breakdown(lib, dims, wl_rows, table, block, reps, torch, only=None):
    """Per-kernel times of one block's steps on the block-0 weights."""
    x, tags, pos = wl_rows
    n = x.shape[0]
    D, Di, F, H, d = dims.hidden, dims.inner, dims.ffn, dims.heads, dims.head_dim
    np_ = lib.padded_rows(n)
    dev = x.device
    cs = torch.empty(np_, d // 2, 2, dtype=torch.float32, device=dev)
    h = torch.empty(n, D, dtype=torch.int16, device=dev)
    q = torch.empty(H, np_, d, dtype=torch.int16, device=dev)
    k = torch.empty_like(q)
    vt = torch.empty(H, d, np_, dtype=torch.int16, device=dev)
    o = torch.empty(n, Di, dtype=torch.int16, device=dev)
    a = torch.empty(n, F, dtype=torch.int16, device=dev)
    xs = x.clone()
    t0 = table[0]
    lib.rope_table(dims, pos, n, cs)
    w = perf_model.block_work(n, D, Di, F)
    steps = {
        "adaln": (lambda: lib.adaln_modulate(dims, xs, tags, t0, 0, h), None, w.norm_bytes),
        "qkv_rope": (lambda: lib.qkv_rope(dims, h, block, cs, n, q, k, vt), w.qkv_flop, None),
        "attention": (lambda: lib.attention(dims, q, k, vt, n, o), w.attn_flop, None),
        "out_proj_resid": (lambda: lib.out_proj_residual(dims, o, block, t0, tags, xs), w.out_flop, None),
        "fc1_swiglu": (lambda: lib.mlp_fc1_swiglu(dims, h, block, a), w.fc1_flop, None),
        "fc2_resid": (lambda: lib.mlp_fc2_residual(dims, a, block, t0, tags, xs), w.fc2_flop, None),
    }
    out = {}
    if only:
        # inputs of the later steps come from running the earlier ones once
        for name, (fn, _, _) in steps.items():
            if name == only:
                break
            fn()
        steps = {only: steps[only]}
    for name, (fn, flop, nbytes) in steps.items():
        ms = _time_launches(fn, reps, torch)
        r = {"ms": round(ms, 4)}
        if flop:
            tf = flop / (ms * 1e-3) / 1e12
            r.update(tflops=round(tf, 1), mfma_frac=round(tf / PEAK, 4))
        if nbytes:
            gbs = nbytes / (ms * 1e-3) / 1e9
            r.update(gbs=round(gbs, 1), hbm_frac=round(gbs / HBM, 4))
        out[name] = r
    if only:
        return out, w
    gemm_flop = w.linear_flop
    gemm_ms = sum(out[s]["ms"] for s in ("qkv_rope", "out_proj_resid", "fc1_swiglu", "fc2_resid"))
    out["gemms_total"] = {"ms": round(gemm_ms, 4), "tflops": round(gemm_flop / gemm_ms / 1e9, 1),
                          "mfma_frac": round(gemm_flop / gemm_ms / 1e9 / PEAK, 4)}
    return out, w


def step_breakdown_w8a8(lib, dims, wl_rows, table, block, reps, torch, only=None):
    """Per-kernel times of one W8A8 block's steps (int8 GEMMs against the int8 peak)."""
    x, tags, pos = wl_rows
    n = x.shape[0]
    D, Di, F, H, d = dims.hidden, dims.inner, dims.ffn, dims.heads, dims.head_dim
    G = dims.w8a8_group
    Gf = F if dims.w8a8_row_fc2 else G
    np_ = lib.padded_rows(n)
    dev = x.device
    cs = torch.empty(np_, d // 2, 2, dtype=torch.float32, device=dev)
    h = torch.empty(n, D, dtype=torch.int16, device=dev)
    hq = torch.empty(lib.quantized_bytes(n, D, G), dtype=torch.uint8, device=dev)
    q = torch.empty(H, np_, d, dtype=torch.int16, device=dev)
    k = torch.empty_like(q)
    vt = torch.empty(H, d, np_, dtype=torch.int16, device=dev)
    o = torch.empty(n, Di, dtype=torch.int16, device=dev)
    oq = torch.empty(lib.quantized_bytes(n, Di, G), dtype=torch.uint8, device=dev)
    a = torch.empty(n, F, dtype=torch.int16, device=dev)
    aq = torch.empty(lib.quantized_bytes(n, F, Gf), dtype=torch.uint8, device=dev)
    xs = x.clone()
    t0 = table[0]
    lib.rope_table(dims, pos, n, cs)
    w = perf_model.block_work(n, D, Di, F)
    I8 = perf_model.PEAK_INT8_TOPS
    qbytes = lambda K, g: 2.0 * n * K + n * K + 4.0 * n * K / g  # noqa: E731
    steps = {
        "adaln": (lambda: lib.adaln_modulate(dims, xs, tags, t0, 0, h), None, 6.0 * n * D, None),
        "quant_h": (lambda: lib.quantize_groups(h, G, hq), None, qbytes(D, G), None),
        "qkv_rope": (lambda: lib.qkv_rope(dims, hq, block, cs, n, q, k, vt), w.qkv_flop, None, I8),
        "attention": (lambda: lib.attention(dims, q, k, vt, n, o), w.attn_flop, None, PEAK),
        "quant_o": (lambda: lib.quantize_groups(o, G, oq), None, qbytes(Di, G), None),
        "out_proj_resid": (lambda: lib.out_proj_residual(dims, oq, block, t0, tags, xs), w.out_flop, None, I8),
        "fc1_swiglu": (lambda: lib.mlp_fc1_swiglu(dims, hq, block, a), w.fc1_flop, None, I8),
        "quant_a": (lambda: lib.quantize_groups(a, Gf, aq), None, qbytes(F, Gf), None),
        "fc2_resid": (lambda: lib.mlp_fc2_residual(dims, aq, block, t0, tags, xs), w.fc2_flop, None, I8),
    }
    out = {}
    if only:
        # inputs of the later steps come from running the earlier ones once
        for name, (fn, _, _, _) in steps.items():
            if name == only:
                break
            fn()
        steps = {only: steps[only]}
    for name, (fn, flop, nbytes, peak) in steps.items():
        ms = _time_launches(fn, reps, torch)
        r = {"ms": round(ms, 4)}
        if flop:
            tf = flop / (ms * 1e-3) / 1e12
            r.update(tops=round(tf, 1), peak=peak, mfma_frac=round(tf / peak, 4))
        if nbytes:
            gbs = nbytes / (ms * 1e-3) / 1e9
            r.update(gbs=round(gbs, 1), hbm_frac=round(gbs / HBM, 4))
        out[name] = r
    if only:
        return out, w
    lin = ("qkv_rope", "out_proj_resid", "fc1_swiglu", "fc2_resid")
    gemm_ms = sum(out[s_]["ms"] for s_ in lin)
    out["gemms_total"] = {"ms": round(gemm_ms, 4), "tops": round(w.linear_flop / gemm_ms / 1e9, 1),
                          "peak": I8, "mfma_frac": round(w.linear_flop / gemm_ms / 1e9 / I8, 4),
                          "bf16_frac_equiv": round(w.linear_flop / gemm_ms / 1e9 / PEAK, 4)}
    return out, w


def io_breakdown(lib, dims, io, wl, reps, torch):
    """Per-call times of the steps around the block stack at the workload's
    segment geometry: the whole input projection, the video patch projection
    alone (its fp32 matrix-core rate and HBM rate), and the two output heads."""
    V = wl.V[0] * wl.V[1] * wl.V[2]
    inp = synth.make_io_inputs(wl, io, seed=0)
    w_host = synth.make_io_weights(dims, io, seed=0)
    dv = lambda a: (None if a is None or len(a) == 0 else  # noqa: E731
                    torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda())
    w = {k: dv(v) for k, v in w_host.items()}
    d = {k: dv(v) for k, v in inp.items()}
    ftab = dv(synth.make_final_table(dims, seed=0))
    x = torch.empty(wl.n_rows, dims.hidden, dtype=torch.float32, device="cuda")
    xv = torch.empty(V, dims.hidden, dtype=torch.float32, device="cuda")
    va = torch.empty(wl.A, io.audio_patch, dtype=torch.float32, device="cuda")
    vv = torch.empty(V, io.video_patch, dtype=torch.float32, device="cuda")
    sg = lib.segments_of(d["text"], d["cond"], d["audio"], d["video"])
    sg_v = lib.make_segments(0, 0, 0, V)
    ws = torch.empty(lib.heads_workspace_size(dims, sg), dtype=torch.uint8, device="cuda")
    iw = perf_model.io_work(wl.L, wl.C, wl.A, V, dims.hidden, io.text_dim, io.video_patch,
                            io.audio_patch)
    calls = {
        "embed_inputs": (lambda: lib.embed_inputs(dims, io, w, d["text"], d["cond"], d["audio"],
                                                  d["video"], x),
                         iw.text_flop + iw.patch_flop, None, PEAK),
        "video_patch_embed": (lambda: lib.embed_inputs(dims, io, w, None, None, None, d["video"], xv),
                              iw.video_patch_flop, iw.video_patch_bytes, perf_model.PEAK_FP32_MFMA_TFLOPS),
        "final_heads": (lambda: lib.final_heads(dims, io, w, sg, x, ftab, va, vv, ws),
                        iw.head_flop, iw.head_norm_bytes, PEAK),
        "video_head": (lambda: lib.final_heads(dims, io, w, sg_v, x[-V:], ftab, None, vv, ws),
                       2.0 * V * dims.hidden * io.video_patch, 6.0 * V * dims.hidden, PEAK),
    }
    out = {}
    for name, (fn, flop, nbytes, peak) in calls.items():
        ms = _time_launches(fn, reps, torch)
        r = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
             "peak_tflops": peak, "mfma_frac": round(flop / (ms * 1e-3) / 1e12 / peak, 4)}
        if nbytes:
            gbs = nbytes / (ms * 1e-3) / 1e9
            r.update(gbs=round(gbs, 1), hbm_frac=round(gbs / HBM, 4))
        out[name] = r
    return out


def visited_flop(n, heads, d, tile, off, idx):
    """4*d FLOP per (query, selected key) pair of block-sparse attention."""
    import numpy as np

    nq = -(-n // tile)
    rows = np.minimum(tile, n - np.arange(nq) * tile)                   # rows per query tile
    keys_per_tile = np.minimum(tile, n - np.arange(nq) * tile)          # valid rows per key tile
    counts = np.add.reduceat(keys_per_tile[idx], off[:-1]) * (np.diff(off) > 0)
    return 4.0 * d * float(np.sum(np.tile(rows, heads) * counts))


def sparse_breakdown(lib, dims, n, reps, torch, keep=0.125, dense_rows=1280):
    """Block-sparse attention at N rows: each tile size at `keep` of the key
    tiles (dense prefix queries), rated on the FLOPs of the pairs it visits."""
    H, d = dims.heads, dims.head_dim
    np_ = lib.padded_rows(n)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    qs = float(1.4426950408889634 / d ** 0.5)
    q = torch.zeros(H, np_, d, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    vt = torch.zeros(H, d, np_, dtype=torch.bfloat16, device="cuda")
    q[:, :n] = (torch.randn(H, n, d, generator=g, device="cuda") * qs).to(torch.bfloat16)
    k[:, :n] = torch.randn(H, n, d, generator=g, device="cuda").to(torch.bfloat16)
    vt[:, :, :n] = torch.randn(H, d, n, generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty(n, H * d, dtype=torch.bfloat16, device="cuda")
    out = {"keep": keep, "dense_prefix_rows": dense_rows}
    dense_ms = _time_launches(lambda: lib.attention(dims, q, k, vt, n, o), reps, torch)
    out["dense_ms"] = round(dense_ms, 3)
    for tile in (128, 64):
        off, idx = synth.make_tile_mask(n, H, tile, keep, dense_rows=dense_rows, seed=0)
        offd, idxd = torch.from_numpy(off).cuda(), torch.from_numpy(idx).cuda()
        ms = _time_launches(lambda: lib.attention_sparse(dims, q, k, vt, n, tile, offd, idxd, o), reps, torch)
        fl = visited_flop(n, H, d, tile, off, idx)
        tf = fl / (ms * 1e-3) / 1e12
        log(f"sparse attention tile {tile}: {ms:.2f} ms")
        out[f"tile{tile}"] = {"ms": round(ms, 3), "visited_fraction": round(fl / (4.0 * d * H * n * n), 4),
                              "visited_tflops": round(tf, 1), "mfma_frac": round(tf / PEAK, 4),
                              "speedup_vs_dense": round(dense_ms / ms, 2)}
    return out


def run_forward(lib, dims, rows, table, blocks, ws, steps, warmup, torch, per_step=None):
    """Seconds per forward over `steps` back-to-back forwards (wall clock around
    all of them).  HIP events on the launch stream between forwards give each
    forward's own time without a host wait; with `per_step` (a dict) their mean
    and sample standard deviation in ms are stored there."""
    x, tags, pos = rows
    fwd = lambda: lib.dit_forward(dims, x, tags, pos, table, blocks, ws)
    for i in range(warmup):
        fwd()
        torch.cuda.synchronize()
        log(f"warmup forward {i + 1}/{warmup} done")
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fwd()
        ev[i + 1].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert bool(torch.isfinite(x).all()), "non-finite output"
    if per_step is not None:
        ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        mean = sum(ms) / len(ms)
        sd = (sum((m - mean) ** 2 for m in ms) / (len(ms) - 1)) ** 0.5 if len(ms) > 1 else 0.0
        per_step.update({"mean_ms": round(mean, 2), "sd_ms": round(sd, 2), "n": len(ms)})
    return dt / steps


def env_receipt(torch):
    """What the numbers were measured on: device, software versions."""
    p = torch.cuda.get_device_properties(0)
    return {"device": p.name, "gcn_arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1), "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None)}


def cpu_baseline(n_target, n_blocks, dims_h3):
    """The oracle as it stands (float64 numpy), timed on the host cores on a
    bounded sample: one full H3-width block at N = 6,437 (the secondary
    workload's packed layout) and at N = 1,192, each after one excluded warmup
    run and then timed three times (mean and sample SD), with the attention step
    timed on its own in every run.  The N = 6,437 block, split into its linear
    part (scaled by N) and its attention (scaled by N^2), gives the 50-block
    N = n_target forward's rate."""
    import statistics

    import numpy as np  # noqa: F401

    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()

    def sample(name, reps=3):
        wl = synth.WORKLOADS[name]
        x, tags, pos, table, weights = synth.make_inputs(wl, seed=0, n_blocks=1)
        runs = []
        for r in range(reps + 1):
            t0 = time.perf_counter()
            st = oracle.block_steps(x, tags, pos, table[0], weights[0], wl.dims)
            t_block = time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.attention(st["q"], st["k"], st["v"])
            t_attn = time.perf_counter() - t0
            if r > 0:                                  # run 0 is the excluded warmup
                runs.append((t_block, t_attn))
        blk = [b for b, _ in runs]
        att = [a for _, a in runs]
        return wl.n_rows, {"n_rows": wl.n_rows, "block_s_mean": round(statistics.mean(blk), 3),
                           "block_s_sd": round(statistics.stdev(blk), 3), "attention_s_mean":
                           round(statistics.mean(att), 3), "attention_s_sd": round(statistics.stdev(att), 3),
                           "reps": reps, "warmup": 1}
    n_small, small = sample("h3_1blk_n1192")
    n_big, big = sample("h3_50blk_n6437")
    t_attn = big["attention_s_mean"]
    t_rest = max(big["block_s_mean"] - t_attn, 1e-9)
    t_fwd = n_blocks * (t_rest * n_target / n_big + t_attn * (n_target / n_big) ** 2)
    cpu_model, blas = "unknown", "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                                 if i.get("user_api") == "blas"})) or blas
    except Exception:
        pass
    return {"value": round(n_target / t_fwd, 4), "unit": "packed tokens/s", "cores": cores,
            "host": {"cpu_model": cpu_model, "nproc": os.cpu_count(), "blas": blas},
            "kind": "oracle", "precision": "float64",
            "measured": {"n6437_block": big, "n1192_block": small},
            "sample": (f"one float64 oracle block of the H3 model at N={n_big} took "
                       f"{big['block_s_mean']:.2f} +- {big['block_s_sd']:.2f} s (3 runs after a warmup; "
                       f"attention {t_attn:.2f} s), at N={n_small} {small['block_s_mean']:.2f} +- "
                       f"{small['block_s_sd']:.2f} s; the N={n_big} block scaled to the {n_blocks}-block "
                       f"N={n_target} forward (linear part x N, attention x N^2)")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="h3_50blk_n49840")
    ap.add_argument("--secondary", default="h3_50blk_n6437", help="'none' to skip")
    ap.add_argument("--secondary-steps", type=int, default=5)
    ap.add_argument("--extra", default="h3_50blk_n7461",
                    help="comma-separated further 50-block workloads timed like the secondary ('none' to skip)")
    ap.add_argument("--breakdown-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --only-step: first run a 1 GiB device-to-device copy three times, "
                         "the known-size reference for HBM byte counters")
    ap.add_argument("--single-block", type=int, default=1,
                    help="also time one H3 block at N=1192 with bf16 and INT8 weights, and whole INT8 and bf16 blocks at N=1192 and the primary size (0: skip)")
    ap.add_argument("--denoise-reuse", type=int, default=2,
                    help="also time the denoising loop with this whole-velocity reuse (1: skip)")
    ap.add_argument("--denoise-steps", type=int, default=4,
                    help="Euler passes of the denoising loop timed at the secondary workload (0: skip)")
    ap.add_argument("--sparse", type=int, default=1,
                    help="also time block-sparse attention and the sparse forward (0: skip)")
    ap.add_argument("--w8a8", type=int, default=1,
                    help="also run the forwards with the W8A8 trunk (0: skip)")
    ap.add_argument("--only-step", default=None,
                    help="time just one step kernel (adaln, qkv_rope, attention, out_proj_resid, "
                         "fc1_swiglu, fc2_resid; with a W8A8 workload also quant_h, quant_o, "
                         "quant_a) on one block's weights, e.g. under a counter run; "
                         "vendor_fc1 / vendor_gemms time the vendor library's plain GEMMs of the "
                         "FC1 / all four linear shapes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from joint_video_audio_h3_amd import lib

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib.load()
    wl = synth.WORKLOADS[args.workload]
    dims = wl.dims
    if args.only_step:
        if args.copy_calibration:
            src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        if args.only_step in ("vendor_fc1", "vendor_gemms"):
            # the vendor library's plain bf16 GEMMs of the block's linear shapes
            # (bf16 out, no epilogue), timed for comparison with the fused kernels
            n, D, Di, F = wl.n_rows, dims.hidden, dims.inner, dims.ffn
            shapes = {"fc1": (D, 2 * F)}
            if args.only_step == "vendor_gemms":
                shapes = {"qkv": (D, 3 * Di), "out_proj": (Di, D), "fc1": (D, 2 * F), "fc2": (F, D)}
            out = {"workload": wl.name, "step": args.only_step}
            total = 0.0
            for name, (K, N) in shapes.items():
                a = torch.randn(n, K, dtype=torch.bfloat16, device="cuda")
                w = torch.randn(N, K, dtype=torch.bfloat16, device="cuda")
                for _ in range(2):
                    c = a @ w.t()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(True), torch.cuda.Event(True)
                e0.record()
                for _ in range(args.breakdown_reps):
                    c = a @ w.t()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / args.breakdown_reps
                total += ms
                out[name] = {"ms": round(ms, 4), "tflops": round(2.0 * n * K * N / ms / 1e9, 1)}
                del a, w, c
            if len(shapes) > 1:
                out["sum_ms"] = round(total, 4)
            print(json.dumps(out))
            return
        table, blocks = synth.make_device_weights(dims, 1, seed=0)
        fn = step_breakdown_w8a8 if dims.wfmt == synth.WFMT_W8A8 else step_breakdown
        bd, _ = fn(lib, dims, synth.make_device_rows(wl, seed=1), table, blocks[0],
                   args.breakdown_reps, torch, only=args.only_step)
        print(json.dumps({"workload": wl.name, "step": args.only_step, **bd[args.only_step]}))
        return
    log(f"generating {wl.n_blocks} blocks of weights on the device")
    table, blocks = synth.make_device_weights(dims, wl.n_blocks, seed=0)
    torch.cuda.synchronize()

    measured_steps = {}

    def measure(wlx, steps, warmup):
        rows = synth.make_device_rows(wlx, seed=0)
        ws = lib.alloc_workspace(dims, wlx.n_rows)
        ps = {}
        sec = run_forward(lib, dims, rows, table[:wlx.n_blocks], blocks[:wlx.n_blocks], ws,
                          steps, warmup, torch, per_step=ps)
        measured_steps[wlx.name] = ps
        log(f"{wlx.name}: {sec * 1e3:.1f} ms per forward")
        bd, w = step_breakdown(lib, dims, synth.make_device_rows(wlx, seed=1), table, blocks[0],
                               args.breakdown_reps, torch)
        del ws
        return sec, bd, w

    sec, bd, w = measure(wl, args.steps, args.warmup)
    n = wl.n_rows
    flop_fwd = wl.n_blocks * w.total_flop
    dom = max(("attention", "fc1_swiglu", "qkv_rope", "fc2_resid", "out_proj_resid"),
              key=lambda s: bd[s]["ms"])
    dom_flop = {"attention": w.attn_flop, "fc1_swiglu": w.fc1_flop, "qkv_rope": w.qkv_flop,
                "fc2_resid": w.fc2_flop, "out_proj_resid": w.out_flop}[dom]
    ach = dom_flop / (bd[dom]["ms"] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK,
                "unit": "TFLOP/s", "frac": round(ach / PEAK, 4),
                "traffic": measured_traffic(wl.name, dom)}
    result = {
        "metric": "packed tokens/s per DiT forward (+ MFMA util)",
        "value": round(n / sec, 2),
        "unit": "packed tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (random-init weights of the H3 shapes, N(0,1) latents)",
        "config": {"workload": wl.name, "n_rows": n, "blocks": wl.n_blocks, "hidden": dims.hidden,
                   "heads": dims.heads, "head_dim": dims.head_dim, "ffn": dims.ffn,
                   "packed": {"L": wl.L, "C": wl.C, "A": wl.A, "V": list(wl.V)}},
        "step_events": measured_steps[wl.name],
        "env": env_receipt(torch),
        "forward_tflops": round(flop_fwd / sec / 1e12, 1),
        "forward_mfma_frac": round(flop_fwd / sec / 1e12 / PEAK, 4),
        "per_step_kernels": bd,
        "roofline": roofline,
    }
    # the steps around the block stack (once per forward), at this workload's segments
    io = synth.H3_IO
    result["io_kernels"] = io_breakdown(lib, dims, io, wl, args.breakdown_reps, torch)
    result["io_kernels"]["share_of_velocity_forward"] = round(
        (result["io_kernels"]["embed_inputs"]["ms"] + result["io_kernels"]["final_heads"]["ms"])
        / (sec * 1e3 + result["io_kernels"]["embed_inputs"]["ms"]
           + result["io_kernels"]["final_heads"]["ms"]), 5)
    if args.secondary != "none":
        wl2 = synth.WORKLOADS[args.secondary]
        sec2, bd2, w2 = measure(wl2, args.secondary_steps, 1)
        result["secondary"] = {
            "workload": wl2.name, "n_rows": wl2.n_rows, "value": round(wl2.n_rows / sec2, 2),
            "unit": "packed tokens/s", "ms_per_step": round(sec2 * 1e3, 2),
            "steps": args.secondary_steps, "step_events": measured_steps[wl2.name],
            "forward_tflops": round(wl2.n_blocks * w2.total_flop / sec2 / 1e12, 1),
            "forward_mfma_frac": round(wl2.n_blocks * w2.total_flop / sec2 / 1e12 / PEAK, 4),
            "per_step_kernels": bd2,
        }
    for name in [x for x in args.extra.split(",") if x and x != "none"]:
        wl3 = synth.WORKLOADS[name]
        sec3, bd3, w3 = measure(wl3, args.secondary_steps, 1)
        result.setdefault("extra", {})[name] = {
            "n_rows": wl3.n_rows, "packed": {"L": wl3.L, "C": wl3.C, "A": wl3.A, "V": list(wl3.V)},
            "value": round(wl3.n_rows / sec3, 2), "unit": "packed tokens/s",
            "ms_per_step": round(sec3 * 1e3, 2), "steps": args.secondary_steps,
            "step_events": measured_steps[wl3.name],
            "forward_tflops": round(wl3.n_blocks * w3.total_flop / sec3 / 1e12, 1),
            "forward_mfma_frac": round(wl3.n_blocks * w3.total_flop / sec3 / 1e12 / PEAK, 4),
            "per_step_kernels": bd3,
        }
    if args.denoise_steps > 0 and args.secondary != "none":
        # the denoising loop at the secondary workload: inputs -> velocity ->
        # Euler, video shift 12 and audio shift 3, tables per pass
        wl2 = synth.WORKLOADS[args.secondary]
        steps_d = args.denoise_steps
        log(f"denoising loop: {wl2.name}, {steps_d} passes")
        io = synth.H3_IO
        g = torch.Generator(device="cuda")
        g.manual_seed(11)
        tabs = (torch.randn(steps_d, wl2.n_blocks, dims.n_tags, 6, dims.hidden, generator=g, device="cuda")
                * 0.316).to(torch.bfloat16)
        fins = (torch.randn(steps_d, 2, 2, dims.hidden, generator=g, device="cuda") * 0.316).to(torch.bfloat16)
        inp = synth.make_io_inputs(wl2, io, seed=0)
        w_host = synth.make_io_weights(dims, io, seed=0)
        dv = lambda a: (None if a is None or len(a) == 0 else  # noqa: E731
                        torch.from_numpy(a.view("int16") if a.dtype.name == "uint16" else a).cuda())
        iw = {k: dv(v) for k, v in w_host.items()}
        d = {k: dv(v) for k, v in inp.items()}
        _, tags2, pos2 = synth.make_device_rows(wl2, seed=0)
        x2 = torch.empty(wl2.n_rows, dims.hidden, dtype=torch.float32, device="cuda")
        ws2 = lib.alloc_denoise_workspace(dims, io, d["text"], d["cond"], d["audio"], d["video"])
        sa, sv = lib.sigma_schedule(steps_d, 3.0), lib.sigma_schedule(steps_d, 12.0)
        def timed_loop(reuse):
            run = lambda: lib.denoise(dims, io, iw, d["text"], d["cond"], d["audio"], d["video"], tags2,  # noqa: E731
                                      pos2, tabs, blocks[:wl2.n_blocks], fins, sa, sv, x2, ws2, reuse=reuse)
            run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run()
            torch.cuda.synchronize()
            return time.perf_counter() - t0
        secd = timed_loop(1)
        assert bool(torch.isfinite(d["video"]).all()), "non-finite latents"
        result["denoise"] = {"workload": wl2.name, "passes": steps_d, "shifts": {"video": 12.0, "audio": 3.0},
                             "s_per_loop": round(secd, 4), "ms_per_pass": round(secd / steps_d * 1e3, 2),
                             "packed_tokens_per_s_per_pass": round(wl2.n_rows * steps_d / secd, 2),
                             "pass_over_dit_forward": round(secd / steps_d / result["secondary"]["ms_per_step"]
                                                            * 1e3, 4)}
        log(f"denoising loop: {secd * 1e3:.1f} ms for {steps_d} passes")
        if args.denoise_reuse > 1:
            # whole-velocity reuse: fresh evaluations at i % r == 0 and the last pass
            secr = timed_loop(args.denoise_reuse)
            fresh = sum(1 for i in range(steps_d) if i % args.denoise_reuse == 0 or i == steps_d - 1)
            result["denoise"]["reuse"] = {"reuse": args.denoise_reuse, "fresh_passes": fresh,
                                          "s_per_loop": round(secr, 4),
                                          "ms_per_fresh_pass": round(secr / fresh * 1e3, 2),
                                          "speedup_vs_reuse_1": round(secd / secr, 3)}
            log(f"denoising loop, reuse {args.denoise_reuse}: {secr * 1e3:.1f} ms ({fresh} fresh passes)")
        del ws2, x2, tabs, fins
    if args.sparse:
        # block-sparse attention (a fixed budget of key tiles per query tile)
        # at the primary workload: the kernel alone, then the 50-block forward
        log("block-sparse attention")
        result["sparse"] = sparse_breakdown(lib, dims, n, args.breakdown_reps, torch)
        tile, keep = 128, result["sparse"]["keep"]
        import numpy as np
        n_masks = 10     # distinct selections, cycled over the blocks
        masks = [synth.make_tile_mask(n, dims.heads, tile, keep, dense_rows=wl.L + wl.C, seed=b)
                 for b in range(n_masks)]
        bases = np.cumsum([0] + [len(m[1]) for m in masks])
        offd = torch.from_numpy(np.concatenate([(masks[b % n_masks][0] + bases[b % n_masks]).astype(np.int32)
                                                for b in range(wl.n_blocks)])).cuda()
        log("sparse forward masks ready")
        idxd = torch.from_numpy(np.concatenate([m[1] for m in masks])).cuda()
        x, tags, pos = synth.make_device_rows(wl, seed=0)
        ws = lib.alloc_workspace(dims, n)
        fwd = lambda: lib.dit_forward_sparse(dims, x, tags, pos, table, blocks, tile, offd, idxd, ws)  # noqa: E731
        fwd()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fwd()
        torch.cuda.synchronize()
        secs = (time.perf_counter() - t0) / args.steps
        assert bool(torch.isfinite(x).all()), "non-finite output"
        result["sparse"]["forward"] = {"tile": tile, "value": round(n / secs, 2), "unit": "packed tokens/s",
                                       "ms_per_step": round(secs * 1e3, 2), "steps": args.steps,
                                       "speedup_vs_dense": round((n / secs) / result["value"], 3),
                                       "masks": "10 generator selections (seeds 0..9) cycled over the blocks"}
        log(f"sparse forward: {secs * 1e3:.1f} ms")
        del ws, x, offd, idxd
    if args.w8a8:
        # the same forwards with the group-scaled W8A8 trunk (int8 weights and
        # activations, one scale per 896 K elements) on the int8 matrix cores
        del table, blocks
        torch.cuda.empty_cache()
        result["w8a8"] = {}
        names = [args.workload] + ([args.secondary] if args.secondary != "none" else [])
        dims8 = synth.WORKLOADS[names[0] + "_w8a8"].dims
        log("generating 50 blocks of W8A8 weights on the device")
        table8, blocks8 = synth.make_device_weights(dims8, wl.n_blocks, seed=0)
        for nm in names:
            wl8 = synth.WORKLOADS[nm + "_w8a8"]
            rows = synth.make_device_rows(wl8, seed=0)
            ws = lib.alloc_workspace(dims8, wl8.n_rows)
            steps8 = args.steps if nm == args.workload else args.secondary_steps
            sec8 = run_forward(lib, dims8, rows, table8[:wl8.n_blocks], blocks8[:wl8.n_blocks], ws,
                               steps8, 1, torch)
            log(f"{wl8.name}: {sec8 * 1e3:.1f} ms per forward")
            del ws
            bd8, w8 = step_breakdown_w8a8(lib, dims8, synth.make_device_rows(wl8, seed=1), table8,
                                          blocks8[0], args.breakdown_reps, torch)
            result["w8a8"][wl8.name] = {
                "n_rows": wl8.n_rows, "value": round(wl8.n_rows / sec8, 2), "unit": "packed tokens/s",
                "ms_per_step": round(sec8 * 1e3, 2), "steps": steps8,
                "speedup_vs_bf16": round((wl8.n_rows / sec8) / (result["value"] if nm == args.workload
                                                                 else result["secondary"]["value"]), 3),
                "per_step_kernels": bd8}
        del table8, blocks8
        torch.cuda.empty_cache()
    if args.single_block:
        # one H3 block at N=1192, bf16 and INT8 W8A16 weights: per-step kernel
        # times (the block-parity shape; the INT8 variant's MFMA utilization)
        result["single_block"] = {}
        for name in ("h3_1blk_n1192", "h3_1blk_n1192_int8"):
            wl1 = synth.WORKLOADS[name]
            t1, b1 = synth.make_device_weights(wl1.dims, 1, seed=0)
            bd1, _ = step_breakdown(lib, wl1.dims, synth.make_device_rows(wl1, seed=1), t1, b1[0],
                                    args.breakdown_reps, torch)
            result["single_block"][name] = {"weights": "int8 g32 + bf16 scales" if wl1.dims.wfmt else "bf16",
                                            "per_step_kernels": bd1}
            del t1, b1
        # whole INT8 W8A16 blocks against bf16 blocks (HIP events): with the full
        # workspace the forward dequantises each linear's weights once and runs
        # the bf16 GEMM; with the smaller one, the kernel that dequantises in LDS
        result["int8_w8a16_block"] = {}
        d8 = synth.WORKLOADS["h3_1blk_n1192_int8"].dims
        for wname in ("h3_1blk_n1192", wl.name):
            wlr = synth.WORKLOADS[wname]
            rows_ = synth.make_device_rows(wlr, seed=1)
            r = {"n_rows": wlr.n_rows}
            for key, dd in (("bf16", wlr.dims), ("int8", d8)):
                t1, b1 = synth.make_device_weights(dd, 1, seed=0)
                full = lib.alloc_workspace(dd, wlr.n_rows)
                wss = {"": full}
                if dd.wfmt:
                    wss["_lds_dequant"] = full[:lib.workspace_size(wlr.dims, wlr.n_rows)]
                for suffix, ws_ in wss.items():
                    xs = rows_[0].clone()
                    ms = _time_launches(lambda: lib.dit_block_forward(dd, xs, rows_[1], rows_[2], t1[0], b1[0], ws_),
                                        args.breakdown_reps, torch)
                    r[f"{key}{suffix}_block_ms"] = round(ms, 4)
                del t1, b1, full, wss
                torch.cuda.empty_cache()
            r["int8_over_bf16"] = round(r["int8_block_ms"] / r["bf16_block_ms"], 4)
            result["int8_w8a16_block"][wname] = r
            del rows_
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(n, wl.n_blocks, dims)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of one frame of the tile-binned splat rasterizer on one MI355X.

A step is the whole hot path on one batch of synthetic input already resident in HBM: intersection count (one
8-byte readback for the size; the splats' depth order is computed behind it), key emission and the stable sort
of the tile bits, tile ranges and compositing. The default workload is
the 1M-splat 1920x1080 frame (64-component clustered mixture, tile 16). Prints one JSON line.

Frames are independent, so the timed steps keep --frames-in-flight frames in flight on as many streams, each fed
by its own host thread (each frame whole, on its own buffers): one frame's latency-bound intersection chain
overlaps another's compositing. The
per-frame latency with one frame at a time is measured first and reported beside the throughput, with the
per-stage times. Before each timed part the frame runs untimed for a quarter of a second (settle), so that a short
run measures the settled device rather than its first frames after an idle start.

    python bench.py [--steps K] [--warmup W] [--config config3] [--frames-in-flight F] [--no-cpu-baseline]

Only one GPU is supported: --gpus above 1 (or a multi-rank launch) exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "isect keys sorted/s; rasterized Mpix/s (1M splats, 1920x1080, 1 GPU)"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# VALU issue limit: each of the 256 x 4 SIMDs issues at most 2 wave64 VALU instructions per 4 cycles (dual issue:
# FP32 add/mul/fma, v_mov and v_add_u32 pair with each other and with compares, selects and conversions, which never
# pair among themselves; measured by the calibration kernels), 64 lanes each, at 2.4 GHz: 78.64 T lane-instructions
# per second, the 157.3 TFLOP/s FP32 figure at 2 flops per fma. Reachable when at least half of a kernel's VALU
# instructions can pair and none is transcendental (the composite: 62% FP32 add/mul/fma, 0.2% transcendental).
PEAK_VALU_TOPS = 256 * 4 * 64 * 2 / 4 * 2.4e9 / 1e12
# VALU wave-instructions per launch of the composite and its backward on the 1M-splat frame, from the profiler's
# instruction counter (exact: calibrated against kernels of known count); valid only while the kernel sources are
# the ones the counters were taken on
VALU_FILE = os.path.join(ROOT, "profiles", "raster_valu_instructions_config3.txt")
BWD_SOURCES = [os.path.join(ROOT, "tile_binned_gaussian_amd", "csrc", f) for f in ("raster_bwd.hip", "raster_common.hpp")]
# lane-operations per evaluation of the composite's definition:
#   every evaluation: 2 (delta) + 9 (quadratic form) + 1 (sign test) + 14 (exponential incl. the >80 test)
#                     + 1 (opacity product) + 1 (clamp) + 1 (cutoff test) = 29
#   alpha >= cutoff:  1 (1 - alpha) + 1 (T product) + 1 (threshold test) = 3
#   composited:       1 (alpha T) + 2 K (colour multiply-add, unfused) = 7 for K = 3
OPS_EVAL, OPS_PASS = 29, 3
# HBM bytes the composite kernel moved per launch on the 1M-splat frame, from two profiler counter runs; valid only
# while the kernel source is the one the counters were taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "raster_cull_kernel_config3_hbm_traffic.txt")
RASTER_SOURCES = [os.path.join(ROOT, "tile_binned_gaussian_amd", "csrc", f)
                  for f in ("raster.hip", "raster_common.hpp")]

WORKLOADS = {
    "tiny": "tiny: 1 camera, 256 splats, 64x64, tile 16",
    "config2": "1 camera, 200k splats (uniform, elliptical radii), 800x800, tile 16",
    "config3": "1 camera, 1M splats (64-component clustered mixture), 1920x1080 (120x68 tiles), tile 16",
    "config4": "4 cameras x 3M splats (per-camera mixtures, 1% radius 0), 1600x1064, tile 16",
    "config5": "1 camera, 6M splats (uniform, r median 6 px, 10% duplicate depths, half opacity < 1/255), "
               "3840x2160, tile 16",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="config3", choices=sorted(WORKLOADS))
    ap.add_argument("--frames-in-flight", type=int, default=2,
                    help="frames in flight at once on separate streams and host threads in the timed steps "
                         "(1 = one at a time)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=0,
                    help="runs per oracle stage in the CPU baseline, median reported (0: 3 for the three smaller "
                         "workloads, 1 for the two largest)")
    ap.add_argument("--cpu-tile-stride", type=int, default=4,
                    help="CPU baseline composites every k-th tile (then scales to the frame)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 device-to-device copies of exactly 1 GiB (a known-size reference for the HBM "
                         "byte counters of a profiler run)")
    ap.add_argument("--valu-calibration", action="store_true",
                    help="also run the VALU calibration kernels (a known vector-instruction count per wave, for the "
                         "instruction counter of a profiler run, and the measured issue rate and shader clock)")
    return ap.parse_args()


CALIB_KINDS = ["v_fmac_f32", "v_mul_f32", "v_cndmask_b32", "v_mov_b32_dpp", "v_exp_f32", "v_cmp_gt_f32",
               "mix(4 fmac,2 mul,1 cndmask,1 exp)", "v_add_f32", "v_sub_f32", "v_fma_f32", "v_fmaak_f32",
               "v_mov_b32", "v_add_u32", "v_rndne_f32", "v_ldexp_f32", "v_cvt_i32_f32", "v_max_f32",
               "composite mix(5 mul,2 add,1 sub,2 fma,2 cndmask,2 cmp,1 rndne,1 ldexp)"]


def valu_calibration(stream):
    """Each calibration kernel 3 times at 1024 rounds, then 3 times at 2048 rounds (16 vector instructions per
    round and wave, every lane active, 8 waves per SIMD). The difference between the two round counts cancels the
    kernels' fixed prologue and epilogue: 16 x 1024 x waves wave-instructions, which is what a profiler's VALU
    instruction counter must read between the two dispatch groups. Returns per kind the lane-instruction rate, the
    wave-instructions issued per SIMD per shader cycle, and the shader clock read from s_memtime against the
    constant-rate s_memrealtime."""
    import ctypes
    import numpy as np
    import torch
    from tile_binned_gaussian_amd import build as hip_build
    lib = ctypes.CDLL(hip_build.CALIB_LIB)
    lib.gs_calib_valu_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.gs_calib_valu_launch.restype = ctypes.c_int
    lib.gs_calib_wall_clock_khz.restype = ctypes.c_int
    blocks = 256 * 8
    waves = blocks * 4
    simds = 256 * 4
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    clocks = torch.zeros(waves * 4, dtype=torch.int64, device="cuda:0")
    s = ctypes.c_void_p(stream.cuda_stream)
    wall_hz = lib.gs_calib_wall_clock_khz() * 1e3
    res = {"blocks": blocks, "waves": waves, "rounds": [1024, 2048], "instructions_per_round": 16,
           "counter_delta_expected": 16 * 1024 * waves, "wall_clock_hz": wall_hz, "kinds": {}}
    for kind, name in enumerate(CALIB_KINDS):
        ms = {}
        for iters in (1024, 2048):
            t = []
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                rc = lib.gs_calib_valu_launch(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                              ctypes.c_void_p(clocks.data_ptr()), s)
                b.record(stream)
                if rc != 0:
                    raise RuntimeError(f"calibration launch failed: {rc}")
                b.synchronize()
                t.append(a.elapsed_time(b))
            ms[iters] = statistics.median(t)
        c = clocks.view(waves, 4).cpu().numpy().astype(np.float64)
        shader_hz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1.0))) * wall_hz
        dt = (ms[2048] - ms[1024]) * 1e-3
        lane_instr = 16 * 1024 * waves * 64
        rate = lane_instr / dt
        res["kinds"][name] = {
            "ms_1024": round(ms[1024], 4), "ms_2048": round(ms[2048], 4),
            "T_lane_instructions_per_s": round(rate / 1e12, 3),
            "wave_instructions_per_simd_cycle": round(16 * 1024 * waves / simds / (dt * shader_hz), 4),
            "shader_clock_GHz": round(shader_hz / 1e9, 4)}
    return res


SETTLE_S = 0.25


def settle(run):
    """Untimed frames for at least SETTLE_S seconds before a warm-up and its timed steps: the device idles while
    the process starts and allocates, and its first ~20 ms of frames after an idle period run up to 15% slower (a
    kernel trace shows the composite falling from ~430 to ~380 us over them), so a short timed run would otherwise
    measure that transition. Returns the milliseconds spent."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        run()
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def stage_bytes(scene, n, tile_passes, generic_passes):
    """Algorithmic HBM bytes per stage (what each step must read and write at least once)."""
    M = scene.C * scene.N
    rb = 8 if scene.radii.ndim == 3 else 4
    pixels = scene.C * scene.width * scene.height
    K = scene.colors.shape[-1]
    return {
        # phase 1: the count scan (means, radii and depths read once, counts and offsets written), the depth order
        # of the splats (4 passes of 4-byte keys and ids read and written) and the offsets in that order (a count per
        # splat gathered, the offset written; the last depth pass computes them)
        "count_depth_order": M * (8 + rb + 4 + 4 + 4) + M * 4 * 16 + M * (4 + 4),
        # phase 2: emission in depth order (order, depth bits, offset, mean, radius per splat; 12 bytes per
        # intersection written; the digit histograms are built on the way) and tile_passes passes of 24 B per
        # intersection
        "emit_sort": M * (4 + 4 + 4 + 8 + rb) + n * 12 + tile_passes * n * 24,
        "ranges": n * 8 + scene.C * scene.tile_width * scene.tile_height * 4,
        "composite": n * (4 + 8 + 12 + 4 + 4 * K) + pixels * (4 * K + 4 + 4 + 4),
        "generic_sort": n * 8 + generic_passes * n * 24 + (n * 24 if generic_passes % 2 else 0),
    }


def _record(path):
    with open(path) as f:
        return {k.strip(): v.strip() for k, v in (line.split(":", 1) for line in f.read().splitlines()
                                                  if ":" in line and not line.startswith(" "))}


def _sha(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_valu(config, which):
    """Profiler-counted VALU wave-instructions per launch of the composite ("composite") or its backward
    ("backward") on this workload, or None if there is no record or the kernel source changed since."""
    try:
        rec = _record(VALU_FILE)
        sha = _sha(RASTER_SOURCES if which == "composite" else BWD_SOURCES)
    except OSError:
        return None
    if rec.get("workload") != config or rec.get(f"{which}_kernel_source_sha256") != sha:
        return None
    return int(rec[f"{which}_valu_wave_instructions_per_launch"])


def measured_traffic(config):
    """Counter-measured HBM bytes per composite launch, or None if there is no record for this workload or the
    kernel source changed since the record was taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = dict(line.split(":", 1) for line in f.read().splitlines() if ":" in line and not line.startswith(" "))
        h = hashlib.sha256()
        for path in RASTER_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()
    except OSError:
        return None
    rec = {k.strip(): v.strip() for k, v in rec.items()}
    if rec.get("workload") != config or rec.get("kernel_source_sha256") != sha:
        return None
    return int(rec["hbm_bytes_per_launch"])


def _cpu_mask():
    """The host's logical CPU count and this process's affinity mask, as ranges ("0-15")."""
    try:
        cpus = sorted(os.sched_getaffinity(0))
    except AttributeError:
        cpus = list(range(os.cpu_count() or 1))
    runs, start = [], None
    for i, c in enumerate(cpus):
        if start is None:
            start = c
        if i + 1 == len(cpus) or cpus[i + 1] != c + 1:
            runs.append(f"{start}-{c}" if c != start else f"{c}")
            start = None
    return os.cpu_count(), ",".join(runs)


def _oracle_stages(scene, tiles, openmp, reps):
    """Per-stage wall times of the oracle on the frame (median over reps runs, each stage timed on its own):
    count + scan, emission, sort, tile offsets over the whole frame, and the composite on the given tiles."""
    import numpy as np
    import oracle
    runs = []
    for _ in range(reps):
        tm = {}
        it = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                                scene.tile_height, sort=True, openmp=openmp, timings=tm)
        t0 = time.perf_counter()
        off = oracle.tile_offsets(it.keys, scene.C, scene.tile_width, scene.tile_height)
        t1 = time.perf_counter()
        oracle.rasterize_fwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                             scene.width, scene.height, scene.tile_size, off, it.flatten_ids, it.n_isects,
                             scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold,
                             tiles=tiles if tiles is not None else np.arange(0, off.size, 1, dtype=np.int64),
                             openmp=openmp)
        t2 = time.perf_counter()
        tm.update(offsets_s=t1 - t0, composite_sample_s=t2 - t1)
        runs.append(tm)
    return {k: statistics.median(r[k] for r in runs) for k in runs[0]}, it, off


def _cpu_report(scene, st, it, off, tiles, threads, kind, reps):
    composite_s = st["composite_sample_s"] * off.size / tiles.size
    isect_s = st["count_scan_s"] + st["emit_s"] + st["sort_s"] + st["offsets_s"]
    frame_s = isect_s + composite_s
    nproc, mask = _cpu_mask()
    return {
        "value": scene.C * scene.width * scene.height / frame_s / 1e6, "unit": "Mpix/s", "cores": threads,
        "kind": kind,
        "sample": f"median of {reps} runs per stage: count+scan, emission, sort and tile offsets over the whole frame, "
                  f"the composite on every {off.size // tiles.size}-th tile ({tiles.size} of {off.size}) scaled to "
                  f"all tiles; {threads} thread(s)",
        "frame_s_estimate": round(frame_s, 3),
        "stages_s": {"count_scan": round(st["count_scan_s"], 4), "emit": round(st["emit_s"], 4),
                     "sort": round(st["sort_s"], 4), "tile_offsets": round(st["offsets_s"], 4),
                     "composite_scaled": round(composite_s, 3)},
        "keys_sorted_per_s": it.n_isects / st["sort_s"] if st["sort_s"] > 0 else None,
        "isect_sort_offsets_s": round(isect_s, 3),
        "host_nproc": nproc, "affinity": mask, "reps": reps,
    }


def cpu_baseline(scene, stride, reps):
    """The oracle as it stands, single thread: every stage timed, median of reps runs (see _oracle_stages)."""
    import numpy as np
    import oracle
    tiles = np.arange(0, scene.C * scene.tile_width * scene.tile_height, stride, dtype=np.int64)
    st, it, off = _oracle_stages(scene, tiles, False, reps)
    return _cpu_report(scene, st, it, off, tiles, oracle.threads(openmp=False), "oracle", reps), tiles


def cpu_baseline_openmp(scene, tiles, reps):
    """The same oracle built with OpenMP (the pages' CPU parallelisation: emission and the sort's merges over
    splats, the composite over tiles with dynamic scheduling) on the host's threads, same stages and tile sample."""
    import oracle
    st, it, off = _oracle_stages(scene, tiles, True, reps)
    return _cpu_report(scene, st, it, off, tiles, oracle.threads(openmp=True), "oracle (OpenMP build)", reps)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the frame is "
              f"rasterized on one GPU and is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from tile_binned_gaussian_amd import binding, frame, synth

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    scene = synth.CONFIGS[args.config]()
    ds = frame.to_device(scene, "cuda:0")
    plan = frame.FramePlan(ds)

    # untimed: count the work the composite's definition implies on this frame
    counts = torch.zeros(5, dtype=torch.int64, device="cuda:0")
    plan.run(eval_counts=counts)
    torch.cuda.synchronize()
    n_eval, n_pass, n_comp, n_exec, n_staged = (int(v) for v in counts.cpu())

    # the timing events exist before the warm-up, so that nothing leaves the device idle between the warm-up and
    # the timed frames
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    settle_ms = settle(plan.run)
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        plan.run(events=events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = plan.n_isects

    names = ["count_depth_order", "emit_sort", "ranges", "composite"]
    stage_ms = {nm: statistics.median(events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps))
                for i, nm in enumerate(names)}
    latency_ms = wall * 1e3 / args.steps
    # the timed steps: frames-in-flight frames at once, each on its own stream and buffers, each stream fed by its
    # own host thread (a frame's host thread waits for its intersection count; the others keep queueing work)
    F = max(1, args.frames_in_flight)
    if F == 1:
        ms_per_step = latency_ms
    else:
        flight = [frame.FramePlan(ds, stream=torch.cuda.Stream()) for _ in range(F)]

        def pipelined(steps):
            """`steps` frames in all, spread over the F plans, each plan fed by its own host thread; returns the
            seconds from the threads' common start to the device's last frame (synchronized on both sides)."""
            share = [steps // F + (1 if i < steps % F else 0) for i in range(F)]
            gate = threading.Barrier(F + 1)
            errors = []

            def feed(p, count):
                gate.wait()
                try:
                    for _ in range(count):
                        p.run()
                except Exception as e:  # re-raised on the main thread below
                    errors.append(e)
            workers = [threading.Thread(target=feed, args=(p, c)) for p, c in zip(flight, share)]
            for w in workers:
                w.start()
            torch.cuda.synchronize()
            gate.wait()
            t0 = time.perf_counter()
            for w in workers:
                w.join()
            torch.cuda.synchronize()
            if errors:
                raise errors[0]
            return time.perf_counter() - t0
        # the settle and the warm-up steps run the same way as the timed ones (threads, streams and all), so the
        # timed steps are not the first the threaded path runs in this process
        settle(lambda: pipelined(2 * F))
        pipelined(max(args.warmup, F))
        ms_per_step = pipelined(args.steps) * 1e3 / args.steps  # exactly K steps
        assert all(p.n_isects == plan.n_isects for p in flight)
        del flight
    # outside the frame: the composite's backward on the last frame (seeded output gradients)
    bwd = frame.BackwardPlan(plan, seed=0)
    for _ in range(2):
        bwd.run()
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(5, args.steps // 2))]
    for a_ev, b_ev in bev:
        a_ev.record(plan.stream)
        bwd.run()
        b_ev.record(plan.stream)
    torch.cuda.synchronize()
    backward_ms = statistics.median(a_ev.elapsed_time(b_ev) for a_ev, b_ev in bev)
    # outside the frame: the traced forward on the last frame (every pixel's composited splat ids, up to 256)
    S_TRACE = 256
    C_, H_, W_, K_ = scene.C, scene.height, scene.width, scene.colors.shape[-1]
    f32, i32 = dict(device="cuda:0"), dict(dtype=torch.int32, device="cuda:0")
    tr_out = binding.TracedRender(torch.empty((C_, H_, W_, K_), **f32), torch.empty((C_, H_, W_), **f32),
                                  torch.empty((C_, H_, W_), **f32), torch.empty((C_, H_, W_), **i32),
                                  torch.empty((C_, H_, W_, S_TRACE), **i32), torch.empty((C_, H_, W_), **i32))

    def traced():
        binding.gs_rasterize_fwd_traced(ds.means2d, ds.conics, ds.colors, ds.opacities, ds.backgrounds, W_, H_,
                                        scene.tile_size, plan.offsets, plan.ids, S_TRACE, n_isects=plan.n_isects,
                                        alpha_cutoff=scene.alpha_cutoff, alpha_clamp=scene.alpha_clamp,
                                        transmittance_threshold=scene.transmittance_threshold, out=tr_out,
                                        stream=plan.stream)
    for _ in range(2):
        traced()
    tev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(5, args.steps // 2))]
    for a_ev, b_ev in tev:
        a_ev.record(plan.stream)
        traced()
        b_ev.record(plan.stream)
    torch.cuda.synchronize()
    traced_ms = statistics.median(a_ev.elapsed_time(b_ev) for a_ev, b_ev in tev)
    traced_steps = int(tr_out.trace_counts.sum())
    traced_capped = int((tr_out.trace_counts == S_TRACE).sum())
    del tr_out
    # outside the frame: the composite with the hardware exponential on the last frame, and how far it lands from
    # the specified one
    hw_out = binding.Render(torch.empty((C_, H_, W_, K_), **f32), torch.empty((C_, H_, W_), **f32),
                            torch.empty((C_, H_, W_), **f32), torch.empty((C_, H_, W_), **i32))

    def hw_composite():
        binding.gs_rasterize_fwd_hwexp(ds.means2d, ds.conics, ds.colors, ds.opacities, ds.backgrounds, W_, H_,
                                       scene.tile_size, plan.offsets, plan.ids, plan.n_isects, scene.alpha_cutoff,
                                       scene.alpha_clamp, scene.transmittance_threshold, out=hw_out,
                                       stream=plan.stream)
    for _ in range(2):
        hw_composite()
    hev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(5, args.steps // 2))]
    for a_ev, b_ev in hev:
        a_ev.record(plan.stream)
        hw_composite()
        b_ev.record(plan.stream)
    torch.cuda.synchronize()
    hw_ms = statistics.median(a_ev.elapsed_time(b_ev) for a_ev, b_ev in hev)
    hw_dc = (hw_out.render_colors - plan.render.render_colors).abs().amax(-1)
    hw_dT = (hw_out.render_T - plan.render.render_T).abs()
    hw_bad = int(((hw_dc > 1e-4) | (hw_dT > 1e-4)).sum())
    hw_max = max(float(hw_dc.max()), float(hw_dT.max()))
    del hw_out, hw_dc, hw_dT
    # outside the frame: fixed-capacity per-tile bins as the alternative to the sort path, and the composite
    # over them (capacity 8192 holds the frame's largest tile)
    CAP = 8192
    radii_d = ds.radii

    def build_bins(out=None):
        return binding.gs_bin_tiles(ds.means2d, radii_d, ds.depths, scene.tile_size, scene.tile_width,
                                    scene.tile_height, CAP, out=out, stream=plan.stream)
    bins = build_bins()
    bin_render = binding.gs_rasterize_fwd_bins(ds.means2d, ds.conics, ds.colors, ds.opacities, ds.backgrounds, W_,
                                               H_, scene.tile_size, bins.bin_ids, bins.bin_counts,
                                               scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold,
                                               stream=plan.stream)
    bev_b = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(max(5, args.steps // 2))]
    for e0, e1, e2 in bev_b:
        e0.record(plan.stream)
        build_bins(out=bins)
        e1.record(plan.stream)
        binding.gs_rasterize_fwd_bins(ds.means2d, ds.conics, ds.colors, ds.opacities, ds.backgrounds, W_, H_,
                                      scene.tile_size, bins.bin_ids, bins.bin_counts, scene.alpha_cutoff,
                                      scene.alpha_clamp, scene.transmittance_threshold, out=bin_render,
                                      stream=plan.stream)
        e2.record(plan.stream)
    torch.cuda.synchronize()
    bins_build_ms = statistics.median(e0.elapsed_time(e1) for e0, e1, _ in bev_b)
    bins_comp_ms = statistics.median(e1.elapsed_time(e2) for _, e1, e2 in bev_b)
    bin_counts = bins.bin_counts.cpu().numpy()
    del bins, bin_render
    # outside the frame: the EWA projection that produces such splats, 1M 3D Gaussians into one 1920x1080 camera
    sc3 = synth.scene3d(19, scene.N, C=1, width=scene.width, height=scene.height)
    d3 = [torch.from_numpy(a).to("cuda:0") for a in (sc3.means, sc3.covars, sc3.viewmats, sc3.Ks)]
    proj = binding.gs_project_fwd(*d3, sc3.width, sc3.height, compensation=True)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(max(5, args.steps // 2))]
    for a_ev, b_ev in pev:
        a_ev.record(plan.stream)
        binding.gs_project_fwd(*d3, sc3.width, sc3.height, compensation=True, out=proj, stream=plan.stream)
        b_ev.record(plan.stream)
    torch.cuda.synchronize()
    project_ms = statistics.median(a_ev.elapsed_time(b_ev) for a_ev, b_ev in pev)
    project_bytes = sc3.N * (12 + 36) + sc3.C * sc3.N * (8 + 8 + 4 + 12 + 4)
    del d3, proj
    # outside the frame: the stand-alone stable sort of the same intersections over all populated key bits
    stage_ms["generic_sort"], _ = plan.run_generic_sort(max(5, args.steps // 2))
    pixels = scene.C * scene.width * scene.height
    bwd_valu = measured_valu(args.config, "backward")
    bwd_issued = None if bwd_valu is None else bwd_valu * 64 / (backward_ms * 1e-3) / 1e12
    bwd_roofline = {"bound": "alu", "achieved": None if bwd_issued is None else round(bwd_issued, 3),
                    "peak": round(PEAK_VALU_TOPS, 2), "unit": "T VALU lane-instructions/s (as roofline)",
                    "frac": None if bwd_issued is None else round(bwd_issued / PEAK_VALU_TOPS, 4),
                    "valu_wave_instructions_per_launch": bwd_valu}
    tile_passes = (plan.end_bit - 32 + 7) // 8
    generic_passes = (plan.end_bit + 7) // 8
    nbytes = stage_bytes(scene, n, tile_passes, generic_passes)
    K = scene.colors.shape[-1]
    # the definition's work, and the work the kernel executes (it skips evaluations its exact cull proves idle)
    ops_def = OPS_EVAL * n_eval + OPS_PASS * n_pass + (1 + 2 * K) * n_comp
    ops = OPS_EVAL * n_exec + OPS_PASS * n_pass + (1 + 2 * K) * n_comp
    stages = {}
    for nm in names + ["generic_sort"]:
        gbs = nbytes[nm] / (stage_ms[nm] * 1e-3) / 1e9
        stages[nm] = {"ms": round(stage_ms[nm], 4), "bytes": nbytes[nm], "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    comp_s = stage_ms["composite"] * 1e-3
    comp_tops = ops / comp_s / 1e12
    stages["composite"].update({"lane_ops_executed": ops, "lane_ops_definition": ops_def,
                                "spec_Tops/s_executed": round(comp_tops, 3),
                                "definition_Tops/s_equivalent": round(ops_def / comp_s / 1e12, 3)})
    # the roofline object is for the longest single kernel, the composite (one launch bracketed by one event
    # pair); the other stages, several kernels each, are reported against HBM in "stages". achieved = the VALU
    # instructions the kernel issues (profiler count x 64 lanes) per second of its live duration
    valu = measured_valu(args.config, "composite")
    issued = None if valu is None else valu * 64 / comp_s / 1e12
    roofline = {"bound": "alu", "kernel": "raster_cull_kernel",
                "achieved": None if issued is None else round(issued, 3), "peak": round(PEAK_VALU_TOPS, 2),
                "unit": "T VALU lane-instructions/s (profiler VALU count x 64 / live duration; peak = 2 wave64 "
                        "instructions per SIMD per 4 cycles x 1024 SIMDs x 2.4 GHz, the measured dual-issue rate)",
                "frac": None if issued is None else round(issued / PEAK_VALU_TOPS, 4),
                "valu_wave_instructions_per_launch": valu,
                "definition_equivalent_Tops": round(ops_def / comp_s / 1e12, 3),
                "definition_equivalent_note": "the definition's lane-operations (every evaluation the tile walk "
                                              "makes, 29 per evaluation + 3 per alpha >= cutoff + 7 per composited "
                                              "splat) per second: what the kernel's exact cull saves",
                "traffic": measured_traffic(args.config),
                "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": nbytes["composite"]}

    result = {
        "metric": METRIC,
        "value": round(pixels / (ms_per_step * 1e-3) / 1e6, 2),
        "unit": "Mpix/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "ms_per_step": round(ms_per_step, 4),
        "frames_in_flight": F,
        "latency_ms_per_frame": round(latency_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config, "cameras": scene.C, "splats": scene.N,
                   "width": scene.width, "height": scene.height, "tile_size": scene.tile_size,
                   "n_isects": n, "sort_end_bit": plan.end_bit, "tile_sort_passes": tile_passes,
                   "generic_sort_passes": generic_passes},
        # the frame's sort is split over both phases of gs_isect_tiles (depth order, then the tile passes): keys
        # per second over the whole of both, emission and counting included
        "isect_keys_sorted_per_s": round(n / ((stage_ms["count_depth_order"] + stage_ms["emit_sort"]) * 1e-3), 1),
        "isect_keys_sorted_per_s_generic_sort": round(n / (stage_ms["generic_sort"] * 1e-3), 1),
        "isect_keys_sorted_per_s_frame": round(n / (ms_per_step * 1e-3), 1),
        "rasterized_mpix_per_s_composite_only": round(pixels / (stage_ms["composite"] * 1e-3) / 1e6, 2),
        "backward": dict({"ms": round(backward_ms, 4), "Mpix/s": round(pixels / (backward_ms * 1e-3) / 1e6, 2),
                          "note": "gs_rasterize_bwd on the last frame with seeded standard-normal output gradients; "
                                  "clears the gradients, then sums them"}, **bwd_roofline),
        "traced_forward": {"ms": round(traced_ms, 4), "max_splat_steps": S_TRACE, "trace_entries": traced_steps,
                           "pixels_at_cap": traced_capped,
                           "trace_bytes_written": 4 * traced_steps + 4 * pixels,
                           "note": "gs_rasterize_fwd_traced on the last frame's lists, no list cap: the composite "
                                   "plus each pixel's trace row and count"},
        "hw_exp_composite": {"ms": round(hw_ms, 4), "Mpix/s": round(pixels / (hw_ms * 1e-3) / 1e6, 2),
                             "pixels_over_1e-4_vs_specified": hw_bad, "max_abs_diff_vs_specified": hw_max,
                             "note": "gs_rasterize_fwd_hwexp (v_exp_f32) on the last frame's lists; the difference "
                                     "is to the specified-exponential composite of the same frame"},
        "fixed_capacity_bins": {
            "capacity": CAP, "build_ms": round(bins_build_ms, 4), "composite_ms": round(bins_comp_ms, 4),
            "sort_path_ms": round(stage_ms["count_depth_order"] + stage_ms["emit_sort"] + stage_ms["ranges"], 4),
            "largest_bin": int(bin_counts.max()), "overflowed_bins": int((bin_counts > CAP).sum()),
            "bin_bytes": int(bin_counts.size) * CAP * 4,
            "note": "gs_bin_tiles (atomic slot claims, then a bitonic sort of each bin in LDS) against the frame's "
                    "intersect + sort + ranges stages; composite_ms is gs_rasterize_fwd_bins over the bins"},
        "projection": {"ms": round(project_ms, 4), "gaussians": sc3.N, "bytes": project_bytes,
                       "GB/s": round(project_bytes / (project_ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(project_bytes / (project_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "note": "gs_project_fwd of 1M seeded 3D Gaussians into one camera at the frame's size, "
                               "with compensation"},
        "composite_work": {"evaluations_definition": n_eval, "evaluations_executed": n_exec,
                           "alpha_ge_cutoff": n_pass, "composited": n_comp, "splats_staged": n_staged},
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration"] = {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "copies": 3}
        del src, dst
    if args.valu_calibration:
        result["valu_calibration"] = valu_calibration(plan.stream)
    if not args.no_cpu_baseline:
        reps = args.cpu_reps if args.cpu_reps > 0 else (3 if args.config in ("config1", "config2", "config3") else 1)
        result["cpu_baseline"], sample = cpu_baseline(scene, args.cpu_tile_stride, reps)
        result["cpu_baseline_openmp"] = cpu_baseline_openmp(scene, sample, reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

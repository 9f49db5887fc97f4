#!/usr/bin/env python3
"""Throughput of the sphere rasterizer: Mpixels/s forward + backward at one
million spheres, 1024x1024, one GPU (the default workload). --workload k runs
the same protocol on another of the five synthetic workloads, with the pixel
count summed over its views.

A step is one pass of the whole path on resident inputs: splat_project,
splat_bin_sort, splat_render_fwd, splat_render_bwd (compositor backward,
per-primitive chain rule and camera reduction). Buffers are allocated and the
pair capacity checked before timing; W warm-up steps, then K timed steps
bracketed by device synchronisation. Per-stage times come from HIP events on
the stream the library launches on (torch's current stream).

Prints one JSON line. At one GPU it also times the CPU oracle on the host
(all cores) over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Mpixels/s fwd+bwd at 1M primitives, 1024x1024; % of VALU/HBM roofline"
# MI355X: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz = 39.3 T single-issue fp32 lane-ops/s
# (packed fp32 doubles the FLOP count but is not used; an fp64 FMA issues at the same
# per-lane rate); HBM3E 8 TB/s.
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
# Algorithmic work of the sphere path per unit (the method's work, not the
# instructions a kernel issues):
#   forward compositor: per list entry a pixel examines before it stops 7 lane-ops
#     (ray distance, scale, compare, bound compare); per contributing sphere 7 + C
#     (D, weight, normalisation, C colour FMAs, top-K bookkeeping); the counts are
#     the oracle's exact per-pixel totals over the frame
#   reverse compositor: per recorded (pixel, sphere) 45 lane-ops of gradient
#     arithmetic; per (8x8 pixel quadrant, recorded sphere) the 8 x 63 additions
#     that reduce its eight values over the quadrant's 64 pixels
#   projection: read position, radius, opacity (20 B), write a 48-byte record
#     and the pair count (4 B) per sphere
#   binning: scan 8 B per sphere; emit 20 B per sphere + 12 B per pair; sort
#     24 B per pair per 8-bit pass over 32 depth bits + ceil(log2 tiles) tile
#     bits; tile ranges 8 B per pair + 8 B per tile
#   gradient tail (chain rule + camera sum): ~60 B per sphere
OPS_PER_ENTRY = 7
OPS_PER_HIT_BASE = 7          # + one fma per channel
OPS_PER_RECORDED = 45
OPS_PER_WAVE_SPHERE = 8 * 63
PROJECT_BYTES_PER_PRIM = 20 + 48 + 4
SCAN_BYTES_PER_PRIM = 8
EMIT_BYTES_PER_PRIM, EMIT_BYTES_PER_PAIR = 20, 12
SORT_BYTES_PER_PAIR_PASS = 24
RANGE_BYTES_PER_PAIR, RANGE_BYTES_PER_TILE = 8, 8
GRAD_BYTES_PER_PRIM = 60
# The Gaussian workloads (parity cases, not the headline) by the same rules, the
# survey's "other configs scale with N and P": projection reads the primitive's
# inputs once (2D: centre, sigma, depth, opacity, 20 B; 3D: mean, scale,
# rotation, opacity, 44 B) and writes a ~32-byte record and the pair count per
# (view, primitive); the gradient tail reads each record's 2D gradients
# ((2 + 3 + 1 + C) fp32, C the view's channels) and the inputs once, and writes
# the inputs' gradients once (plus 4 B per feature channel)
GAUSS_READ_BYTES = {0: 20, 1: 44}
GAUSS_RECORD_BYTES = 32 + 4
GAUSS_GRAD_WRITE_BYTES = {0: 8 + 4 + 4, 1: 44}
# HBM bytes (read + written) per launch of the forward sphere compositor on this
# workload, from two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE) scaled by
# a plain copy of known size; they hold for the sources with this digest only.
FWD_TRAFFIC_BYTES = 186399035
FWD_TRAFFIC_SOURCES = ("sphere_rasterization_amd/csrc/render_fwd.hip",
                       "sphere_rasterization_amd/csrc/render_common.h",
                       "sphere_rasterization_amd/csrc/splat_internal.h")
FWD_TRAFFIC_SHA256 = "818b483a06c12f81074d13769b1f6a59c185b3144b6c981626c2c4e0da705c4c"
BIN_KERNELS = ("k_thist", "k_col_scan", "k_tscatter", "k_seg_sort", "k_tile_scan1", "k_scan_reduce", "k_scan_top",
               "k_tile_ranges", "k_fill_u32", "k_tile_count", "k_bucket")


def binning_bytes(n, npairs, total_tiles):
    """Algorithmic HBM bytes of scan, emit, sort and tile ranges (see above)."""
    bits = 32 + max(1, math.ceil(math.log2(max(total_tiles, 2))))
    passes = math.ceil(bits / 8)
    return (SCAN_BYTES_PER_PRIM * n + EMIT_BYTES_PER_PRIM * n + EMIT_BYTES_PER_PAIR * npairs
            + SORT_BYTES_PER_PAIR_PASS * passes * npairs + RANGE_BYTES_PER_PAIR * npairs
            + RANGE_BYTES_PER_TILE * total_tiles), passes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=1024,
                    help="image rows the CPU oracle renders (fwd + bwd) on all host cores for the baseline")
    ap.add_argument("--cpu-1t-rows", type=int, default=1024,
                    help="image rows the CPU oracle renders (fwd + bwd) on one thread")
    ap.add_argument("--atomic-direct-max", type=int, default=0,
                    help="spheres: entries recorded by at most this many lanes of a wavefront add their gradient "
                         "terms lane by lane instead of after the wavefront reduction (0: always reduce)")
    ap.add_argument("--no-kernel-profile", action="store_true",
                    help="skip the pass that takes per-kernel device times with torch.profiler")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run three plain device copies of this many MiB (read + write of a "
                         "known size, to scale hardware byte counters)")
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="1: 4096 screen-space Gaussians 128x128; 2: 100k 3D Gaussians 512x512; 3: 1M spheres "
                         "1024x1024 (default, the headline metric); 4: 2M Gaussians 1920x1080, 32 channels; "
                         "5: the same scene from 6 cameras 1280x720 and a 2048x64 lidar view")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured peaks (sustained clock, FMA rate, copy and LDS bandwidth)")
    ap.add_argument("--assemble", action="store_true",
                    help="instead of the rendering step, time the per-frame parameter assembly (keyframe "
                         "interpolation of 2M primitives, 4 keyframes) and its reverse pass against the HBM peak")
    return ap.parse_args()


WORKLOAD_NAMES = {1: "gauss2d_4096_128x128", 2: "gauss3d_100k_512x512", 3: "spheres_1m_1024x1024",
                  4: "gauss3d_2m_1920x1080_c32", 5: "gauss3d_2m_6x1280x720_lidar_2048x64"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from sphere_rasterization_amd import scenes as S
    from sphere_rasterization_amd.raster import Rasterizer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.assemble:
        print(json.dumps(assemble_bench(args, torch, dev)), flush=True)
        return
    wl = args.workload
    scene = S.make_config(wl)
    pixels = sum(c.width * c.height for c in scene.cams)
    rz = Rasterizer(scene, device=dev)
    rz.forward(check=True)                       # sizes the pair buffers once
    g_np = S.upstream_grads(scene, S.CONFIGS[wl]["grad_seed"])
    dimg = torch.from_numpy(np.concatenate([g.reshape(-1) for g in g_np])).to(dev)
    want = ("pos", "scale", "rot", "opacity", "feat", "cam_R", "cam_t")
    grads = rz.alloc_grads(want)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        rz.project()
        if ev is not None:
            ev[1].record()
        rz.bin_sort()
        if ev is not None:
            ev[2].record()
        rz.render_fwd()
        if ev is not None:
            ev[3].record()
        # all views in one call (camera and lidar views run separate kernels)
        rz.backward(dimg, grads=grads, atomic_direct_max=args.atomic_direct_max)
        if ev is not None:
            ev[4].record()

    def fwd_timed_step(ev):
        # the timed steps carry one pair of events, around the forward compositor
        # (the roofline's kernel); per-stage events go in a separate pass below,
        # since every event marker on the stream adds a gap between kernels
        rz.project()
        rz.bin_sort()
        ev[0].record()
        rz.render_fwd()
        ev[1].record()
        rz.backward(dimg, grads=grads, atomic_direct_max=args.atomic_direct_max)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        fwd_timed_step(fev[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert int(rz.overflow.item()) == 0
    ms = (t1 - t0) * 1e3 / args.steps
    fwd_kernel_ms = float(np.median([fev[k][0].elapsed_time(fev[k][1]) for k in range(args.steps)]))
    # stage breakdown (diagnostic): the same steps with an event between stages
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    if args.copy_calibration_mib > 0:
        nf = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(nf, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)     # reads and writes nf * 4 bytes
        torch.cuda.synchronize()
        del src, dst
    stages = ["project", "bin_sort", "render_fwd", "render_bwd"]
    st_ms = {s: float(np.median([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
             for i, s in enumerate(stages)}
    value = pixels / (ms / 1e3) / 1e6
    npairs = int(rz.num_pairs.item())
    ktimes = None
    if not args.no_kernel_profile:
        ktimes = kernel_times(torch, step, min(args.steps, 20))

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "Mpixels/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[wl], "primitives": scene.n,
                   "width": scene.cams[0].width, "height": scene.cams[0].height, "pixels": pixels,
                   "channels": scene.channels, "views": rz.V, "pairs": npairs},
        "stage_ms": {k: round(v, 4) for k, v in st_ms.items()},
    }

    if wl != 3:
        out["metric"] = f"Mpixels/s fwd+bwd, {WORKLOAD_NAMES[wl]}"
    cpu = None
    if not args.no_cpu_baseline and wl == 3:
        cpu = cpu_baseline(scene, g_np, args.cpu_sample_rows, args.cpu_1t_rows)
        out["cpu_baseline"] = cpu["json"]
    if wl == 3:
        out["roofline"] = roofline(fwd_kernel_ms, cpu, scene)
    out["kernels"] = kernel_rooflines(ktimes, cpu, scene, npairs, rz.total_tiles)
    if not args.no_peaks:
        out["measured_peaks"] = measured_peaks(torch, dev)
        add_measured_fracs(out, out["measured_peaks"])
    print(json.dumps(out), flush=True)


# Per-frame assembly, algorithmic HBM bytes per primitive: forward reads the two
# bracketing keyframes' centre and rotation (2 x 28 B) and writes 28 B; the
# reverse pass reads the upstream gradients (28 B) and both rotations (32 B, for
# the shorter-arc sign) and adds into both keyframes' gradient rows (2 x 28 B read
# and written).
ASM_FWD_BYTES = 84
ASM_BWD_BYTES = 28 + 32 + 112


def assemble_bench(args, torch, dev):
    import numpy as np
    from sphere_rasterization_amd import _lib as L
    from sphere_rasterization_amd.raster import _ptr, _stream
    K, n = 4, 2_000_000
    rng = np.random.default_rng(7)
    times = np.cumsum(rng.uniform(0.05, 0.2, K)).astype(np.float32)
    t = float(np.float32(times[1] + 0.37 * (times[2] - times[1])))
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    kp = torch.randn((K, n, 3), device=dev, generator=gen)
    kr = torch.randn((K, n, 4), device=dev, generator=gen)
    pos = torch.empty((n, 3), device=dev)
    rot = torch.empty((n, 4), device=dev)
    gp = torch.randn((n, 3), device=dev, generator=gen)
    gq = torch.randn((n, 4), device=dev, generator=gen)
    dkp = torch.zeros((K, n, 3), device=dev)
    dkq = torch.zeros((K, n, 4), device=dev)
    fwd = lambda: L.splat_interpolate(list(times), t, n, _ptr(kp), _ptr(kr), _ptr(pos), _ptr(rot), _stream())
    bwd = lambda: L.splat_interpolate_bwd(list(times), t, n, _ptr(kr), _ptr(gp), _ptr(gq), _ptr(dkp), _ptr(dkq),
                                          _stream())
    res = {}
    for name, fn, nbytes in (("forward", fwd, ASM_FWD_BYTES), ("reverse", bwd, ASM_BWD_BYTES)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        gbs = nbytes * n / (ms / 1e3) / 1e9
        res[name] = {"ms": round(ms, 5), "bytes_per_launch": nbytes * n,
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}
    f = res["forward"]
    return {"metric": "Mprimitives/s assembled per frame (keyframe interpolation)",
            "value": round(n / (f["ms"] / 1e3) / 1e6, 1), "unit": "Mprimitives/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": f["ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "assemble_2m_4keys", "primitives": n, "keyframes": K},
            "roofline": f["roofline"], "reverse": res["reverse"]}


def measured_peaks(torch, dev):
    """Peaks measured on this GPU (sphere_rasterization_amd.peaks): the shader
    clock sustained under a full-chip fp32 FMA loop and the single-issue FMA
    rate it reaches, the HBM bandwidth of a 16-byte copy of 1 GiB, and the LDS
    bandwidth of broadcast reads in the compositors' pattern."""
    from sphere_rasterization_amd import peaks
    return peaks.measure(torch, dev)


def add_measured_fracs(out, peaks):
    """Each stage's achieved figure against the measured peaks as well: HBM
    stages against the copy bandwidth, the compositors' lane-ops against the
    highest VALU rate measured (the fp32 FMA loop: its fp32 FMAs issue faster
    than one wave64 instruction per four cycles, the fp64 loop runs at that
    rate; its clock, under full FMA load, is below the compositors')."""
    if not peaks:
        return
    valu = max(peaks["valu_fma_Tlane_ops"], peaks["valu_fma64_Tlane_ops"])
    for e in (out.get("kernels") or {}).values():
        if isinstance(e, dict) and e.get("achieved") is not None:
            if e.get("bound") == "hbm":
                e["frac_measured"] = round(e["achieved"] / peaks["hbm_copy_GBps"], 4)
            elif e.get("bound") == "alu":
                e["frac_measured"] = round(e["achieved"] / valu, 4)
    r = out.get("roofline")
    if r and r.get("achieved") is not None:
        r["peak_measured"] = valu
        r["frac_measured"] = round(r["achieved"] / valu, 4)


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_times(torch, step, steps):
    """Average device time per launch (us) of every library kernel over `steps`
    steps, taken with torch.profiler (a diagnostic pass after the timed steps)."""
    import re
    try:
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
        out = {}
        for e in prof.key_averages():
            m = re.search(r"(k_\w+)(<[^()]*>)?\(", e.key)
            if not m:
                continue
            name = m.group(1) + (m.group(2) or "")
            us = float(getattr(e, "device_time", 0.0) or 0.0)
            out[name] = {"us": round(us, 3), "launches_per_step": round(e.count / steps, 3)}
        return out or None
    except Exception as ex:                  # the profiler is a diagnostic: never fail the run
        print(f"kernel profile skipped: {ex}", file=sys.stderr)
        return None


def _frac(work, us, peak, unit_scale):
    achieved = work / (us * 1e-6) / unit_scale
    return round(achieved, 3), round(achieved / peak, 4)


def project_bytes(scene):
    """Algorithmic HBM bytes of the projection (see above)."""
    V = len(scene.cams)
    if scene.kind == 2:
        return PROJECT_BYTES_PER_PRIM * V * scene.n
    return GAUSS_READ_BYTES[scene.kind] * scene.n + GAUSS_RECORD_BYTES * V * scene.n


def grad_tail_bytes(scene):
    """Algorithmic HBM bytes of the gradient tail (see above)."""
    if scene.kind == 2:
        return GRAD_BYTES_PER_PRIM * scene.n
    rows = sum(4 * (6 + scene.view_channels(v)) for v in range(len(scene.cams)))
    return (rows + GAUSS_READ_BYTES[scene.kind] + GAUSS_GRAD_WRITE_BYTES[scene.kind] + 4 * scene.channels) * scene.n


def kernel_rooflines(kt, cpu, scene, npairs, total_tiles):
    """Each stage's kernels against their own roofline, with the survey's
    algorithmic units (see the constants above) and the profiled device times.
    The compositors' lane-op counts need the oracle's per-pixel totals over the
    whole frame (the headline workload only); the other workloads' compositor
    lines carry their times."""
    if not kt:
        return None
    pick = lambda pre: {k: v for k, v in kt.items() if k.split("<")[0] == pre}
    tsum = lambda d: sum(v["us"] * v["launches_per_step"] for v in d.values())
    n, C = scene.n, scene.channels
    nrec = n * len(scene.cams)
    out = {}
    proj = pick("k_project")
    if proj:
        b = project_bytes(scene)
        a, f = _frac(b, tsum(proj), HBM_PEAK_GBS, 1e9)
        out["project"] = {"kernels": sorted(proj), "us": round(tsum(proj), 2), "bound": "hbm", "bytes": b,
                          "achieved": a, "unit": "GB/s", "frac": f}
    bink = {k: v for k, v in kt.items() if k.split("<")[0] in BIN_KERNELS}
    if bink:
        b, passes = binning_bytes(nrec, npairs, total_tiles)
        a, f = _frac(b, tsum(bink), HBM_PEAK_GBS, 1e9)
        out["bin_sort"] = {"kernels": sorted(bink), "us": round(tsum(bink), 2), "bound": "hbm", "bytes": b,
                           "radix_passes_counted": passes, "achieved": a, "unit": "GB/s", "frac": f}
        if proj:
            b2 = b + project_bytes(scene)
            us2 = tsum(bink) + tsum(proj)
            a, f = _frac(b2, us2, HBM_PEAK_GBS, 1e9)
            out["project_bin_sort"] = {"us": round(us2, 2), "bound": "hbm", "bytes": b2, "achieved": a,
                                       "unit": "GB/s", "frac": f}
    full = cpu is not None and cpu["rows"] == cpu["H"]
    fwd = pick("k_fwd_sphere")
    if fwd:
        e = {"kernels": sorted(fwd), "us": round(tsum(fwd), 2), "bound": "alu", "unit": "Tops/s"}
        if full:
            ops = cpu["processed"] * OPS_PER_ENTRY + cpu["hits"] * (OPS_PER_HIT_BASE + C)
            e["ops"] = ops
            e["achieved"], e["frac"] = _frac(ops, tsum(fwd), VALU_PEAK_TOPS, 1e12)
        out["render_fwd"] = e
    bwd = {k: v for k, v in kt.items() if k.split("<")[0] in ("k_bwd_sphere", "k_bwd_sphere_dense")}
    if bwd:
        e = {"kernels": sorted(bwd), "us": round(tsum(bwd), 2), "bound": "alu", "unit": "Tops/s"}
        if full:
            ops = cpu["recorded"] * OPS_PER_RECORDED + cpu["wave_spheres"] * OPS_PER_WAVE_SPHERE
            e["ops"] = ops
            e["achieved"], e["frac"] = _frac(ops, tsum(bwd), VALU_PEAK_TOPS, 1e12)
        out["render_bwd"] = e
    for name, pre in (("render_fwd", ("k_fwd_alpha", "k_fwd_split")), ("render_bwd", ("k_bwd_alpha", "k_bwd_split"))):
        ks = {k: v for k, v in kt.items() if k.split("<")[0] in pre}
        if ks:
            out[name] = {"kernels": sorted(ks), "us": round(tsum(ks), 2), "bound": "alu"}
    tail = {k: v for k, v in kt.items()
            if k.split("<")[0] in ("k_sphere_grads", "k_cam_final", "k_zero", "k_proj_bwd_gauss",
                                    "k_feat_grads_gauss", "k_cam_grad_sphere")}
    if tail:
        b = grad_tail_bytes(scene)
        a, f = _frac(b, tsum(tail), HBM_PEAK_GBS, 1e9)
        out["grad_tail"] = {"kernels": sorted(tail), "us": round(tsum(tail), 2), "bound": "hbm", "bytes": b,
                            "achieved": a, "unit": "GB/s", "frac": f}
    out["all_kernels_us"] = {k: v["us"] for k, v in sorted(kt.items())}
    return out


def _oracle_frame(O, scene, g_np, rows):
    """Oracle on the first `rows` image rows: projection and binning of every
    sphere, then compositing and reverse pass of those rows' pixels. Returns the
    wall times (s) and the forward outputs."""
    import numpy as np
    W = scene.cams[0].width
    t0 = time.perf_counter()
    orc = O.Oracle(scene)
    orc.bin()
    t1 = time.perf_counter()
    pix = np.arange(rows * W, dtype=np.int64)
    r = orc.render(pix)
    t2 = time.perf_counter()
    g = [np.array(x, copy=True) for x in g_np]
    g[0][:, rows:, :] = 0.0
    orc.backward(g)
    t3 = time.perf_counter()
    orc.close()
    return dict(prep=t1 - t0, fwd=t2 - t1, bwd=t3 - t2, r=r)


def cpu_baseline(scene, g_np, rows, rows_1t):
    """The CPU oracle on the host: all its threads over the first `rows` rows, then
    one thread over the first `rows_1t` rows; each reports the sampled pixels over
    its wall time (projection and binning of every sphere included)."""
    import numpy as np
    from oracle import oracle as O
    H, W = scene.cams[0].height, scene.cams[0].width
    rows = max(1, min(rows, H))
    rows_1t = max(1, min(rows_1t, H))
    nthr = O.threads()
    a = _oracle_frame(O, scene, g_np, rows)
    O.threads(1)
    try:
        b = _oracle_frame(O, scene, g_np, rows_1t)
    finally:
        O.threads(nthr)
    wall = a["prep"] + a["fwd"] + a["bwd"]
    mpix = rows * W / wall / 1e6
    wall1 = b["prep"] + b["fwd"] + b["bwd"]
    r = a["r"]
    top = r["top"]
    pix = np.arange(rows * W, dtype=np.int64)
    quad = (pix // W // 8) * ((W + 7) // 8) + (pix % W) // 8
    rec = top >= 0
    qid = np.unique(quad[:, None].repeat(top.shape[1], 1)[rec] * scene.n + top[rec])
    return {"json": {"value": round(mpix, 4), "unit": "Mpixels/s", "cores": nthr, "kind": "oracle",
                     "sample": f"first {rows} of {H} rows of the 1M-sphere 1024x1024 frame on {nthr} threads: "
                               f"projection and binning of all spheres, compositing and reverse pass of "
                               f"{rows * W} pixels (fp64, {wall:.1f} s wall)",
                     "fwd_s": round(a["prep"] + a["fwd"], 3), "bwd_s": round(a["bwd"], 3),
                     "one_thread": {"value": round(rows_1t * W / wall1 / 1e6, 4), "unit": "Mpixels/s",
                                    "cores": 1, "fwd_s": round(b["prep"] + b["fwd"], 3),
                                    "bwd_s": round(b["bwd"], 3),
                                    "sample": f"first {rows_1t} of {H} rows on one thread: projection and binning "
                                              f"of all spheres, compositing and reverse pass of {rows_1t * W} "
                                              f"pixels ({wall1:.1f} s wall)"}},
            "processed": int(r["processed"].sum()), "hits": int(r["ncontrib"].sum()),
            "recorded": int(rec.sum()), "wave_spheres": int(len(qid)), "rows": rows, "H": H}


def roofline(fwd_ms, cpu, scene):
    """Forward compositor against the single-issue VALU peak, from the oracle's
    exact count of list entries examined and contributions made per pixel in the
    survey's units (7 lane-ops per entry, 7 + C per contribution); fwd_ms: the
    kernel's median time over the timed steps (HIP events on its stream)."""
    traffic = FWD_TRAFFIC_BYTES if sources_digest(FWD_TRAFFIC_SOURCES) == FWD_TRAFFIC_SHA256 else None
    if cpu is None or cpu["rows"] != cpu["H"]:
        return {"bound": "alu", "kernel": "k_fwd_sphere", "achieved": None, "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "Tops/s", "frac": None, "traffic": traffic, "kernel_ms": round(fwd_ms, 4)}
    ops = cpu["processed"] * OPS_PER_ENTRY + cpu["hits"] * (OPS_PER_HIT_BASE + scene.channels)
    achieved = ops / (fwd_ms / 1e3) / 1e12
    return {"bound": "alu", "kernel": "k_fwd_sphere", "achieved": round(achieved, 3),
            "peak": round(VALU_PEAK_TOPS, 2), "unit": "Tops/s", "frac": round(achieved / VALU_PEAK_TOPS, 4),
            "traffic": traffic, "ops_per_launch": ops, "kernel_ms": round(fwd_ms, 4)}


if __name__ == "__main__":
    main()

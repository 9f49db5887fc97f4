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
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Mpixels/s fwd+bwd at 1M primitives, 1024x1024; % of VALU/HBM roofline"
# MI355X: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz = 39.3 T single-issue fp32 lane-ops/s
# (packed fp32 doubles the FLOP count but is not used); HBM3E 8 TB/s.
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
# Algorithmic VALU lane-ops of the sphere compositor (see the design notes):
# per list entry a pixel examines before it stops, and per contributing sphere.
OPS_PER_ENTRY = 15
OPS_PER_HIT_BASE = 5          # + one fma per channel
# HBM bytes (read + written) per launch of the forward sphere compositor on this
# workload, from two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE) scaled by
# a plain copy of known size; they hold for the sources with this digest only.
FWD_TRAFFIC_BYTES = 210637709
FWD_TRAFFIC_SOURCES = ("sphere_rasterization_amd/csrc/render_fwd.hip",
                       "sphere_rasterization_amd/csrc/render_common.h",
                       "sphere_rasterization_amd/csrc/splat_internal.h")
FWD_TRAFFIC_SHA256 = "e8c85bf7b5fd546051e7d95c864bc7b88fbc8dcef44b7ae727f06827abbf7956"
# Algorithmic HBM bytes of the projection and binning stages:
#   projection: per primitive read position, radius, opacity and the three
#     features (20 + 12 B), write the bin, draw and backward records and the
#     pair count (16 + 64 + 16 + 4 B)
#   binning: per record the 16-byte bin record twice (counting and scatter
#     passes, 32 B; the pair count is its rectangle's tile count); per pair the
#     bucketed word written and read (16 B) and the sorted key and value
#     written (12 B)
PROJECT_BYTES_PER_PRIM = 20 + 12 + 16 + 64 + 16 + 4
BIN_BYTES_PER_REC = 32
BIN_BYTES_PER_PAIR = 28


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=1024,
                    help="image rows the CPU oracle renders (fwd + bwd) for the baseline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run three plain device copies of this many MiB (read + write of a "
                         "known size, to scale hardware byte counters)")
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="1: 4096 screen-space Gaussians 128x128; 2: 100k 3D Gaussians 512x512; 3: 1M spheres "
                         "1024x1024 (default, the headline metric); 4: 2M Gaussians 1920x1080, 32 channels; "
                         "5: the same scene from 6 cameras 1280x720 and a 2048x64 lidar view")
    ap.add_argument("--hbm-copy", action="store_true",
                    help="also time a plain 1 GiB device copy and report the measured HBM bandwidth")
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
        rz.backward(dimg, grads=grads)
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
        rz.backward(dimg, grads=grads)

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
        cpu = cpu_baseline(scene, g_np, args.cpu_sample_rows)
        out["cpu_baseline"] = cpu["json"]
    if wl == 3:
        out["roofline"] = roofline(fwd_kernel_ms, cpu, scene)
        out["stage_hbm"] = stage_hbm(st_ms, scene.n, npairs)
    if args.hbm_copy:
        out["hbm_copy_GBps"] = hbm_copy(torch, dev)
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


def hbm_copy(torch, dev, mib=1024, reps=10):
    """Measured HBM bandwidth of a plain device copy (bytes read + written / time)."""
    nf = mib * (1 << 20) // 4
    src = torch.ones(nf, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    return round(2 * nf * 4 / sec / 1e9, 1)


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stage_hbm(st_ms, n, npairs):
    """Projection and binning against the HBM peak, from their algorithmic bytes."""
    out = {}
    for name, nbytes in (("project", PROJECT_BYTES_PER_PRIM * n),
                         ("bin_sort", BIN_BYTES_PER_REC * n + BIN_BYTES_PER_PAIR * npairs)):
        gbs = nbytes / (st_ms[name] / 1e3) / 1e9
        out[name] = {"bytes": nbytes, "GB/s": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def cpu_baseline(scene, g_np, rows):
    """Oracle forward + backward on the host over the first `rows` image rows."""
    import numpy as np
    from oracle import oracle as O
    H, W = scene.cams[0].height, scene.cams[0].width
    rows = max(1, min(rows, H))
    t0 = time.perf_counter()
    orc = O.Oracle(scene)
    orc.bin()
    pix = np.arange(rows * W, dtype=np.int64)
    r = orc.render(pix)
    g = [np.array(x, copy=True) for x in g_np]
    g[0][:, rows:, :] = 0.0
    orc.backward(g)
    dt = time.perf_counter() - t0
    cores = os.cpu_count() or 1
    try:
        cores = int(os.environ.get("OMP_NUM_THREADS", cores))
    except ValueError:
        pass
    mpix = rows * W / dt / 1e6
    return {"json": {"value": round(mpix, 4), "unit": "Mpixels/s", "cores": cores, "kind": "oracle",
                     "sample": f"first {rows} of {H} rows of the 1M-sphere 1024x1024 frame: projection and "
                               f"binning of all spheres, compositing and reverse pass of {rows * W} pixels "
                               f"(fp64, {dt:.1f} s wall)"},
            "processed": int(r["processed"].sum()), "hits": int(r["ncontrib"].sum()),
            "rows": rows, "H": H}


def roofline(fwd_ms, cpu, scene):
    """Forward compositor against the single-issue VALU peak, from the oracle's
    exact count of list entries examined and contributions made per pixel;
    fwd_ms: the kernel's median time over the timed steps (HIP events on its stream)."""
    traffic = FWD_TRAFFIC_BYTES if sources_digest(FWD_TRAFFIC_SOURCES) == FWD_TRAFFIC_SHA256 else None
    if cpu is None or cpu["rows"] != cpu["H"]:
        return {"bound": "alu", "kernel": "k_fwd_sphere", "achieved": None, "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "Tops/s", "frac": None, "traffic": traffic}
    ops = cpu["processed"] * OPS_PER_ENTRY + cpu["hits"] * (OPS_PER_HIT_BASE + scene.channels)
    achieved = ops / (fwd_ms / 1e3) / 1e12
    return {"bound": "alu", "kernel": "k_fwd_sphere", "achieved": round(achieved, 3),
            "peak": round(VALU_PEAK_TOPS, 2), "unit": "Tops/s", "frac": round(achieved / VALU_PEAK_TOPS, 4),
            "traffic": traffic, "ops_per_launch": ops}


if __name__ == "__main__":
    main()

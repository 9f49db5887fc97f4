#!/usr/bin/env python3
"""Throughput of the sphere rasterizer: Mpixels/s forward + backward at one
million spheres, 1024x1024, one GPU.

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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=1024,
                    help="image rows the CPU oracle renders (fwd + bwd) for the baseline")
    return ap.parse_args()


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
    scene = S.pulsar_spheres()
    W, H = scene.cams[0].width, scene.cams[0].height
    rz = Rasterizer(scene, device=dev)
    rz.forward(check=True)                       # sizes the pair buffers once
    g_np = S.upstream_grads(scene, 103)
    dimg = torch.from_numpy(np.concatenate([g.reshape(-1) for g in g_np])).to(dev)
    grads = rz.alloc_grads(("pos", "scale", "opacity", "feat", "cam_R", "cam_t"))
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
        rz.backward(dimg, grads=grads)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert int(rz.overflow.item()) == 0
    ms = (t1 - t0) * 1e3 / args.steps
    stages = ["project", "bin_sort", "render_fwd", "render_bwd"]
    st_ms = {s: float(np.median([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
             for i, s in enumerate(stages)}
    pixels = W * H
    value = pixels / (ms / 1e3) / 1e6
    npairs = int(rz.num_pairs.item())

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "Mpixels/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "spheres_1m_1024x1024", "primitives": scene.n, "width": W, "height": H,
                   "channels": scene.channels, "views": 1, "pairs": npairs},
        "stage_ms": {k: round(v, 4) for k, v in st_ms.items()},
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(scene, g_np, args.cpu_sample_rows)
        out["cpu_baseline"] = cpu["json"]
    out["roofline"] = roofline(st_ms, cpu, scene)
    print(json.dumps(out), flush=True)


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


def roofline(st_ms, cpu, scene):
    """Forward compositor against the single-issue VALU peak, from the oracle's
    exact count of list entries examined and contributions made per pixel."""
    fwd_ms = st_ms["render_fwd"]
    if cpu is None or cpu["rows"] != cpu["H"]:
        return {"bound": "alu", "kernel": "k_fwd_sphere", "achieved": None, "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "Tops/s", "frac": None, "traffic": None}
    ops = cpu["processed"] * OPS_PER_ENTRY + cpu["hits"] * (OPS_PER_HIT_BASE + scene.channels)
    achieved = ops / (fwd_ms / 1e3) / 1e12
    return {"bound": "alu", "kernel": "k_fwd_sphere", "achieved": round(achieved, 3),
            "peak": round(VALU_PEAK_TOPS, 2), "unit": "Tops/s", "frac": round(achieved / VALU_PEAK_TOPS, 4),
            "traffic": None, "ops_per_launch": ops}


if __name__ == "__main__":
    main()

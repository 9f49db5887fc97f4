"""ctypes binding of libsplat_peaks (include/splat_peaks.h): measurement kernels
that give the roofline its peaks as measured on the GPU at hand. Argument
marshalling and timing only; the kernels are in csrc/peaks.hip."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsplat_peaks.so")
EXPORTS = ("splat_peaks_copy", "splat_peaks_fma_per_iter", "splat_peaks_lds", "splat_peaks_lds_bytes_per_iter",
           "splat_peaks_valu", "splat_peaks_valu64", "splat_peaks_wall_clock_khz")
_lib = None


def load():
    """The loaded library (fails loudly when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        lib = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int, C.c_size_t
        lib.splat_peaks_valu.argtypes = [vp, vp, i32, i32, vp]
        lib.splat_peaks_valu64.argtypes = [vp, vp, i32, i32, vp]
        lib.splat_peaks_copy.argtypes = [vp, vp, sz, i32, vp]
        lib.splat_peaks_lds.argtypes = [vp, i32, i32, vp]
        lib.splat_peaks_wall_clock_khz.argtypes = [i32, C.POINTER(i32)]
        for f in EXPORTS:
            getattr(lib, f).restype = i32
        _lib = lib
    return _lib


def _ptr(t):
    return C.c_void_p(t.data_ptr())


def _stream(torch, dev):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _timed(torch, launch, reps=1):
    """Best event time (ms) of `reps` launches; raises if a launch fails."""
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = launch()
        e1.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"peak probe failed ({rc})")
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return best


def valu(torch, dev, blocks=4096, iters=20000, fp64=False):
    """(sustained shader clock in MHz, fp32 (or fp64) FMA lane-ops per second, no
    packed math)."""
    import numpy as np
    lib, st = load(), _stream(torch, dev)
    fn = lib.splat_peaks_valu64 if fp64 else lib.splat_peaks_valu
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    _timed(torch, lambda: fn(_ptr(clk), _ptr(sink), blocks, max(1, iters // 20), st))
    ms = _timed(torch, lambda: fn(_ptr(clk), _ptr(sink), blocks, iters, st))
    khz = C.c_int(0)
    if lib.splat_peaks_wall_clock_khz(dev.index or 0, C.byref(khz)) != 0 or khz.value <= 0:
        raise RuntimeError("wall clock rate query failed")
    c = clk.cpu().numpy().reshape(-1, 2).astype(np.float64)
    mhz = float(np.median(c[:, 0] / (c[:, 1] / (khz.value * 1e3)))) / 1e6
    fma = blocks * 256 * iters * lib.splat_peaks_fma_per_iter()
    return mhz, fma / (ms / 1e3)


def copy(torch, dev, src, dst, blocks=8192, reps=5):
    """dst = src; returns bytes read + written per second (best of `reps`)."""
    lib, st = load(), _stream(torch, dev)
    nbytes = src.numel() * src.element_size()
    ms = _timed(torch, lambda: lib.splat_peaks_copy(_ptr(src), _ptr(dst), nbytes, blocks, st), reps)
    return 2 * nbytes / (ms / 1e3)


def lds(torch, dev, sink, blocks, iters):
    """Broadcast LDS reads into sink [blocks * 256] int32; returns bytes delivered per second."""
    lib, st = load(), _stream(torch, dev)
    ms = _timed(torch, lambda: lib.splat_peaks_lds(_ptr(sink), blocks, iters, st))
    return blocks * 256 * iters * lib.splat_peaks_lds_bytes_per_iter() / (ms / 1e3)


def measure(torch, dev):
    """The benchmark's measured peaks (the copy: the best of several grids)."""
    mhz, fma = valu(torch, dev)
    _, fma64 = valu(torch, dev, fp64=True)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    gbs = 0.0
    for blocks in (8192, 32768, 131072):
        copy(torch, dev, src, dst, blocks=blocks, reps=1)
        gbs = max(gbs, copy(torch, dev, src, dst, blocks=blocks) / 1e9)
    del src, dst
    lblocks = 2048
    sink = torch.empty(lblocks * 256, dtype=torch.int32, device=dev)
    lds(torch, dev, sink, lblocks, 100)
    tbs = lds(torch, dev, sink, lblocks, 2000) / 1e12
    return {"clock_mhz": round(mhz, 1),
            "valu_fma_Tlane_ops": round(fma / 1e12, 2),
            "valu_fma64_Tlane_ops": round(fma64 / 1e12, 2),
            "valu_at_clock_Tlane_ops": round(256 * 64 * mhz * 1e6 / 1e12, 2),
            "hbm_copy_GBps": round(gbs, 1),
            "lds_broadcast_TBps": round(tbs, 2)}

"""ctypes binding of libsplat's C ABI (include/splat.h).

Argument marshalling only: each function here has the name of the C entry
point it calls and passes device pointers (ints) straight through. The
library must be built (see build.py); nothing here computes any part of the
rasterizer, and there is no fallback when the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsplat.so")

SPLAT_OK, SPLAT_ERR_INVALID_ARG, SPLAT_ERR_CAPACITY, SPLAT_ERR_HIP, SPLAT_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
SPLAT_PRIM_GAUSS2D, SPLAT_PRIM_GAUSS3D, SPLAT_PRIM_SPHERE = 0, 1, 2
SPLAT_CAM_PINHOLE, SPLAT_CAM_SPHERICAL = 0, 1
SPLAT_MAX_VIEWS, SPLAT_MAX_CHANNELS = 16, 64

# include/splat.h: size of the fixed device array splat_bin_sort_noalloc sorts in
SPLAT_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ["splat_projected_bytes", "splat_total_tiles", "splat_sort_workspace_bytes",
           "splat_bwd_workspace_bytes", "splat_project", "splat_bin_sort", "splat_bin_sort_noalloc", "splat_render_fwd",
           "splat_render_bwd", "splat_interpolate", "splat_interpolate_bwd", "splat_status_string"]


class splat_camera(C.Structure):
    _fields_ = [("kind", C.c_int32), ("width", C.c_int32), ("height", C.c_int32),
                ("R", C.c_float * 9), ("t", C.c_float * 3),
                ("fx", C.c_float), ("fy", C.c_float), ("cx", C.c_float), ("cy", C.c_float),
                ("el_min_deg", C.c_float), ("el_max_deg", C.c_float),
                ("znear", C.c_float), ("zfar", C.c_float)]


class splat_prims(C.Structure):
    _fields_ = [("kind", C.c_int32), ("n", C.c_int32), ("channels", C.c_int32),
                ("pos", C.c_void_p), ("scale", C.c_void_p), ("rot", C.c_void_p),
                ("opacity", C.c_void_p), ("depth", C.c_void_p), ("feat", C.c_void_p)]


class splat_params(C.Structure):
    _fields_ = [("alpha_min", C.c_float), ("alpha_max", C.c_float), ("T_min", C.c_float),
                ("gamma", C.c_float), ("bg_weight", C.c_float), ("tau", C.c_float),
                ("top_k", C.c_int32), ("background", C.POINTER(C.c_float)), ("top_by_depth", C.c_int32),
                ("max_shift", C.c_int32), ("serial_views", C.c_int32)]


class splat_grads(C.Structure):
    _fields_ = [("pos", C.c_void_p), ("scale", C.c_void_p), ("rot", C.c_void_p),
                ("opacity", C.c_void_p), ("feat", C.c_void_p), ("cam_R", C.c_void_p),
                ("cam_t", C.c_void_p), ("cam_K", C.c_void_p), ("accumulate", C.c_int32),
                ("normalize", C.c_int32), ("sums_cleared", C.c_int32),
                ("atomic_direct_max", C.c_int32)]


class SplatError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


_L = None


def lib():
    """Load libsplat.so (raises if it has not been built)."""
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (sphere_rasterization_amd.build)")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
        cam_p = C.POINTER(splat_camera)
        L.splat_projected_bytes.restype = sz
        L.splat_projected_bytes.argtypes = [i32, i32]
        L.splat_total_tiles.restype = i64
        L.splat_total_tiles.argtypes = [cam_p, i32]
        L.splat_sort_workspace_bytes.restype = sz
        L.splat_sort_workspace_bytes.argtypes = [cam_p, i32, i32, i64]
        L.splat_bwd_workspace_bytes.restype = sz
        L.splat_bwd_workspace_bytes.argtypes = [i32, i32, i32]
        L.splat_project.restype = i32
        L.splat_project.argtypes = [cam_p, i32, C.POINTER(splat_prims), C.POINTER(splat_params), vp, vp, vp]
        L.splat_bin_sort.restype = i32
        L.splat_bin_sort.argtypes = [cam_p, i32, i32, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.splat_bin_sort_noalloc.restype = i32
        L.splat_bin_sort_noalloc.argtypes = [cam_p, i32, i32, vp, vp, i64, vp, vp, vp, vp, vp, vp]
        L.splat_render_fwd.restype = i32
        L.splat_render_fwd.argtypes = [cam_p, i32, C.POINTER(splat_prims), C.POINTER(splat_params), vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.splat_render_bwd.restype = i32
        L.splat_render_bwd.argtypes = [cam_p, i32, i32, i32, C.POINTER(splat_prims), C.POINTER(splat_params),
                                       vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, C.POINTER(splat_grads), vp, sz, vp]
        fp = C.POINTER(C.c_float)
        L.splat_interpolate.restype = i32
        L.splat_interpolate.argtypes = [fp, i32, C.c_float, i32, vp, vp, vp, vp, vp]
        L.splat_interpolate_bwd.restype = i32
        L.splat_interpolate_bwd.argtypes = [fp, i32, C.c_float, i32, vp, vp, vp, vp, vp, vp]
        L.splat_status_string.restype = C.c_char_p
        L.splat_status_string.argtypes = [i32]
        _L = L
    return _L


def status_string(status: int) -> str:
    return lib().splat_status_string(int(status)).decode()


def _check(fn, st):
    if st != SPLAT_OK:
        raise SplatError(fn, st)
    return st


# ---- same names as the C entry points ---------------------------------------

def splat_projected_bytes(n_views, n):
    return lib().splat_projected_bytes(n_views, n)


def splat_total_tiles(cams, n_views):
    return lib().splat_total_tiles(cams, n_views)


def splat_sort_workspace_bytes(cams, n_views, n, capacity):
    return lib().splat_sort_workspace_bytes(cams, n_views, n, capacity)


def splat_bwd_workspace_bytes(n_views, n, channels):
    return lib().splat_bwd_workspace_bytes(n_views, n, channels)


def splat_project(cams, n_views, prims, params, proj, pair_counts, stream):
    return _check("splat_project", lib().splat_project(cams, n_views, C.byref(prims), C.byref(params), proj,
                                                       pair_counts, stream))


def splat_bin_sort(cams, n_views, n, proj, pair_counts, capacity, keys, vals, tile_ranges, num_pairs, overflow,
                   workspace, ws_bytes, stream):
    return _check("splat_bin_sort", lib().splat_bin_sort(cams, n_views, n, proj, pair_counts, capacity, keys, vals,
                                                         tile_ranges, num_pairs, overflow, workspace, ws_bytes,
                                                         stream))


def splat_bin_sort_noalloc(cams, n_views, n, proj, pair_counts, capacity, keys, vals, tile_ranges, num_pairs,
                           overflow, stream):
    return _check("splat_bin_sort_noalloc", lib().splat_bin_sort_noalloc(cams, n_views, n, proj, pair_counts,
                                                                         capacity, keys, vals, tile_ranges,
                                                                         num_pairs, overflow, stream))


def splat_render_fwd(cams, n_views, prims, params, proj, vals, tile_ranges, overflow, img, T_final, last, norm, topk,
                     bwd_workspace, bwd_ws_bytes, stream):
    return _check("splat_render_fwd", lib().splat_render_fwd(cams, n_views, C.byref(prims), C.byref(params), proj,
                                                             vals, tile_ranges, overflow, img, T_final, last, norm,
                                                             topk, bwd_workspace, bwd_ws_bytes, stream))


def splat_render_bwd(cams, n_views, view_begin, view_count, prims, params, proj, vals, tile_ranges, overflow, img,
                     T_final, last, norm, topk, dL_dimg, grads, workspace, ws_bytes, stream):
    return _check("splat_render_bwd", lib().splat_render_bwd(cams, n_views, view_begin, view_count, C.byref(prims),
                                                             C.byref(params), proj, vals, tile_ranges, overflow, img,
                                                             T_final, last, norm, topk, dL_dimg, C.byref(grads),
                                                             workspace, ws_bytes, stream))


def _times(key_times):
    kt = (C.c_float * len(key_times))(*[float(x) for x in key_times])
    return kt, len(key_times)


def splat_interpolate(key_times, t, n, key_pos, key_rot, pos, rot, stream):
    kt, nk = _times(key_times)
    return _check("splat_interpolate", lib().splat_interpolate(kt, nk, float(t), n, key_pos, key_rot, pos, rot,
                                                               stream))


def splat_interpolate_bwd(key_times, t, n, key_rot, d_pos, d_rot, d_key_pos, d_key_rot, stream):
    kt, nk = _times(key_times)
    return _check("splat_interpolate_bwd", lib().splat_interpolate_bwd(kt, nk, float(t), n, key_rot, d_pos, d_rot,
                                                                       d_key_pos, d_key_rot, stream))

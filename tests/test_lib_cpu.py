"""The C-ABI library builds, loads and exports what include/splat.h declares;
host-side size queries and argument checks work with no GPU present."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from sphere_rasterization_amd import _lib as L
from sphere_rasterization_amd import scenes as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "splat.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(splat_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    assert os.path.exists(L.LIB_PATH), "build libsplat.so first"
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (splat_[a-z_]+)$", out, flags=re.M))
    declared = _declared()
    assert len(declared) >= 9
    missing = [d for d in declared if d not in exported]
    assert not missing, missing
    assert sorted(L.EXPORTS) == declared
    lib = L.lib()
    for d in declared:
        assert hasattr(lib, d)


def test_size_queries():
    from sphere_rasterization_amd.raster import make_cams
    sc = S.pulsar_spheres(n=10)
    cams = make_cams(sc.cams)
    assert L.splat_total_tiles(cams, 1) == 64 * 64
    assert L.splat_projected_bytes(1, 1000) >= 1000 * (16 + 32 + 32)
    assert L.splat_sort_workspace_bytes(cams, 1, 1000, 5000) >= 5000 * 12
    assert L.splat_bwd_workspace_bytes(1, 1000, 3) >= 1000 * 11 * 4
    multi = make_cams(S.multisensor(n=10).cams)
    assert L.splat_total_tiles(multi, 7) == 6 * 80 * 45 + 128 * 4
    bad = make_cams([S.Camera(S.CAM_SPHERICAL, 100, 32, np.eye(3), np.zeros(3), el_min_deg=-10, el_max_deg=10)])
    assert L.splat_total_tiles(bad, 1) == -1          # spherical width must be a multiple of 16
    assert L.status_string(L.SPLAT_ERR_CAPACITY) == "buffer or workspace too small"


def test_argument_errors_are_returned_before_any_launch():
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.pulsar_spheres(n=10)
    cams = make_cams(sc.cams)
    prm, _ = make_params(sc.params, 3)
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 2, 10, 3
    lib = L.lib()
    assert lib.splat_project(None, 1, C.byref(pr), C.byref(prm), None, None, None) == L.SPLAT_ERR_INVALID_ARG
    assert lib.splat_project(cams, 0, C.byref(pr), C.byref(prm), None, None, None) == L.SPLAT_ERR_INVALID_ARG
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), None, None, None) == L.SPLAT_ERR_INVALID_ARG
    pr.kind = 7
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), None, None, None) == L.SPLAT_ERR_INVALID_ARG
    pr.kind = 2
    prm.top_k = 9
    assert lib.splat_render_fwd(cams, 1, C.byref(pr), C.byref(prm), None, None, None, None, None, None, None, None,
                                None, None, 0, None) == L.SPLAT_ERR_INVALID_ARG
    lid = make_cams([S.Camera(S.CAM_SPHERICAL, 128, 32, np.eye(3), np.zeros(3), el_min_deg=-10, el_max_deg=10)])
    prm.top_k = 5
    pr.pos = pr.scale = pr.opacity = pr.feat = 8
    assert lib.splat_project(lid, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_UNSUPPORTED
    # workspace smaller than the query
    ws = L.splat_sort_workspace_bytes(cams, 1, 10, 100)
    rc = lib.splat_bin_sort(cams, 1, 10, 8, 8, 100, 8, 8, 8, 8, 8, 8, ws - 1, None)
    assert rc == L.SPLAT_ERR_CAPACITY
    rc = lib.splat_bin_sort(cams, 1, 10, 8, 8, -1, 8, 8, 8, 8, 8, 8, ws, None)
    assert rc == L.SPLAT_ERR_INVALID_ARG


def test_orthographic_views_and_intrinsic_gradients_are_sphere_only():
    """An orthographic view with Gaussian primitives, and intrinsic gradients
    requested for Gaussians, are refused on the host (no launch)."""
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.pulsar_spheres(n=10)
    prm, _ = make_params(sc.params, 3)
    orth = make_cams([S.Camera(S.CAM_ORTHO, 64, 48, np.eye(3), np.zeros(3), fx=10.0, fy=10.0, cx=32.0, cy=24.0,
                               znear=1.0, zfar=21.0)])
    assert L.splat_total_tiles(orth, 1) == 4 * 3
    bad = make_cams([S.Camera(S.CAM_ORTHO, 64, 48, np.eye(3), np.zeros(3), fx=0.0, fy=10.0, cx=32.0, cy=24.0)])
    assert L.splat_total_tiles(bad, 1) == -1          # scale must be positive
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 1, 10, 3
    pr.pos = pr.scale = pr.rot = pr.opacity = pr.feat = 8
    assert lib.splat_project(orth, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_UNSUPPORTED
    pin = make_cams(sc.cams)
    g = L.splat_grads()
    g.cam_K = 8
    rc = lib.splat_render_bwd(pin, 1, 0, 1, C.byref(pr), C.byref(prm), 8, 8, 8, 8, 8, 8, 8, None, None, 8,
                              C.byref(g), 8, 1 << 40, None)
    assert rc == L.SPLAT_ERR_UNSUPPORTED


def test_gradient_normalisation_is_sphere_only():
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.pulsar_spheres(n=10)
    prm, _ = make_params(sc.params, 3)
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 1, 10, 3
    pr.pos = pr.scale = pr.rot = pr.opacity = pr.feat = 8
    g = L.splat_grads()
    g.normalize = 1
    rc = lib.splat_render_bwd(make_cams(sc.cams), 1, 0, 1, C.byref(pr), C.byref(prm), 8, 8, 8, 8, 8, 8, 8, None,
                              None, 8, C.byref(g), 8, 1 << 40, None)
    assert rc == L.SPLAT_ERR_UNSUPPORTED


def test_top_by_depth_values():
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.pulsar_spheres(n=10)
    cams = make_cams(sc.cams)
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 2, 10, 3
    pr.pos = pr.scale = pr.opacity = pr.feat = 8
    prm, _ = make_params(S.Params(top_by_depth=2), 3)
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_INVALID_ARG
    pr.kind = 1
    pr.rot = 8
    prm, _ = make_params(S.Params(top_by_depth=1), 3)
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_UNSUPPORTED


def test_interpolate_argument_errors():
    lib = L.lib()
    good = (C.c_float * 3)(0.0, 1.0, 2.0)
    bad = (C.c_float * 3)(0.0, 2.0, 1.0)
    assert lib.splat_interpolate(bad, 3, 0.5, 10, 16, 16, 16, 16, None) == L.SPLAT_ERR_INVALID_ARG
    assert lib.splat_interpolate(good, 0, 0.5, 10, 16, 16, 16, 16, None) == L.SPLAT_ERR_INVALID_ARG
    assert lib.splat_interpolate(good, 3, float("nan"), 10, 16, 16, 16, 16, None) == L.SPLAT_ERR_INVALID_ARG
    assert lib.splat_interpolate(good, 3, 0.5, -1, 16, 16, 16, 16, None) == L.SPLAT_ERR_INVALID_ARG
    assert lib.splat_interpolate(good, 3, 0.5, 10, None, None, None, None, None) == L.SPLAT_ERR_INVALID_ARG
    assert lib.splat_interpolate(good, 3, 0.5, 10, 16, 20, 16, 16, None) == L.SPLAT_ERR_INVALID_ARG   # misaligned
    assert lib.splat_interpolate_bwd(good, 3, 0.5, 10, None, 16, 16, 16, 16, None) == L.SPLAT_ERR_INVALID_ARG


def test_small_gamma_needs_max_shift():
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.pulsar_spheres(n=10)
    cams = make_cams(sc.cams)
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 2, 10, 3
    pr.pos = pr.scale = pr.opacity = pr.feat = 8
    prm, _ = make_params(S.Params(gamma=0.005), 3)
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_INVALID_ARG
    prm, _ = make_params(S.Params(gamma=0.02, max_shift=3), 3)
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_INVALID_ARG
    pr.kind, pr.rot = 1, 8
    prm, _ = make_params(S.Params(max_shift=1), 3)
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_UNSUPPORTED


def test_sphere_views_need_a_depth_span():
    """Spheres normalise depth by zfar - znear: a view with zfar <= znear is
    refused on the host (no launch)."""
    from sphere_rasterization_amd.raster import make_cams, make_params
    prm, _ = make_params(S.Params(), 3)
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 2, 10, 3
    pr.pos = pr.scale = pr.opacity = pr.feat = 8
    for zn, zf in ((1.0, 1.0), (5.0, 2.0)):
        cams = make_cams([S.Camera(S.CAM_PINHOLE, 64, 64, np.eye(3), np.zeros(3), fx=64.0, fy=64.0, cx=32.0,
                                   cy=32.0, znear=zn, zfar=zf)])
        assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_INVALID_ARG


def test_gaussian_T_min_floor():
    """A transmittance threshold that would let the stored fp32 T_final underflow
    (the reverse pass divides it back) is refused for Gaussians."""
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.gauss3d(n=10)
    cams = make_cams(sc.cams)
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 1, 10, 3
    pr.pos = pr.scale = pr.rot = pr.opacity = pr.feat = 8
    for tmin in (0.0, 1e-35):
        prm, _ = make_params(S.Params(T_min=tmin), 3)
        assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_INVALID_ARG


def test_noalloc_sort_size_limit_on_host():
    """splat_bin_sort_noalloc: the header's array size matches the binding's, and a
    workspace beyond it is refused on the host (no device touched)."""
    src = open(os.path.join(ROOT, "include", "splat.h")).read()
    m = re.search(r"#define SPLAT_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == L.SPLAT_NOALLOC_SCRATCH_BYTES
    from sphere_rasterization_amd.raster import make_cams
    sc = S.pulsar_spheres(n=10)
    cams = make_cams(sc.cams)
    big = 16 << 20
    assert L.splat_sort_workspace_bytes(cams, 1, 10, big) > L.SPLAT_NOALLOC_SCRATCH_BYTES
    lib = L.lib()
    assert lib.splat_bin_sort_noalloc(cams, 1, 10, 8, 8, big, 8, 8, 8, 8, 8, None) == L.SPLAT_ERR_CAPACITY
    assert lib.splat_bin_sort_noalloc(cams, 1, 10, 8, 8, 100, 8, 8, None, 8, 8, None) == L.SPLAT_ERR_INVALID_ARG


def test_negative_atomic_direct_max_is_rejected():
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.pulsar_spheres(n=10)
    prm, _ = make_params(sc.params, 3)
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 2, 10, 3
    pr.pos = pr.scale = pr.opacity = pr.feat = 8
    g = L.splat_grads()
    g.atomic_direct_max = -1
    rc = lib.splat_render_bwd(make_cams(sc.cams), 1, 0, 1, C.byref(pr), C.byref(prm), 8, 8, 8, 8, 8, None, None, 8,
                              8, 8, C.byref(g), 8, 1 << 40, None)
    assert rc == L.SPLAT_ERR_INVALID_ARG


def test_serial_views_values():
    from sphere_rasterization_amd.raster import make_cams, make_params
    sc = S.gauss3d(n=10)
    lib = L.lib()
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = 1, 10, 3
    pr.pos = pr.scale = pr.rot = pr.opacity = pr.feat = 8
    prm, _ = make_params(S.Params(serial_views=2), 3)
    assert lib.splat_project(make_cams(sc.cams), 1, C.byref(pr), C.byref(prm), 8, 8, None) == L.SPLAT_ERR_INVALID_ARG


def test_peaks_library_exports_every_declared_symbol():
    from sphere_rasterization_amd import peaks as PK
    assert os.path.exists(PK.LIB_PATH), "build libsplat_peaks.so first"
    src = open(os.path.join(ROOT, "include", "splat_peaks.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    declared = sorted(set(re.findall(r"\b(splat_peaks_[a-z0-9_]+)\s*\(", src)))
    out = subprocess.run(["nm", "-D", "--defined-only", PK.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (splat_peaks_[a-z0-9_]+)$", out, flags=re.M))
    assert declared and sorted(PK.EXPORTS) == declared
    assert not [d for d in declared if d not in exported]
    lib = PK.load()
    assert lib.splat_peaks_fma_per_iter() == 8 and lib.splat_peaks_lds_bytes_per_iter() == 128
    # argument errors are returned before any launch
    assert lib.splat_peaks_copy(None, None, 16, 1, None) == -1
    assert lib.splat_peaks_lds(None, 1, 1, None) == -1
    assert lib.splat_peaks_valu(None, None, 1, 1, None) == -1
    assert lib.splat_peaks_valu64(None, None, 1, 1, None) == -1


def test_sort_word_order_reads_alike_as_fp64():
    """The segment sort compares its (depth bits << 32 | record) words partly as
    fp64 (v_min_f64 / v_max_f64) and partly as 64-bit unsigned integers, and
    pads with the largest finite double. For words whose high half is a
    non-negative fp32 bit pattern (zero, denormal, normal, infinity: every key
    the projection writes) both readings must order alike, and none may be a
    NaN."""
    rng = np.random.default_rng(5)
    hi = np.concatenate([
        np.array([0, 1, 2, 0x007FFFFF, 0x00800000, 0x3F800000, 0x7F7FFFFF, 0x7F800000], np.uint64),
        rng.integers(0, 0x7F800001, size=4000, dtype=np.uint64),
    ])
    lo = rng.integers(0, 1 << 32, size=hi.size, dtype=np.uint64)
    lo[:8] = np.array([0, 1, 0xFFFFFFFF, 7, 0, 12345, 0xFFFFFFFF, 0xFFFFFFFF], np.uint64)
    words = np.concatenate([(hi << np.uint64(32)) | lo, np.array([0x7FEFFFFFFFFFFFFF], np.uint64)])
    as_f64 = words.view(np.float64)
    assert np.isfinite(as_f64).all() and (as_f64 >= 0).all()
    assert as_f64[-1] == np.finfo(np.float64).max and words[-1] > words[:-1].max()
    np.testing.assert_array_equal(np.argsort(words, kind="stable"), np.argsort(as_f64, kind="stable"))
    # pairwise: min / max of two words agree in both readings
    a, b = words[:-1:2], words[1::2]
    fa, fb = as_f64[:-1:2], as_f64[1::2]
    np.testing.assert_array_equal(np.minimum(fa, fb).view(np.uint64), np.minimum(a, b))
    np.testing.assert_array_equal(np.maximum(fa, fb).view(np.uint64), np.maximum(a, b))

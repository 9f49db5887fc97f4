"""splat_bin_sort_noalloc (sort workspace in the library's fixed device array)
against splat_bin_sort (caller's workspace): bit-identical keys, values, tile
ranges, pair count and overflow flag, on consecutive calls whose second input
is smaller (the array keeps the previous call's contents)."""
import ctypes as C

import numpy as np
import pytest
import torch

from sphere_rasterization_amd import _lib as L
from sphere_rasterization_amd import scenes as S
from tests import oracle_scenes as TS

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _sort_both(sc, name):
    from sphere_rasterization_amd.raster import Rasterizer
    _log(f"[case] no-alloc sort: {name}")
    rz = Rasterizer(sc, device="cuda")
    rz.forward(check=True)
    torch.cuda.synchronize()
    need = L.splat_sort_workspace_bytes(rz.c_cams, rz.V, rz.n, rz.capacity)
    assert need <= L.SPLAT_NOALLOC_SCRATCH_BYTES, (need, name)
    ref = dict(keys=rz.keys.clone(), vals=rz.vals.clone(), ranges=rz.tile_ranges.clone(),
               num=rz.num_pairs.clone(), ovf=rz.overflow.clone())
    keys = torch.full_like(rz.keys, -1)
    vals = torch.full_like(rz.vals, -1)
    ranges = torch.full_like(rz.tile_ranges, -1)
    num = torch.full_like(rz.num_pairs, -1)
    ovf = torch.full_like(rz.overflow, -1)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    L.splat_bin_sort_noalloc(rz.c_cams, rz.V, rz.n, _ptr(rz.proj), _ptr(rz.pair_counts), rz.capacity, _ptr(keys),
                             _ptr(vals), _ptr(ranges), _ptr(num), _ptr(ovf), stream)
    torch.cuda.synchronize()
    n = int(ref["num"].item())
    assert int(num.item()) == n and int(ovf.item()) == int(ref["ovf"].item()) == 0
    assert torch.equal(keys[:n], ref["keys"][:n])
    assert torch.equal(vals[:n], ref["vals"][:n])
    assert torch.equal(ranges, ref["ranges"])
    _log(f"  ok: {n} pairs, workspace {need / 2**20:.1f} MiB")
    return rz


def test_noalloc_sort_matches_workspace_sort():
    # 1M spheres at 1024x1024, then a smaller scene, then a three-view batch
    # (per-view scans, the other scatter path) on the same array
    _sort_both(S.pulsar_spheres(), "spheres 1M @1024x1024")
    _sort_both(S.pulsar_spheres(seed=29, n=60_000, width=320, height=240), "spheres 60k @320x240")
    mv = S.gauss3d(seed=34, n=20_000)
    R1 = TS.rotation(np.random.default_rng(2))
    mv.cams = [mv.cams[0],
               S.Camera(S.CAM_PINHOLE, 320, 200, R1, [0.2, -0.1, 9.0], fx=300.0, fy=310.0, cx=160.0, cy=100.0,
                        znear=0.2, zfar=100.0),
               TS.lidar(512, 64, t=[0.0, 0.0, 0.0])]
    _sort_both(mv, "gauss3d 20k, 2 pinhole + lidar")


def test_noalloc_sort_rejects_oversize():
    """A capacity whose workspace exceeds the array is refused before any launch,
    and a capacity overflow is reported on the device as with splat_bin_sort."""
    from sphere_rasterization_amd.raster import Rasterizer
    sc = S.pulsar_spheres(seed=29, n=60_000, width=320, height=240)
    rz = Rasterizer(sc, device="cuda")
    rz.forward(check=True)
    big = 16 << 20
    assert L.splat_sort_workspace_bytes(rz.c_cams, rz.V, rz.n, big) > L.SPLAT_NOALLOC_SCRATCH_BYTES
    rc = L.lib().splat_bin_sort_noalloc(rz.c_cams, rz.V, rz.n, _ptr(rz.proj), _ptr(rz.pair_counts), big,
                                        _ptr(rz.keys), _ptr(rz.vals), _ptr(rz.tile_ranges), _ptr(rz.num_pairs),
                                        _ptr(rz.overflow), None)
    assert rc == L.SPLAT_ERR_CAPACITY
    # too small a pair capacity: the device-side overflow report
    need = int(rz.num_pairs.item())
    num = torch.zeros_like(rz.num_pairs)
    ovf = torch.zeros_like(rz.overflow)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    L.splat_bin_sort_noalloc(rz.c_cams, rz.V, rz.n, _ptr(rz.proj), _ptr(rz.pair_counts), 1000, _ptr(rz.keys),
                             _ptr(rz.vals), _ptr(rz.tile_ranges), _ptr(num), _ptr(ovf), stream)
    torch.cuda.synchronize()
    assert int(ovf.item()) == 1 and int(num.item()) == need

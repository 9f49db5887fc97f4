"""Buffer management around the four libsplat calls.

torch provides device memory and the stream; every step of projection,
binning, sorting, compositing and the reverse pass runs in libsplat's HIP
kernels through the C ABI (see _lib.py). The only host/device traffic is the
optional overflow check after binning (one 8-byte read), done lazily.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional

import numpy as np
import torch

from . import _lib as L
from .scenes import CAM_SPHERICAL, Camera, Params, Scene


def make_cams(cams: List[Camera]):
    arr = (L.splat_camera * len(cams))()
    for v, c in enumerate(cams):
        a = arr[v]
        a.kind, a.width, a.height = int(c.kind), int(c.width), int(c.height)
        for k, x in enumerate(np.asarray(c.R, np.float32).reshape(9)):
            a.R[k] = float(x)
        for k, x in enumerate(np.asarray(c.t, np.float32).reshape(3)):
            a.t[k] = float(x)
        a.fx, a.fy, a.cx, a.cy = c.fx, c.fy, c.cx, c.cy
        a.el_min_deg, a.el_max_deg, a.znear, a.zfar = c.el_min_deg, c.el_max_deg, c.znear, c.zfar
    return arr


def make_params(p: Params, channels: int):
    s = L.splat_params()
    s.alpha_min, s.alpha_max, s.T_min = p.alpha_min, p.alpha_max, p.T_min
    s.gamma, s.bg_weight, s.tau, s.top_k = p.gamma, p.bg_weight, p.tau, int(p.top_k)
    s.top_by_depth = int(getattr(p, "top_by_depth", 0))
    s.max_shift = int(getattr(p, "max_shift", 0))
    s.serial_views = int(getattr(p, "serial_views", 0))
    keep = None
    if p.background is not None:
        keep = (C.c_float * channels)(*[float(x) for x in np.asarray(p.background, np.float32)[:channels]])
        s.background = C.cast(keep, C.POINTER(C.c_float))
    return s, keep


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class Rasterizer:
    """One scene (device tensors) seen by a fixed set of views."""

    def __init__(self, scene: Scene, device="cuda", capacity: Optional[int] = None,
                 tensors: Optional[Dict[str, torch.Tensor]] = None):
        self.scene = scene
        self.device = torch.device(device)
        self.kind, self.n, self.C = scene.kind, scene.n, scene.channels
        self.cams = list(scene.cams)
        self.V = len(self.cams)
        self.t = tensors if tensors is not None else self.upload(scene, self.device)
        self.c_cams = make_cams(self.cams)
        self.c_params, self._bg_keep = make_params(scene.params, self.C)
        self.c_prims = L.splat_prims()
        self._bind_prims()
        V, n, dev = self.V, self.n, self.device
        self.total_tiles = L.splat_total_tiles(self.c_cams, V)
        self.total_pix = sum(c.width * c.height for c in self.cams)
        self.img_sizes = [scene.view_channels(v) * c.width * c.height for v, c in enumerate(self.cams)]
        self.proj = torch.empty(L.splat_projected_bytes(V, n), dtype=torch.uint8, device=dev)
        self.pair_counts = torch.empty(V * n, dtype=torch.int32, device=dev)
        self.tile_ranges = torch.empty(2 * self.total_tiles, dtype=torch.int32, device=dev)
        self.num_pairs = torch.zeros(1, dtype=torch.int64, device=dev)
        self.overflow = torch.zeros(1, dtype=torch.int32, device=dev)
        self.img = torch.empty(sum(self.img_sizes), dtype=torch.float32, device=dev)
        sph = self.kind == 2
        # spheres use T_final only for the per-pixel shift of max-shifted blending
        need_T = (not sph) or bool(getattr(scene.params, "max_shift", 0))
        self.T_final = torch.empty(self.total_pix, dtype=torch.float32, device=dev) if need_T else None
        self.last = None if sph else torch.empty(self.total_pix, dtype=torch.int32, device=dev)
        K = scene.params.top_k
        self.norm = torch.empty(self.total_pix, dtype=torch.float32, device=dev) if sph else None
        self.topk = torch.empty(self.total_pix * K, dtype=torch.int32, device=dev) if sph else None
        self.bwd_ws = None
        self.sums_cleared = False   # the last forward cleared the backward's sums
        self.capacity = 0
        self._alloc_pairs(capacity if capacity is not None else max(1024, 4 * V * n))

    @staticmethod
    def upload(scene: Scene, device) -> Dict[str, torch.Tensor]:
        out = {}
        for k in ("pos", "scale", "rot", "opacity", "depth", "feat"):
            a = getattr(scene, k)
            out[k] = None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
        return out

    def _bind_prims(self):
        p, t = self.c_prims, self.t
        p.kind, p.n, p.channels = self.kind, self.n, self.C
        p.pos, p.scale, p.rot = _ptr(t["pos"]), _ptr(t["scale"]), _ptr(t.get("rot"))
        p.opacity, p.depth, p.feat = _ptr(t["opacity"]), _ptr(t.get("depth")), _ptr(t.get("feat"))

    def _alloc_pairs(self, capacity: int):
        capacity = int(min(capacity, 2 ** 32 - 2))
        self.capacity = capacity
        self.keys = torch.empty(max(capacity, 1), dtype=torch.int64, device=self.device)
        self.vals = torch.empty(max(capacity, 1), dtype=torch.int32, device=self.device)
        self.sort_ws_bytes = L.splat_sort_workspace_bytes(self.c_cams, self.V, self.n, capacity)
        self.sort_ws = torch.empty(max(self.sort_ws_bytes, 1), dtype=torch.uint8, device=self.device)

    # ---- the four calls -------------------------------------------------
    def project(self):
        L.splat_project(self.c_cams, self.V, self.c_prims, self.c_params, _ptr(self.proj),
                        _ptr(self.pair_counts), _stream())

    def bin_sort(self):
        L.splat_bin_sort(self.c_cams, self.V, self.n, _ptr(self.proj), _ptr(self.pair_counts), self.capacity,
                         _ptr(self.keys), _ptr(self.vals), _ptr(self.tile_ranges), _ptr(self.num_pairs),
                         _ptr(self.overflow), _ptr(self.sort_ws), self.sort_ws_bytes, _stream())

    def render_fwd(self):
        # once a backward has allocated its workspace, the forward clears the sums
        # the next backward accumulates into (the library skips its own clearing)
        ws = self.bwd_ws
        L.splat_render_fwd(self.c_cams, self.V, self.c_prims, self.c_params, _ptr(self.proj), _ptr(self.vals),
                           _ptr(self.tile_ranges), _ptr(self.overflow), _ptr(self.img), _ptr(self.T_final),
                           _ptr(self.last), _ptr(self.norm), _ptr(self.topk), _ptr(ws),
                           self.bwd_ws_bytes if ws is not None else 0, _stream())
        self.sums_cleared = ws is not None

    def ensure_capacity(self, slack: float = 1.25) -> bool:
        """Read the pair count (one small device->host copy); grow and re-bin on
        overflow, or shrink a capacity more than twice what is needed."""
        need = int(self.num_pairs.item())
        if need > self.capacity:
            self._alloc_pairs(int(need * slack) + 1024)
            self.bin_sort()
            return True
        if self.capacity > 2 * (int(need * slack) + 1024):
            self._alloc_pairs(int(need * slack) + 1024)
            self.bin_sort()
        return False

    def forward(self, check: bool = True):
        self.project()
        self.bin_sort()
        if check:
            self.ensure_capacity()
        self.render_fwd()
        return self.img

    def backward(self, dimg: torch.Tensor, want=("pos", "scale", "rot", "opacity", "feat", "cam_R", "cam_t", "cam_K"),
                 view_begin: int = 0, view_count: Optional[int] = None, grads=None, accumulate=False,
                 normalize=False, atomic_direct_max: int = 0):
        if view_count is None:
            view_count = self.V - view_begin
        if self.bwd_ws is None:
            self.bwd_ws_bytes = L.splat_bwd_workspace_bytes(self.V, self.n, self.C)
            self.bwd_ws = torch.empty(max(self.bwd_ws_bytes, 1), dtype=torch.uint8, device=self.device)
        if grads is None:
            grads = self.alloc_grads(want)
        g = L.splat_grads()
        for k in ("pos", "scale", "rot", "opacity", "feat", "cam_R", "cam_t", "cam_K"):
            setattr(g, k, _ptr(grads.get(k)))
        g.accumulate = 1 if accumulate else 0
        g.normalize = 1 if normalize else 0
        g.atomic_direct_max = int(atomic_direct_max)
        # only the first backward after a clearing forward may skip the clearing
        g.sums_cleared = 1 if self.sums_cleared else 0
        self.sums_cleared = False
        L.splat_render_bwd(self.c_cams, self.V, view_begin, view_count, self.c_prims, self.c_params,
                           _ptr(self.proj), _ptr(self.vals), _ptr(self.tile_ranges), _ptr(self.overflow),
                           _ptr(self.img), _ptr(self.T_final), _ptr(self.last), _ptr(self.norm), _ptr(self.topk),
                           _ptr(dimg), g, _ptr(self.bwd_ws), self.bwd_ws_bytes, _stream())
        return grads

    def alloc_grads(self, want) -> Dict[str, torch.Tensor]:
        out = {}
        for k in want:
            if k in ("cam_R", "cam_t", "cam_K"):
                if self.kind != 2:
                    continue
                out[k] = torch.zeros((self.V, {"cam_R": 9, "cam_t": 3, "cam_K": 4}[k]), dtype=torch.float32,
                                     device=self.device)
            else:
                src = self.t.get(k)
                if src is None:
                    continue
                out[k] = torch.zeros_like(src)
        return out

    # ---- views of the outputs -------------------------------------------
    def view_images(self, flat: Optional[torch.Tensor] = None) -> List[torch.Tensor]:
        flat = self.img if flat is None else flat
        out, off = [], 0
        for v, c in enumerate(self.cams):
            sz = self.img_sizes[v]
            out.append(flat[off:off + sz].view(self.scene.view_channels(v), c.height, c.width))
            off += sz
        return out

    def view_pixels(self, t: torch.Tensor, per=1) -> List[torch.Tensor]:
        out, off = [], 0
        for c in self.cams:
            sz = c.width * c.height * per
            out.append(t[off:off + sz].view(c.height, c.width, per) if per > 1 else t[off:off + sz].view(c.height, c.width))
            off += sz
        return out

    def pairs(self):
        n = int(self.num_pairs.item())
        return self.keys[:n], self.vals[:n]


def interpolate(key_times, t: float, key_pos: torch.Tensor, key_rot: torch.Tensor):
    """Assemble one frame's centres [n,3] and rotations [n,4] from keyframe tensors
    key_pos [K,n,3] and key_rot [K,n,4] (device, float32) at time t."""
    n = key_pos.shape[1]
    pos = torch.empty((n, 3), dtype=torch.float32, device=key_pos.device)
    rot = torch.empty((n, 4), dtype=torch.float32, device=key_pos.device)
    L.splat_interpolate(list(key_times), t, n, _ptr(key_pos), _ptr(key_rot), _ptr(pos), _ptr(rot), _stream())
    return pos, rot


def interpolate_backward(key_times, t: float, key_rot: torch.Tensor, d_pos, d_rot, d_key_pos=None, d_key_rot=None):
    """Add the keyframe gradients of one frame (d_key_* zero-initialised if not given)."""
    K, n = key_rot.shape[0], key_rot.shape[1]
    if d_key_pos is None:
        d_key_pos = torch.zeros((K, n, 3), dtype=torch.float32, device=key_rot.device)
    if d_key_rot is None:
        d_key_rot = torch.zeros((K, n, 4), dtype=torch.float32, device=key_rot.device)
    L.splat_interpolate_bwd(list(key_times), t, n, _ptr(key_rot), _ptr(d_pos), _ptr(d_rot), _ptr(d_key_pos),
                            _ptr(d_key_rot), _stream())
    return d_key_pos, d_key_rot

"""Seeded synthetic scenes for the rasterizer (inputs only).

This module draws primitives, cameras and upstream gradients with numpy's
PCG64 generator. It holds none of the rasterizer's arithmetic: no projection,
binning, compositing or gradient code lives here. Both the HIP path and the
CPU oracle consume what it returns, so every parity test and the benchmark
see identical inputs.

Workload shapes follow the pages' own workloads:
  * Pulsar (arXiv 2004.07484), section 4 and Table 2: one million spheres
    rendered at about 1000x1000 (here 1024x1024, the size quoted in section 1).
  * NuRec on page 2: Gaussian splats of driving scenes seen by several cameras
    and a lidar, with a long tail of uneven per-tile work.
Values the pages leave open (camera placement, focal lengths, distributions)
are fixed here once and documented alongside each config.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PRIM_GAUSS2D = 0
PRIM_GAUSS3D = 1
PRIM_SPHERE = 2

CAM_PINHOLE = 0
CAM_SPHERICAL = 1
CAM_ORTHO = 2          # orthographic (spheres only): u = fx x + cx, v = fy y + cy


def _f32(x) -> float:
    return float(np.float32(x))


@dataclass
class Camera:
    """World-to-sensor camera: q = R @ x + t (R row-major, float32 values)."""
    kind: int
    width: int
    height: int
    R: np.ndarray                 # (3, 3) float32
    t: np.ndarray                 # (3,) float32
    fx: float = 0.0
    fy: float = 0.0
    cx: float = 0.0
    cy: float = 0.0
    el_min_deg: float = 0.0
    el_max_deg: float = 0.0
    znear: float = 0.2
    zfar: float = 1000.0

    def __post_init__(self):
        self.R = np.asarray(self.R, dtype=np.float32).reshape(3, 3)
        self.t = np.asarray(self.t, dtype=np.float32).reshape(3)
        for k in ("fx", "fy", "cx", "cy", "el_min_deg", "el_max_deg", "znear", "zfar"):
            setattr(self, k, _f32(getattr(self, k)))

    @property
    def tiles_x(self) -> int:
        return (self.width + 15) // 16

    @property
    def tiles_y(self) -> int:
        return (self.height + 15) // 16


@dataclass
class Params:
    """Compositing constants (float32 values, as the library receives them)."""
    alpha_min: float = 1.0 / 255.0
    alpha_max: float = 0.99
    T_min: float = 1e-4
    gamma: float = 0.02
    bg_weight: float = 1.0
    tau: float = 1e-5
    top_k: int = 5
    background: Optional[np.ndarray] = None   # [channels] float32 or None (= 0)
    top_by_depth: int = 0      # spheres: 1 = record the top_k closest intersections, not the first top_k
    max_shift: int = 0         # spheres: 1 = weights relative to a per-pixel shift (needed for gamma < 1/88)
    serial_views: int = 0      # Gaussians: 1 = camera and spherical views on the caller's stream only

    def __post_init__(self):
        for k in ("alpha_min", "alpha_max", "T_min", "gamma", "bg_weight", "tau"):
            setattr(self, k, _f32(getattr(self, k)))
        if self.background is not None:
            self.background = np.asarray(self.background, dtype=np.float32)


@dataclass
class Scene:
    """SoA primitive arrays (float32, C-contiguous) plus cameras and params."""
    kind: int
    n: int
    channels: int
    pos: np.ndarray                      # GAUSS2D [n,2] pixel centres; else [n,3]
    scale: np.ndarray                    # GAUSS3D [n,3]; GAUSS2D sigma [n]; SPHERE radius [n]
    opacity: np.ndarray                  # [n]
    feat: Optional[np.ndarray]           # [n,channels] or None
    rot: Optional[np.ndarray] = None     # GAUSS3D [n,4] (w,x,y,z)
    depth: Optional[np.ndarray] = None   # GAUSS2D [n]
    cams: List[Camera] = field(default_factory=list)
    params: Params = field(default_factory=Params)
    name: str = ""

    def view_channels(self, v: int) -> int:
        """Image channels of view v: features for pinhole, (depth, opacity) for lidar."""
        return 2 if self.cams[v].kind == CAM_SPHERICAL else self.channels

    def pixels(self) -> int:
        return sum(c.width * c.height for c in self.cams)


def _c32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _unit_quats(rng, n):
    q = rng.standard_normal((n, 4))
    return q / np.linalg.norm(q, axis=1, keepdims=True)


def _rot_y(deg):
    a = math.radians(deg)
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]])


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def tiny_2d(seed=1, n=4096, width=128, height=128) -> Scene:
    """4,096 isotropic screen-space Gaussians on 128x128, 3 channels."""
    rng = np.random.default_rng(seed)
    centre = rng.uniform(0.0, [width, height], size=(n, 2))
    sigma = np.exp(rng.uniform(math.log(1.0), math.log(8.0), size=n))
    opac = rng.uniform(0.05, 0.95, size=n)
    depth = rng.uniform(1.0, 10.0, size=n)
    col = rng.uniform(0.0, 1.0, size=(n, 3))
    cam = Camera(CAM_PINHOLE, width, height, np.eye(3), np.zeros(3),
                 fx=1.0, fy=1.0, cx=0.0, cy=0.0, znear=0.0, zfar=1e30)
    return Scene(PRIM_GAUSS2D, n, 3, _c32(centre), _c32(sigma), _c32(opac), _c32(col),
                 depth=_c32(depth), cams=[cam], name="gauss2d_4k_128")


def gauss3d(seed=2, n=100_000, width=512, height=512) -> Scene:
    """100k anisotropic 3D Gaussians in [-5,5]^3, pinhole camera 10 units back."""
    rng = np.random.default_rng(seed)
    mu = rng.uniform(-5.0, 5.0, size=(n, 3))
    s = np.exp(rng.uniform(math.log(0.01), math.log(0.3), size=(n, 3)))
    q = _unit_quats(rng, n)
    o = 1.0 / (1.0 + np.exp(-rng.standard_normal(n)))
    col = rng.uniform(0.0, 1.0, size=(n, 3))
    cam = Camera(CAM_PINHOLE, width, height, np.eye(3), [0.0, 0.0, 10.0],
                 fx=500.0, fy=500.0, cx=width / 2, cy=height / 2, znear=0.2, zfar=1000.0)
    return Scene(PRIM_GAUSS3D, n, 3, _c32(mu), _c32(s), _c32(o), _c32(col), rot=_c32(q),
                 cams=[cam], name="gauss3d_100k_512")


def pulsar_spheres(seed=3, n=1_000_000, width=1024, height=1024) -> Scene:
    """1M spheres, uniform in image position and in depth U(2,20), 1024x1024.

    Radius log-uniform [0.005, 0.05], opacity U(0.1, 1), 3 feature channels.
    """
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, width, size=n)
    v = rng.uniform(0.0, height, size=n)
    z = rng.uniform(2.0, 20.0, size=n)
    r = np.exp(rng.uniform(math.log(0.005), math.log(0.05), size=n))
    o = rng.uniform(0.1, 1.0, size=n)
    f = rng.uniform(0.0, 1.0, size=(n, 3))
    fx = float(width)
    qc = np.stack([z * (u - width / 2) / fx, z * (v - height / 2) / fx, z], axis=1)
    R0 = _rot_y(10.0)
    t0 = np.array([0.1, -0.2, 0.3])
    p = (qc - t0) @ R0          # R0^T (q - t0), row-vector form
    cam = Camera(CAM_PINHOLE, width, height, R0, t0, fx=fx, fy=fx,
                 cx=width / 2, cy=height / 2, znear=1.0, zfar=21.0)
    return Scene(PRIM_SPHERE, n, 3, _c32(p), _c32(r), _c32(o), _c32(f), cams=[cam],
                 name="spheres_1m_1024")


def ortho_spheres(seed=21, n=300_000, width=600, height=450, px_per_unit=100.0) -> Scene:
    """Spheres under an orthographic camera (px_per_unit pixels per world unit):
    uniform in image position, depth U(2, 20), radius log-uniform [0.005, 0.05]
    (0.5 to 5 px), opacity U(0.1, 1), 3 feature channels."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, width, size=n)
    v = rng.uniform(0.0, height, size=n)
    z = rng.uniform(2.0, 20.0, size=n)
    r = np.exp(rng.uniform(math.log(0.005), math.log(0.05), size=n))
    o = rng.uniform(0.1, 1.0, size=n)
    f = rng.uniform(0.0, 1.0, size=(n, 3))
    cx, cy = width / 2 - 0.25, height / 2 + 0.5
    qc = np.stack([(u - cx) / px_per_unit, (v - cy) / px_per_unit, z], axis=1)
    R0 = _rot_y(10.0)
    t0 = np.array([0.1, -0.2, 0.3])
    p = (qc - t0) @ R0          # R0^T (q - t0), row-vector form
    cam = Camera(CAM_ORTHO, width, height, R0, t0, fx=px_per_unit, fy=0.95 * px_per_unit, cx=cx, cy=cy,
                 znear=1.0, zfar=21.0)
    return Scene(PRIM_SPHERE, n, 3, _c32(p), _c32(r), _c32(o), _c32(f), cams=[cam], name="spheres_ortho")


def _driving_geometry(rng, n):
    n_ground = int(round(0.6 * n))
    n_clust = int(round(0.3 * n))
    n_bg = n - n_ground - n_clust
    g = np.stack([rng.uniform(0, 100, n_ground), rng.uniform(-10, 10, n_ground),
                  np.zeros(n_ground)], axis=1)
    centres = np.stack([rng.uniform(0, 100, 50), rng.uniform(-10, 10, 50),
                        rng.uniform(0, 3, 50)], axis=1)
    assign = rng.integers(0, 50, n_clust)
    c = centres[assign] + rng.standard_normal((n_clust, 3))
    b = np.stack([rng.uniform(-100, 200, n_bg), rng.uniform(-100, 100, n_bg),
                  rng.uniform(0, 30, n_bg)], axis=1)
    mu = np.concatenate([g, c, b], axis=0)
    s = np.exp(rng.uniform(math.log(0.01), math.log(0.3), size=(n, 3)))
    q = _unit_quats(rng, n)
    o = 1.0 / (1.0 + np.exp(-rng.standard_normal(n)))
    return mu, s, q, o


def _look_camera(pos, fwd, right, down, **kw):
    R = np.stack([right, down, fwd], axis=0).astype(np.float64)
    t = -R @ np.asarray(pos, dtype=np.float64)
    return Camera(CAM_PINHOLE, R=R, t=t, **kw)


def driving(seed=4, n=2_000_000, width=1920, height=1080, channels=32) -> Scene:
    """2M Gaussians: 60% road strip, 30% in 50 clusters, 10% background.

    Camera 1.5 m above the road looking down +x; 32 feature channels.
    """
    rng = np.random.default_rng(seed)
    mu, s, q, o = _driving_geometry(rng, n)
    feat = rng.uniform(0.0, 1.0, size=(n, channels))
    cam = _look_camera([0.0, 0.0, 1.5], [1, 0, 0], [0, -1, 0], [0, 0, -1],
                       width=width, height=height, fx=1000.0, fy=1000.0,
                       cx=width / 2, cy=height / 2, znear=0.2, zfar=1000.0)
    return Scene(PRIM_GAUSS3D, n, channels, _c32(mu), _c32(s), _c32(o), _c32(feat),
                 rot=_c32(q), cams=[cam], name="driving_2m_1080p_c32")


def multisensor(seed=4, color_seed=5, n=2_000_000) -> Scene:
    """Driving geometry seen by 6 pinhole cameras (1280x720) and one lidar (64x2048)."""
    rng = np.random.default_rng(seed)
    mu, s, q, o = _driving_geometry(rng, n)
    col = np.random.default_rng(color_seed).uniform(0.0, 1.0, size=(n, 3))
    rig = np.array([50.0, 0.0, 1.5])
    cams = []
    for k in range(6):
        psi = math.radians(60.0 * k)
        fwd = np.array([math.cos(psi), math.sin(psi), 0.0])
        right = np.array([math.sin(psi), -math.cos(psi), 0.0])
        cams.append(_look_camera(rig, fwd, right, [0, 0, -1], width=1280, height=720,
                                 fx=640.0, fy=640.0, cx=640.0, cy=360.0,
                                 znear=0.2, zfar=1000.0))
    cams.append(Camera(CAM_SPHERICAL, 2048, 64, np.eye(3), -rig,
                       el_min_deg=-25.0, el_max_deg=15.0, znear=0.2, zfar=1000.0))
    return Scene(PRIM_GAUSS3D, n, 3, _c32(mu), _c32(s), _c32(o), _c32(col), rot=_c32(q),
                 cams=cams, name="multisensor_2m_6cam_lidar")


CONFIGS = {
    1: dict(make=tiny_2d, grad_seed=101),
    2: dict(make=gauss3d, grad_seed=102),
    3: dict(make=pulsar_spheres, grad_seed=103),
    4: dict(make=driving, grad_seed=104),
    5: dict(make=multisensor, grad_seed=(106, 105)),
}


def make_config(k: int, **kw) -> Scene:
    return CONFIGS[k]["make"](**kw)


def upstream_grads(scene: Scene, seed) -> List[np.ndarray]:
    """dL/d(image) ~ N(0,1) fp32, one [channels, H, W] array per view.

    For the multi-sensor rig, seed is (camera_seed, lidar_seed): camera views
    draw from the first generator in view order, the lidar view (depth,
    opacity) from the second.
    """
    if isinstance(seed, tuple):
        cam_rng = np.random.default_rng(seed[0])
        lid_rng = np.random.default_rng(seed[1])
    else:
        cam_rng = lid_rng = np.random.default_rng(seed)
    out = []
    for v, c in enumerate(scene.cams):
        rng = lid_rng if c.kind == CAM_SPHERICAL else cam_rng
        out.append(_c32(rng.standard_normal((scene.view_channels(v), c.height, c.width))))
    return out


def subset(scene: Scene, idx) -> Scene:
    """A scene holding only the primitives idx (same cameras and params)."""
    idx = np.asarray(idx)
    take = lambda a: None if a is None else _c32(a[idx])
    return Scene(scene.kind, len(idx), scene.channels, take(scene.pos), take(scene.scale),
                 take(scene.opacity), take(scene.feat), rot=take(scene.rot),
                 depth=take(scene.depth), cams=list(scene.cams), params=scene.params,
                 name=scene.name + f"_sub{len(idx)}")


def crop_camera(cam: Camera, width: int, height: int) -> Camera:
    """Same camera with a smaller sensor (principal point kept)."""
    return Camera(cam.kind, width, height, cam.R, cam.t, cam.fx, cam.fy, cam.cx, cam.cy,
                  cam.el_min_deg, cam.el_max_deg, cam.znear, cam.zfar)

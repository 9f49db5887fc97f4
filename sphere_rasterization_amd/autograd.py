"""PyTorch autograd over the four libsplat calls.

The scene and camera are tensors that feed autograd, and the reverse pass runs
only for what is asked for (Pulsar sec. 4 "Ease of Use": scene and camera as
PyTorch tensors; appendix B.2: gradients computed only when requested). This
module marshals arguments only: projection, binning, compositing and the
reverse pass all run in libsplat's kernels.

    rz = Rasterizer(scene)                       # buffers for one scene shape and set of views
    img = render(rz, pos=pos, scale=scale, opacity=opacity, feat=feat, cam_R=R, cam_t=t)
    loss = (img * target).sum(); loss.backward() # pos.grad, ..., R.grad filled

A Rasterizer holds the forward's buffers for its backward: run the backward of one
render before the next render on the same Rasterizer (another render in between
raises in the backward).
"""
from __future__ import annotations

from typing import Optional

import torch

from .raster import Rasterizer, make_cams

PRIM_NAMES = ("pos", "scale", "rot", "opacity", "feat")
CAM_NAMES = ("cam_R", "cam_t", "cam_K")


def _device_input(rz: Rasterizer, name: str, t: Optional[torch.Tensor]):
    if t is None:
        return rz.t.get(name)
    ref = rz.t.get(name)
    if ref is None or tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} does not match the scene's")
    if t.device != ref.device or t.dtype != torch.float32:
        raise ValueError(f"{name}: expected float32 on {ref.device}, got {t.dtype} on {t.device}")
    return t.detach().contiguous()


def _bind_cameras(rz: Rasterizer, cam_R, cam_t, cam_K):
    """Rebuild the host camera structs from camera tensors (values read on the host)."""
    if cam_R is None and cam_t is None and cam_K is None:
        return
    cams = []
    for v, c in enumerate(rz.cams):
        c2 = type(c)(**{k: getattr(c, k) for k in c.__dataclass_fields__})
        if cam_R is not None:
            c2.R = cam_R[v].detach().cpu().reshape(3, 3).numpy()
        if cam_t is not None:
            c2.t = cam_t[v].detach().cpu().reshape(3).numpy()
        if cam_K is not None:
            k = cam_K[v].detach().cpu().reshape(4).tolist()
            c2.fx, c2.fy, c2.cx, c2.cy = k
        c2.__post_init__()
        cams.append(c2)
    rz.c_cams = make_cams(cams)


class _Render(torch.autograd.Function):
    @staticmethod
    def forward(ctx, rz, pos, scale, rot, opacity, feat, cam_R, cam_t, cam_K):
        for name, t in zip(PRIM_NAMES, (pos, scale, rot, opacity, feat)):
            x = _device_input(rz, name, t)
            if x is not None:
                rz.t[name] = x
        rz._bind_prims()
        _bind_cameras(rz, cam_R, cam_t, cam_K)
        rz.forward(check=True)
        rz._autograd_version = getattr(rz, "_autograd_version", 0) + 1
        ctx.rz = rz
        ctx.version = rz._autograd_version
        ctx.cam_devices = [None if t is None else t.device for t in (cam_R, cam_t, cam_K)]
        out = rz.img.clone()
        return out

    @staticmethod
    def backward(ctx, dimg):
        rz = ctx.rz
        if getattr(rz, "_autograd_version", 0) != ctx.version:
            raise RuntimeError("the Rasterizer ran another render before this backward; run them in turn")
        need = ctx.needs_input_grad[1:]
        names = PRIM_NAMES + CAM_NAMES
        want = tuple(n for n, k in zip(names, need) if k)
        if not want:
            return (None,) * 9
        grads = rz.backward(dimg.contiguous(), want=want)
        out = [None]
        for i, n in enumerate(names):
            g = grads.get(n) if need[i] else None
            if g is not None and i >= len(PRIM_NAMES):
                dev = ctx.cam_devices[i - len(PRIM_NAMES)]
                g = g.reshape((rz.V, 3, 3) if n == "cam_R" else (rz.V, -1)).to(dev)
            out.append(g)
        return tuple(out)


def render(rz: Rasterizer, pos=None, scale=None, rot=None, opacity=None, feat=None, cam_R=None, cam_t=None,
           cam_K=None) -> torch.Tensor:
    """Forward render through libsplat with autograd. Primitive tensors (device,
    float32, the scene's shapes) replace the Rasterizer's; camera tensors (any
    device; cam_R [V, 3, 3], cam_t [V, 3], cam_K [V, 4] = fx, fy, cx, cy) replace
    its cameras' values. Returns the flat image (views concatenated, [Cv][H][W]
    each; Rasterizer.view_images splits it). Gradients flow to every argument
    that requires them (camera gradients: spheres only)."""
    return _Render.apply(rz, pos, scale, rot, opacity, feat, cam_R, cam_t, cam_K)

"""Element-wise comparison of the HIP path (through the C ABI) with the CPU oracle.

Tolerances: images 1e-4 absolute; gradients
    |d| <= 1e-3 (|ref| + 1e-2 rms(ref)) + 32 u mag,   u = 2^-24,
where mag is the oracle's sum of the magnitudes of the terms behind each
gradient: the GPU forms every term in single precision, so a sum of many
terms that cancel is accurate relative to mag, not to its own value (the extra
term is negligible wherever mag is close to |ref|); integer outputs (pair counts, sorted keys and values, tile ranges,
last index, top-K ids) bit-exact. Pixels the oracle flags as sitting within a
few ulps of a discrete decision (skip threshold, stop rule, clamp, sphere edge)
are left out of the image comparison and get zero upstream gradient on both
sides.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O

IMG_ATOL = 1e-4
GRAD_RTOL = 1e-3
GRAD_FLOOR = 1e-2
EPS_SUM = 32.0 * 2.0 ** -24


def _np(t):
    return t.detach().cpu().numpy()


def _log(msg):
    print(msg, flush=True)


def compare_binning(rz, orc):
    torch.cuda.synchronize()
    pr = orc.proj()
    np.testing.assert_array_equal(_np(rz.pair_counts).astype(np.int64), pr["ntiles"], err_msg="pair counts")
    okeys, ovals, oranges = orc.pairs()
    n = int(rz.num_pairs.item())
    assert n == len(okeys), f"pair count {n} vs oracle {len(okeys)}"
    assert int(rz.overflow.item()) == 0
    gk, gv = rz.pairs()
    np.testing.assert_array_equal(_np(gk).view(np.uint64), okeys, err_msg="sorted keys")
    np.testing.assert_array_equal(_np(gv).view(np.uint32), ovals, err_msg="sorted values")
    np.testing.assert_array_equal(_np(rz.tile_ranges).view(np.uint32).reshape(-1, 2), oranges, err_msg="tile ranges")
    return n


def gpu_pixel_outputs(rz, pix):
    """Gather the GPU forward outputs at global pixel ids pix (numpy int64)."""
    cams = rz.cams
    out_img = np.zeros((len(pix), max(rz.C, 2)))
    imgs = [_np(x) for x in rz.view_images()]
    offs = np.cumsum([0] + [c.width * c.height for c in cams])
    T = _np(rz.T_final) if rz.T_final is not None else None
    last = _np(rz.last) if rz.last is not None else None
    N = _np(rz.norm) if rz.norm is not None else None
    K = rz.scene.params.top_k
    view = np.searchsorted(offs, pix, side="right") - 1
    top = None
    if rz.topk is not None:
        # positions in the sorted pair list -> primitive ids
        pos = _np(rz.topk).reshape(-1, K)[pix].astype(np.int64)
        vals = _np(rz.vals).view(np.uint32).astype(np.int64)
        top = np.where(pos >= 0, vals[np.clip(pos, 0, None)] - (view * rz.n)[:, None], -1)
    for v, c in enumerate(cams):
        sel = np.nonzero(view == v)[0]
        lp = pix[sel] - offs[v]
        jj, ii = lp // c.width, lp % c.width
        Cv = imgs[v].shape[0]
        out_img[sel, :Cv] = imgs[v][:, jj, ii].T
    res = dict(img=out_img)
    if T is not None:
        res["T"] = T[pix]
    if last is not None:
        res["last"] = last[pix]
    if N is not None:
        res["N"], res["top"] = N[pix], top
    return res


def compare_forward(rz, orc, ref=None, pix=None, check_bins=True):
    """ref: oracle.render_views() (full) or None with pix = sampled global pixel ids."""
    torch.cuda.synchronize()
    stats = {}
    if check_bins:
        stats["pairs"] = compare_binning(rz, orc)
    if pix is None:
        pix = np.arange(orc.total_pix, dtype=np.int64)
    r = orc.render(pix)
    g = gpu_pixel_outputs(rz, pix)
    flags = r["flags"]
    ok = (flags & O.IMAGE_FLAGS) == 0
    stats["flag_frac"] = float(1.0 - ok.mean())
    # images: per view channel count
    cams = orc.cams
    offs = np.cumsum([0] + [c.width * c.height for c in cams])
    view = np.searchsorted(offs, pix, side="right") - 1
    err = 0.0
    for v, c in enumerate(cams):
        sel = np.nonzero((view == v) & ok)[0]
        Cv = 2 if c.kind == 1 else orc.C
        if len(sel):
            d = np.abs(g["img"][sel, :Cv] - r["img"][sel, :Cv])
            if c.kind == 1:
                # expected depth is in metres: relative above 1 m
                d[:, 0] /= np.maximum(1.0, np.abs(r["img"][sel, 0]))
            err = max(err, float(d.max()))
    stats["img_err"] = err
    assert err <= IMG_ATOL, f"image error {err:.3e} > {IMG_ATOL}"
    if "T" in g:
        # Gaussians: transmittance; max-shifted spheres: the shift m (tens to
        # hundreds: fp32 rounding of the log-weight, relative above 1)
        tmask = ok
        d = np.abs(g["T"][tmask] - r["T"][tmask]) / np.maximum(1.0, np.abs(r["T"][tmask]))
        terr = float(d.max()) if tmask.any() else 0.0
        stats["T_err"] = terr
        assert terr <= IMG_ATOL, f"T error {terr:.3e}"
    if "last" in g:
        bad = (g["last"][ok].astype(np.int64) != r["last"][ok])
        assert not bad.any(), f"last index differs at {bad.sum()} pixels"
    if "N" in g:
        rel = np.abs(g["N"][ok] - r["N"][ok]) / np.abs(r["N"][ok])
        stats["N_rel"] = float(rel.max()) if len(rel) else 0.0
        assert stats["N_rel"] <= 1e-4, f"norm rel error {stats['N_rel']:.3e}"
        # a near tie of entry depths (closest-K recording) leaves the recorded set open
        tok = ok & ((flags & O.FLAG_SPH_ZTIE) == 0)
        bad = (g["top"][tok] != r["top"][tok]).any(axis=1)
        assert not bad.any(), f"top-K ids differ at {bad.sum()} pixels"
    return stats


def masked_grads(orc, g_views, pix_flags=None):
    """Zero the upstream gradient at every flagged pixel (all flag kinds)."""
    full = orc.render()
    flags = full["flags"]
    out, off = [], 0
    for v, c in enumerate(orc.cams):
        hw = c.width * c.height
        f = flags[off:off + hw].reshape(c.height, c.width)
        gv = np.array(g_views[v], dtype=np.float32, copy=True)
        gv[:, f != 0] = 0.0
        out.append(gv)
        off += hw
    return out, float((flags != 0).mean())


def grad_check(name, got, ref, mag=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bound = GRAD_RTOL * (np.abs(ref) + GRAD_FLOOR * rms) + 1e-30
    if mag is not None:
        bound = bound + EPS_SUM * np.asarray(mag, np.float64).reshape(bound.shape)
    ratio = np.abs(got - ref) / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        k = int(np.argmax(ratio))
        raise AssertionError(f"{name}: worst ratio {worst:.2f} at flat {k}: got {got.reshape(-1)[k]:.6e} "
                             f"ref {ref.reshape(-1)[k]:.6e} (rms {rms:.3e}, {int((ratio > 1).sum())} over)")
    return worst


def compare_backward(rz, orc, ref, g_views, masked=None, names=None, view_groups=None, normalize=False):
    """Run both backward passes on the same (flag-masked) upstream gradient.

    view_groups: list of (view_begin, view_count) GPU calls accumulating into one
    set of gradients (default: one call over all views)."""
    if masked is None:
        masked, _ = masked_grads(orc, g_views)
    dimg = torch.from_numpy(np.concatenate([m.reshape(-1) for m in masked])).to(rz.device)
    if view_groups is None:
        grads = rz.backward(dimg, normalize=normalize)
    else:
        grads = None
        for b, c in view_groups:
            grads = rz.backward(dimg, view_begin=b, view_count=c, grads=grads, accumulate=grads is not None,
                                normalize=normalize)
    torch.cuda.synchronize()
    og = orc.backward(masked, with_mag=True, normalize=normalize)
    names = names or [k for k in ("pos", "scale", "rot", "opacity", "feat", "cam_R", "cam_t", "cam_K") if k in grads]
    worst = 0.0
    per = {}
    for k in names:
        got = _np(grads[k])
        refk = og[k]
        per[k] = grad_check(k, got, refk.reshape(got.shape), og["mag"][k])
        worst = max(worst, per[k])
    return dict(worst=worst, per=per)

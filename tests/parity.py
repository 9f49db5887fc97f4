"""Element-wise comparison of the HIP path (through the C ABI) with the CPU oracle.

Tolerances: images 1e-4 absolute; gradients
    |d| <= 1e-3 (|ref| + 1e-2 rms(ref)) + 32 u mag,   u = 2^-24,
where mag is the oracle's sum of the magnitudes of the terms behind each
gradient: the GPU forms every term in single precision, so a sum of many
terms that cancel is accurate relative to mag, not to its own value (the extra
term is negligible wherever mag is close to |ref|); integer outputs (pair
counts, sorted keys and values, tile ranges, last index, top-K ids) bit-exact.

Near ties. Where a pixel meets a decision that single-precision arithmetic may
take either way (an alpha at the skip threshold, a transmittance at the stop
threshold, a sphere bound at tau N, a sphere edge before the K-th hit), both
outcomes are correct. The oracle enumerates them (render_alts); the GPU's
output at such a pixel must match one of them to the same tolerances, and the
oracle's reverse pass then follows the outcome the GPU took, so the pixel's
gradients are compared too. Only pixels whose gradient is ambiguous from the
forward outputs (an opacity at the alpha clamp, a closest-K depth tie, more
ties than enumerated) get zero upstream gradient on both sides; their share is
asserted. At every other pixel the GPU's transmittance (Gaussians) or
normalisation (spheres) must stay within the oracle's rounding bound of an fp32
evaluation, the bound the tie windows are drawn from.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O

IMG_ATOL = 1e-4
GRAD_RTOL = 1e-3
GRAD_FLOOR = 1e-2
EPS_SUM = 32.0 * 2.0 ** -24
U32 = 2.0 ** -24
# flags whose pixels' upstream gradient is zeroed (ambiguous from the forward outputs)
GRAD_MASK_FLAGS = O.FLAG_CLAMP | O.FLAG_SPH_ZTIE | O.FLAG_UNRESOLVED


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


def _view_of(orc, pix):
    offs = np.cumsum([0] + [c.width * c.height for c in orc.cams])
    return np.searchsorted(offs, pix, side="right") - 1


def _img_err(orc, view, got, ref):
    """Per pixel max abs image error over the view's channels (lidar expected depth:
    relative above 1 m). got, ref: [..., Cm]; view broadcast over the leading axes."""
    d = np.zeros(got.shape[:-1])
    for v, c in enumerate(orc.cams):
        Cv = 2 if c.kind == 1 else orc.C
        sel = view == v
        if not sel.any():
            continue
        e = np.abs(got[..., :Cv] - ref[..., :Cv])
        if c.kind == 1:
            e[..., 0] = e[..., 0] / np.maximum(1.0, np.abs(ref[..., 0]))
        d = np.where(sel, e.max(axis=-1), d)
    return d


def _t_err(r_T, g_T):
    # Gaussians: transmittance; max-shifted spheres: the shift m (relative above 1)
    return np.abs(g_T - r_T) / np.maximum(1.0, np.abs(r_T))


def compare_forward(rz, orc, ref=None, pix=None, check_bins=True, max_flagged=1e-3, max_masked=1e-4):
    """Forward outputs at global pixel ids pix (default: all) against the oracle.

    Pixels with near-tie decisions are compared with every outcome the oracle
    enumerates and must match one; the matched outcome is kept (orc.branch_map,
    orc.set_branches) for the reverse pass. max_flagged bounds the share of
    pixels with near ties, max_masked the share whose gradient stays ambiguous."""
    torch.cuda.synchronize()
    stats = {}
    if check_bins:
        stats["pairs"] = compare_binning(rz, orc)
    full = pix is None
    if full:
        pix = np.arange(orc.total_pix, dtype=np.int64)
    r = orc.render(pix)
    g = gpu_pixel_outputs(rz, pix)
    flags = r["flags"]
    view = _view_of(orc, pix)
    sph = orc.kind == 2
    ms = sph and bool(getattr(orc.params, "max_shift", 0))
    dec = (flags & O.DECISION_FLAGS) != 0
    ok = ~dec
    stats["flag_frac"] = float(dec.mean())
    # default outcome where no decision is near a tie
    err = _img_err(orc, view[ok], g["img"][ok], r["img"][ok])
    stats["img_err"] = float(err.max()) if err.size else 0.0
    assert stats["img_err"] <= IMG_ATOL, f"image error {stats['img_err']:.3e} > {IMG_ATOL}"
    if "T" in g:
        d = _t_err(r["T"][ok], g["T"][ok])
        stats["T_err"] = float(d.max()) if d.size else 0.0
        assert stats["T_err"] <= IMG_ATOL, f"T error {stats['T_err']:.3e}"
        if not sph:
            # the rounding model the transmittance tie windows come from
            rel = np.abs(g["T"][ok] - r["T"][ok]) / np.maximum(r["T"][ok], 1e-300)
            bound = r["errb"][ok] * 1.0 + 2.0 * U32 + 1e-12
            stats["T_model"] = float((rel / bound).max()) if rel.size else 0.0
            assert stats["T_model"] <= 1.0, f"transmittance error beyond its rounding bound ({stats['T_model']:.2f})"
    if "last" in g:
        bad = (g["last"][ok].astype(np.int64) != r["last"][ok])
        assert not bad.any(), f"last index differs at {bad.sum()} pixels"
    if "N" in g:
        rel = np.abs(g["N"][ok] - r["N"][ok]) / np.abs(r["N"][ok])
        stats["N_rel"] = float(rel.max()) if len(rel) else 0.0
        assert stats["N_rel"] <= 1e-4, f"norm rel error {stats['N_rel']:.3e}"
        if not ms:
            bound = r["errb"][ok] + 2.0 * U32
            stats["N_model"] = float((rel / bound).max()) if rel.size else 0.0
            assert stats["N_model"] <= 1.0, f"normalisation error beyond its rounding bound ({stats['N_model']:.2f})"
        # a near tie of entry depths (closest-K recording) leaves the recorded set open
        tok = ok & ((flags & O.FLAG_SPH_ZTIE) == 0)
        bad = (g["top"][tok] != r["top"][tok]).any(axis=1)
        assert not bad.any(), f"top-K ids differ at {bad.sum()} pixels"
    # near ties: the GPU must match one of the enumerated outcomes
    chosen = np.zeros(len(pix), np.int32)
    unres = (flags & O.FLAG_UNRESOLVED) != 0
    idx = np.nonzero(dec)[0]
    stats["alt_taken"] = 0
    if len(idx):
        a = orc.render_alts(pix[idx])
        NA = a["mask"].shape[1]
        valid = np.arange(NA)[None, :] < a["nalt"][:, None]
        vv = np.broadcast_to(view[idx][:, None], valid.shape)
        e_img = _img_err(orc, vv, np.broadcast_to(g["img"][idx][:, None, :], a["img"].shape), a["img"])
        good = valid & (e_img <= IMG_ATOL)
        score = e_img.copy()
        if "T" in g:
            et = _t_err(a["T"], g["T"][idx][:, None])
            good &= et <= IMG_ATOL
            if not sph:
                score = score + np.abs(a["T"] - g["T"][idx][:, None]) / np.maximum(a["T"], 1e-300)
        if "last" in g:
            good &= a["last"] == g["last"][idx].astype(np.int64)[:, None]
        if "N" in g:
            en = np.abs(a["N"] - g["N"][idx][:, None]) / np.where(valid, np.abs(a["N"]), 1.0)
            good &= en <= 1e-4
            score = score + en
            zt = (flags[idx] & O.FLAG_SPH_ZTIE) != 0
            good &= zt[:, None] | (a["top"] == g["top"][idx][:, None, :]).all(axis=2)
        hit = good.any(axis=1)
        if not hit.all():
            k = int(np.nonzero(~hit)[0][0])
            raise AssertionError(f"{int((~hit).sum())} near-tie pixels match none of their outcomes "
                                 f"(first: pixel {int(pix[idx[k]])}, flags {int(flags[idx[k]])})")
        best = np.argmin(np.where(good, score, np.inf), axis=1)
        chosen[idx] = a["mask"][np.arange(len(idx)), best]
        unres[idx] |= a["unresolved"]
        stats["alt_taken"] = int((chosen[idx] != 0).sum())
    # the reverse pass: matched outcomes followed, ambiguous gradients masked
    masked = unres | ((flags & GRAD_MASK_FLAGS) != 0)
    stats["masked_frac"] = float(masked.mean())
    if full:
        # a sampled comparison leaves the other pixels' outcomes unknown: then
        # masked_grads falls back to masking every pixel with a near tie
        branch = np.where(masked, -1, chosen).astype(np.int32)
        orc.branch_map = branch
        orc.set_branches(np.maximum(branch, 0))
    assert stats["flag_frac"] <= max_flagged, f"near-tie share {stats['flag_frac']:.2e} > {max_flagged:.1e}"
    assert stats["masked_frac"] <= max_masked, f"masked share {stats['masked_frac']:.2e} > {max_masked:.1e}"
    return stats


def _all_flags(orc):
    return orc.render()["flags"]


def masked_grads(orc, g_views, pix_flags=None):
    """Zero the upstream gradient where the oracle's reverse pass cannot follow the
    GPU's outcome: the pixels compare_forward marked (orc.branch_map < 0), or, if
    it did not run, every pixel with a near tie."""
    bm = getattr(orc, "branch_map", None)
    if bm is None:
        bm = np.where(_all_flags(orc) != 0, -1, 0)
        orc.set_branches(None)
    out, off = [], 0
    for v, c in enumerate(orc.cams):
        hw = c.width * c.height
        f = bm[off:off + hw].reshape(c.height, c.width)
        gv = np.array(g_views[v], dtype=np.float32, copy=True)
        gv[:, f < 0] = 0.0
        out.append(gv)
        off += hw
    return out, float((bm < 0).mean())


def grad_check(name, got, ref, mag=None, info=None):
    """Elementwise gradient check; returns the worst ratio |d| / bound. info (a
    dict, optional) receives the audit of the summation term: the worst ratio
    against the bound without it and how many elements pass only with it."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    base = GRAD_RTOL * (np.abs(ref) + GRAD_FLOOR * rms) + 1e-30
    bound = base
    if mag is not None:
        bound = base + EPS_SUM * np.asarray(mag, np.float64).reshape(base.shape)
    diff = np.abs(got - ref)
    ratio = diff / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    if info is not None:
        r0 = diff / base
        info[name] = dict(worst=worst, worst_nomag=float(r0.max()) if r0.size else 0.0,
                          need_mag=int(((r0 > 1.0) & (ratio <= 1.0)).sum()), n=int(ref.size))
    if worst > 1.0:
        k = int(np.argmax(ratio))
        raise AssertionError(f"{name}: worst ratio {worst:.2f} at flat {k}: got {got.reshape(-1)[k]:.6e} "
                             f"ref {ref.reshape(-1)[k]:.6e} (rms {rms:.3e}, {int((ratio > 1).sum())} over)")
    return worst


def compare_backward(rz, orc, ref, g_views, masked=None, names=None, view_groups=None, normalize=False,
                     bwd_kw=None):
    """Run both backward passes on the same (flag-masked) upstream gradient.

    view_groups: list of (view_begin, view_count) GPU calls accumulating into one
    set of gradients (default: one call over all views)."""
    if masked is None:
        masked, _ = masked_grads(orc, g_views)
    dimg = torch.from_numpy(np.concatenate([m.reshape(-1) for m in masked])).to(rz.device)
    kw = dict(bwd_kw or {})
    if view_groups is None:
        grads = rz.backward(dimg, normalize=normalize, **kw)
    else:
        grads = None
        for b, c in view_groups:
            grads = rz.backward(dimg, view_begin=b, view_count=c, grads=grads, accumulate=grads is not None,
                                normalize=normalize, **kw)
    torch.cuda.synchronize()
    og = orc.backward(masked, with_mag=True, normalize=normalize)
    names = names or [k for k in ("pos", "scale", "rot", "opacity", "feat", "cam_R", "cam_t", "cam_K") if k in grads]
    worst = 0.0
    per, audit = {}, {}
    for k in names:
        got = _np(grads[k])
        refk = og[k]
        per[k] = grad_check(k, got, refk.reshape(got.shape), og["mag"][k], info=audit)
        worst = max(worst, per[k])
    return dict(worst=worst, per=per, audit=audit)

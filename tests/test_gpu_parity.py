"""GPU parity: the HIP path through the C ABI against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sphere_rasterization_amd import scenes as S
from tests import oracle_scenes as TS
from tests.parity import compare_backward, compare_binning, compare_forward, masked_grads

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _rz(scene, **kw):
    from sphere_rasterization_amd.raster import Rasterizer
    return Rasterizer(scene, device="cuda", **kw)


def _run(scene, grad_seed, name, check_grads=True, view_groups=None, normalize=False, fwd_kw=None, bwd_kw=None):
    _log(f"[case] {name}: n={scene.n} views={len(scene.cams)} kind={scene.kind}")
    rz = _rz(scene)
    rz.forward()
    orc = O.Oracle(scene)
    st = compare_forward(rz, orc, **(fwd_kw or {}))
    _log(f"  fwd ok pairs={st.get('pairs')} img_err={st['img_err']:.2e} near-tie={st['flag_frac']:.2e} "
         f"other-outcome={st['alt_taken']} grad-masked={st['masked_frac']:.2e} "
         f"T_model={st.get('T_model', 0):.2f} N_model={st.get('N_model', 0):.2f}")
    if check_grads:
        g = S.upstream_grads(scene, grad_seed)
        bw = compare_backward(rz, orc, None, g, view_groups=view_groups, normalize=normalize, bwd_kw=bwd_kw)
        _log(f"  bwd ok worst={bw['worst']:.3f} " + " ".join(f"{k}={v:.2f}" for k, v in bw["per"].items()))
        _log("  sum-term audit: " + " ".join(f"{k}:{a['worst_nomag']:.2f}/{a['need_mag']}of{a['n']}"
                                             for k, a in bw["audit"].items()))
    return rz, orc


def test_config1_tiny_2d_full():
    _run(S.tiny_2d(), 101, "gauss2d 4096 @128x128")


def test_config2_gauss3d_full():
    _run(S.gauss3d(), 102, "gauss3d 100k @512x512")


def test_config3_spheres_full():
    _run(S.pulsar_spheres(), 103, "spheres 1M @1024x1024")


def test_ragged_spheres():
    sc = S.pulsar_spheres(seed=13, n=150_000, width=1000, height=600)
    sc.cams = [S.Camera(S.CAM_PINHOLE, 1000, 600, sc.cams[0].R, sc.cams[0].t, fx=1024.0, fy=1000.0,
                        cx=480.3, cy=310.7, znear=1.0, zfar=21.0)]
    _run(sc, 7, "spheres 150k @1000x600 ragged")


def test_large_spheres():
    """Spheres of up to ~200 px radius in front of a dense field: a recorded
    sphere's row then takes the sums of hundreds of 8x8 quadrants (the reverse
    pass accumulates fp32 rows), and the pixels see long tile lists."""
    sc = S.pulsar_spheres(seed=71, n=40_000, width=640, height=480)
    rng = np.random.default_rng(72)
    cam = sc.cams[0]
    big = rng.random(sc.n) < 0.01
    z = np.where(big, rng.uniform(2.0, 4.0, sc.n), rng.uniform(2.0, 20.0, sc.n))
    u, v = rng.uniform(0, 640, sc.n), rng.uniform(0, 480, sc.n)
    qs = np.stack([z * (u - cam.cx) / cam.fx, z * (v - cam.cy) / cam.fy, z], 1)
    R, t = cam.R.astype(np.float64), cam.t.astype(np.float64)
    sc.pos = np.ascontiguousarray(((qs - t) @ R).astype(np.float32))
    r = np.where(big, np.exp(rng.uniform(np.log(0.1), np.log(0.6), sc.n)), sc.scale.astype(np.float64))
    sc.scale = np.ascontiguousarray(r.astype(np.float32))
    _run(sc, 73, "spheres 40k @640x480 with 1% of radius 0.1-0.6")


def test_spheres_behind_the_far_plane():
    """Depths U(2, 30) against zfar = 21: spheres whose fp32 front depth is not
    below zfar are culled on both sides (beyond it the stop bound would not hold),
    those straddling it are drawn; forward and reverse pass."""
    sc = S.pulsar_spheres(seed=61, n=120_000, width=320, height=240)
    rng = np.random.default_rng(62)
    cam = sc.cams[0]
    z = rng.uniform(2.0, 30.0, sc.n)
    u, v = rng.uniform(0, 320, sc.n), rng.uniform(0, 240, sc.n)
    qs = np.stack([z * (u - cam.cx) / cam.fx, z * (v - cam.cy) / cam.fy, z], 1)
    R, t = cam.R.astype(np.float64), cam.t.astype(np.float64)
    sc.pos = np.ascontiguousarray(((qs - t) @ R).astype(np.float32))
    _run(sc, 63, "spheres 120k @320x240 depths beyond zfar")


def test_sphere_direct_atomics():
    """The reverse pass's lane-by-lane atomics for entries few lanes recorded
    (atomic_direct_max, the DISTWAR-style split) give the oracle's gradients, with
    thresholds that route a small and a large share of the entries that way."""
    sc = S.pulsar_spheres(seed=64, n=150_000, width=400, height=300)
    for k in (2, 16):
        _run(sc, 65, f"spheres 150k @400x300, direct atomics up to {k} lanes", bwd_kw=dict(atomic_direct_max=k))


def test_sphere_channel_counts():
    """Sphere features of one and four channels (carried in the draw records) and of six
    channels (gathered from the feature array by the compositors), each against the
    oracle, forward and reverse pass."""
    base = S.pulsar_spheres(seed=37, n=40_000, width=200, height=150)
    rng = np.random.default_rng(38)
    for ch in (1, 4, 6):
        feat = np.ascontiguousarray(rng.uniform(0.0, 1.0, size=(base.n, ch)).astype(np.float32))
        sc = S.Scene(S.PRIM_SPHERE, base.n, ch, base.pos, base.scale, base.opacity, feat, cams=base.cams,
                     params=base.params)
        _run(sc, 40 + ch, f"spheres 40k @200x150, {ch} channels")


def test_gauss_channel_counts_few_tiles():
    """3D Gaussians with one, two and four feature channels on an image of 160
    tiles, where the camera compositors take the split walk (four waves per
    quadrant list, parts chained per pixel; below the chip's compute-unit count),
    and with five channels, which stays on the one-wave-per-quadrant kernels;
    each against the oracle, forward and reverse pass."""
    base = S.gauss3d(seed=44, n=20_000, width=256, height=160)
    rng = np.random.default_rng(45)
    for ch in (1, 2, 4, 5):
        feat = np.ascontiguousarray(rng.uniform(0.0, 1.0, size=(base.n, ch)).astype(np.float32))
        sc = S.Scene(S.PRIM_GAUSS3D, base.n, ch, base.pos, base.scale, base.opacity, feat, rot=base.rot,
                     cams=base.cams, params=base.params)
        _run(sc, 50 + ch, f"gauss3d 20k @256x160, {ch} channels")


def test_orthographic_spheres():
    # parallel projection: 300k spheres on 600x450 (ragged tiles), intrinsics gradients included
    _run(S.ortho_spheres(), 9, "spheres 300k @600x450 orthographic")


def test_normalised_sphere_gradients():
    # Pulsar's gradient normalisation (per-sphere averaging, camera over area and 1e-3)
    _run(S.pulsar_spheres(seed=23, n=200_000, width=640, height=480), 10, "spheres 200k @640x480 normalised",
         normalize=True)
    _run(S.ortho_spheres(seed=24, n=150_000), 11, "spheres 150k @600x450 orthographic normalised",
         normalize=True)


def test_closest_five_spheres():
    # each pixel records the five contributing spheres its ray enters first
    sc = S.pulsar_spheres(seed=25, n=300_000, width=640, height=480)
    sc.params = S.Params(top_by_depth=1)
    _run(sc, 12, "spheres 300k @640x480 closest five")
    so = S.ortho_spheres(seed=26, n=150_000)
    so.params = S.Params(top_by_depth=1)
    _run(so, 13, "spheres 150k @600x450 orthographic closest five")


def test_parameter_assembly():
    """Keyframe interpolation of 2M primitives (config-4 scale, ragged n) against
    the float64 oracle at times before, on, between and after the keyframes, and
    its reverse pass."""
    from oracle import assemble as A
    from sphere_rasterization_amd.raster import interpolate, interpolate_backward
    rng = np.random.default_rng(51)
    K, n = 4, 2_000_003
    times = np.cumsum(rng.uniform(0.05, 0.2, K)).astype(np.float32)
    kp = (rng.standard_normal((K, n, 3)) * 10).astype(np.float32)
    kr = rng.standard_normal((K, n, 4)).astype(np.float32)
    kp_d, kr_d = torch.from_numpy(kp).cuda(), torch.from_numpy(kr).cuda()
    u = 2.0 ** -24
    ts = [times[0] - 1, times[0], 0.5 * (times[1] + times[2]), times[2] + 0.3 * (times[3] - times[2]), times[3],
          times[3] + 1]
    for t in ts:
        t32 = float(np.float32(t))
        _log(f"[case] assemble n={n} K={K} t={t32:.6f}")
        pos, rot = interpolate(times, t32, kp_d, kr_d)
        torch.cuda.synchronize()
        rp, rq = A.interpolate(times, t32, kp, kr)
        k, k1, w = A.bracket(times, t32)
        # fp32 blend: a few roundings of the two terms and of w (and of 1 - w)
        mp = np.abs(kp[k]) + np.abs(kp[k1])
        mq = np.abs(kr[k]) + np.abs(kr[k1])
        assert (np.abs(pos.cpu().numpy() - rp) <= 4 * u * mp + 1e-30).all()
        tie = A.sign_ties(times, t32, kr)
        dq = np.abs(rot.cpu().numpy() - rq)[~tie]
        assert (dq <= 4 * u * mq[~tie] + 1e-30).all(), float((dq / (mq[~tie] + 1e-30)).max())
    # one keyframe, and no primitives: the single frame, and nothing to do
    p1, q1 = interpolate(times[:1], float(times[0]) + 0.5, kp_d[:1, :1000], kr_d[:1, :1000])
    torch.cuda.synchronize()
    assert torch.equal(p1, kp_d[0, :1000]) and torch.equal(q1, kr_d[0, :1000])
    p0, q0 = interpolate(times, float(times[1]), kp_d[:, :0], kr_d[:, :0])
    assert p0.shape == (0, 3) and q0.shape == (0, 4)
    # reverse pass at an interior time
    t32 = float(np.float32(ts[3]))
    gp = rng.standard_normal((n, 3)).astype(np.float32)
    gq = rng.standard_normal((n, 4)).astype(np.float32)
    dkp, dkq = interpolate_backward(times, t32, kr_d, torch.from_numpy(gp).cuda(), torch.from_numpy(gq).cuda())
    torch.cuda.synchronize()
    rkp, rkq = A.interpolate_backward(times, t32, kr, gp, gq)
    tie = A.sign_ties(times, t32, kr)
    for got, ref, g in ((dkp.cpu().numpy(), rkp, gp), (dkq.cpu().numpy(), rkq, gq)):
        d = np.abs(got - ref)
        bound = 3 * u * np.abs(g)[None] + 1e-30
        if g is gq:
            d, bound = d[:, ~tie], bound[:, ~tie]
        assert (d <= bound).all()
    _log("  assemble ok")


def test_max_shifted_spheres():
    # gamma = 1/200: unshifted weights exp(o zhat / gamma) would overflow fp32
    sc = S.pulsar_spheres(seed=27, n=200_000, width=640, height=480)
    sc.params = S.Params(gamma=0.005, max_shift=1)
    _run(sc, 14, "spheres 200k @640x480 gamma 1/200 max-shifted")
    s2 = S.pulsar_spheres(seed=28, n=150_000, width=512, height=384)
    s2.params = S.Params(max_shift=1, top_by_depth=1)
    _run(s2, 15, "spheres 150k @512x384 max-shifted, closest five")


def test_ragged_gauss3d():
    sc = S.gauss3d(seed=12, n=30_000, width=500, height=300)
    _run(sc, 8, "gauss3d 30k @500x300 ragged")


def test_sort_extreme_depths():
    """Depth keys over the whole positive fp32 range: denormal depths (down to
    1e-44), depths near the largest float, and many exact ties (broken by the
    record index). The segment sort compares the (depth bits, record) words in
    fp64 min/max and 64-bit integer compares, which order alike only for these
    non-negative bit patterns; both the one-wave path (short tiles) and the
    long-segment path must give the oracle's order bit for bit."""
    for n, seed in ((3000, 41), (20000, 42)):
        sc = S.tiny_2d(seed=seed, n=n)
        rng = np.random.default_rng(seed + 100)
        d = np.exp(rng.uniform(np.log(1e-44), np.log(3e38), size=n))
        ties = rng.random(n) < 0.2
        d[ties] = rng.choice(np.array([1e-44, 3e-39, 1.0, 2.5e38], dtype=np.float64), size=int(ties.sum()))
        sc.depth = np.ascontiguousarray(d.astype(np.float32))
        assert (sc.depth > 0).all() and np.isfinite(sc.depth).all()
        _log(f"[case] gauss2d {n} @128x128 extreme depths")
        rz = _rz(sc)
        rz.forward()
        orc = O.Oracle(sc)
        npairs = compare_binning(rz, orc)
        r = rz.tile_ranges.cpu().numpy().view(np.uint32).reshape(-1, 2).astype(np.int64)
        _log(f"  binning ok pairs={npairs} longest tile={int((r[:, 1] - r[:, 0]).max())}")
        orc.close()


def test_long_tile_lists():
    """Thousands of pairs per tile: the segments take the long-segment sort."""
    sc = S.gauss3d(seed=15, n=400_000, width=128, height=96)
    _run(sc, 9, "gauss3d 400k @128x96 long tile lists")


def test_view_beyond_lds_counters():
    """A view with more tiles than the LDS counters hold takes the global-counter binning."""
    sc = S.gauss3d(seed=16, n=20_000, width=2304, height=2048)
    _run(sc, 10, "gauss3d 20k @2304x2048 (18432 tiles)")


def test_tile_scan_beyond_one_workgroup():
    """More than 65536 tiles (the three-kernel tile scan, long-segment work lists
    filled with atomics) and a cluster of large Gaussians whose tiles hold up to
    12k pairs (the MSD split ahead of the LDS merge sort). Binning is compared in
    full, the image on a pixel sample around and away from the cluster, and the
    gradients of a reverse pass whose upstream gradient lives on that sample."""
    sc = S.gauss3d(seed=18, n=120_000, width=4160, height=4128)
    c = sc.cams[0]
    sc.cams = [S.Camera(S.CAM_PINHOLE, 4160, 4128, c.R, c.t, fx=1500.0, fy=1500.0, cx=2000.0, cy=2100.0,
                        znear=0.2, zfar=1000.0)]
    rng = np.random.default_rng(5)
    k = 12_000
    sc.pos[:k] = rng.normal(0.0, 0.4, size=(k, 3)).astype(np.float32)
    sc.scale[:k] = np.float32(0.25)
    _log(f"[case] gauss3d 120k @4160x4128 clustered (67080 tiles)")
    rz = _rz(sc)
    rz.forward()
    orc = O.Oracle(sc)
    prng = np.random.default_rng(6)
    pix = np.concatenate([prng.choice(4160 * 4128, 20_000, replace=False),
                          (2100 + prng.integers(-300, 300, 20_000)) * 4160 + 2000 + prng.integers(-300, 300, 20_000)])
    pix = np.unique(pix).astype(np.int64)
    st = compare_forward(rz, orc, pix=pix)
    _log(f"  fwd ok pairs={st.get('pairs')} img_err={st['img_err']:.2e} flagged={st['flag_frac']:.2e}")
    # reverse pass with the upstream gradient on the sampled pixels only (those
    # without a near tie), so the oracle's reverse pass composites just those
    flags = orc.render(pix)["flags"]
    keep = pix[flags == 0]
    g = np.zeros((sc.channels, 4128, 4160), np.float32)
    g.reshape(sc.channels, -1)[:, keep] = np.random.default_rng(7).standard_normal((sc.channels, len(keep)))
    orc.set_branches(None)
    dimg = torch.from_numpy(g.reshape(-1)).cuda()
    grads = rz.backward(dimg)
    torch.cuda.synchronize()
    og = orc.backward([g], with_mag=True)
    from tests.parity import grad_check
    for k in ("pos", "scale", "rot", "opacity", "feat"):
        w = grad_check(k, grads[k].cpu().numpy(), og[k].reshape(grads[k].shape), og["mag"][k].reshape(grads[k].shape))
        _log(f"  bwd {k} worst={w:.3f} (upstream gradient on {len(keep)} pixels)")


def test_multiview_with_lidar():
    """Two pinhole views and a spherical view in one call; camera and lidar backward
    run as separate calls that accumulate into the same gradients, then as one call."""
    sc = S.gauss3d(seed=14, n=20_000)
    R1 = TS.rotation(np.random.default_rng(1))
    sc.cams = [sc.cams[0],
               S.Camera(S.CAM_PINHOLE, 320, 200, R1, [0.2, -0.1, 9.0], fx=300.0, fy=310.0, cx=160.0, cy=100.0,
                        znear=0.2, zfar=100.0),
               TS.lidar(512, 64, t=[0.0, 0.0, 0.0])]
    _log("[case] multiview: 2 pinhole + 1 spherical")
    rz = _rz(sc)
    rz.forward()
    orc = O.Oracle(sc)
    st = compare_forward(rz, orc)
    _log(f"  fwd ok img_err={st['img_err']:.2e} flagged={st['flag_frac']:.2e}")
    g = [np.random.default_rng(40 + v).standard_normal((sc.view_channels(v), c.height, c.width)).astype(np.float32)
         for v, c in enumerate(sc.cams)]
    masked, _ = masked_grads(orc, g)
    dimg = torch.from_numpy(np.concatenate([m.reshape(-1) for m in masked])).cuda()
    grads = rz.backward(dimg, view_begin=0, view_count=2)
    rz.backward(dimg, view_begin=2, view_count=1, grads=grads, accumulate=True)
    torch.cuda.synchronize()
    og = orc.backward(masked, with_mag=True)
    from tests.parity import grad_check
    for k in ("pos", "scale", "rot", "opacity", "feat"):
        w = grad_check(k, grads[k].cpu().numpy(), og[k], og["mag"][k])
        _log(f"  {k} worst={w:.3f}")
    # one call over all three views: the camera views run beside the lidar view
    one = rz.backward(dimg)
    torch.cuda.synchronize()
    for k in ("pos", "scale", "rot", "opacity", "feat"):
        w = grad_check(k, one[k].cpu().numpy(), og[k], og["mag"][k])
        _log(f"  one call {k} worst={w:.3f}")


def test_lidar_half_turn_footprints():
    """Lidar view with Gaussians whose footprints wrap past half the panorama:
    list entries centred near the antipode of their tile, where the column wrap
    of each pixel's offset decides which image of the centre it sees (the
    kernels take the per-pixel wrap for those entries only). Forward and
    reverse pass against the oracle."""
    _run(TS.lidar_half_turn(), 62, "gauss3d 6400 lidar 256x32, footprints past half a turn")


def test_two_small_pinhole_views():
    """Two pinhole views of 48 and 24 tiles in one launch (the split camera
    walk across views: each tile finds its view and pixel offsets), forward
    and reverse pass against the oracle."""
    sc = S.gauss3d(seed=46, n=20_000, width=128, height=96)
    R1 = TS.rotation(np.random.default_rng(47))
    sc.cams = [sc.cams[0],
               S.Camera(S.CAM_PINHOLE, 96, 64, R1, [0.1, 0.2, 9.0], fx=120.0, fy=125.0, cx=48.0, cy=32.0,
                        znear=0.2, zfar=100.0)]
    _run(sc, 48, "gauss3d 20k, pinhole 128x96 + 96x64")


def test_multiview_serial_views():
    """splat_params.serial_views = 1 (every kernel on the caller's stream, no side
    stream): the same forward outputs bit for bit as the forked call, and gradients
    that agree with the oracle."""
    sc = S.gauss3d(seed=14, n=20_000)
    R1 = TS.rotation(np.random.default_rng(1))
    sc.cams = [sc.cams[0],
               S.Camera(S.CAM_PINHOLE, 320, 200, R1, [0.2, -0.1, 9.0], fx=300.0, fy=310.0, cx=160.0, cy=100.0,
                        znear=0.2, zfar=100.0),
               TS.lidar(512, 64, t=[0.0, 0.0, 0.0])]
    _log("[case] multiview, serial views")
    forked = _rz(sc)
    forked.forward()
    img_f, T_f, last_f = forked.img.clone(), forked.T_final.clone(), forked.last.clone()
    sc.params = S.Params(serial_views=1)
    rz = _rz(sc)
    rz.forward()
    torch.cuda.synchronize()
    assert torch.equal(rz.img, img_f) and torch.equal(rz.T_final, T_f) and torch.equal(rz.last, last_f)
    orc = O.Oracle(sc)
    compare_forward(rz, orc)
    g = [np.random.default_rng(40 + v).standard_normal((sc.view_channels(v), c.height, c.width)).astype(np.float32)
         for v, c in enumerate(sc.cams)]
    bw = compare_backward(rz, orc, None, g)
    _log(f"  bwd ok worst={bw['worst']:.3f}")


def test_autograd_render():
    """render() as a torch.autograd.Function: loss.backward() gives the oracle's
    gradients for the primitive tensors and the camera R, t that require them; an
    input that does not require grad gets none; a second render before the
    backward is refused. Spheres, then 3D Gaussians."""
    from sphere_rasterization_amd.autograd import render
    from tests.parity import grad_check
    sc = S.pulsar_spheres(seed=66, n=60_000, width=256, height=192)
    _log("[case] autograd: spheres 60k @256x192 with camera R, t")
    rz = _rz(sc)
    pos = rz.t["pos"].clone().requires_grad_(True)
    scale = rz.t["scale"].clone()                       # not asked for
    opacity = rz.t["opacity"].clone().requires_grad_(True)
    feat = rz.t["feat"].clone().requires_grad_(True)
    cam_R = torch.tensor(np.asarray(sc.cams[0].R, np.float32)).reshape(1, 3, 3).requires_grad_(True)
    cam_t = torch.tensor(np.asarray(sc.cams[0].t, np.float32)).reshape(1, 3).requires_grad_(True)
    img = render(rz, pos=pos, scale=scale, opacity=opacity, feat=feat, cam_R=cam_R, cam_t=cam_t)
    orc = O.Oracle(sc)
    compare_forward(rz, orc)
    masked, _ = masked_grads(orc, S.upstream_grads(sc, 67))
    gm = torch.from_numpy(np.concatenate([m.reshape(-1) for m in masked])).cuda()
    (img * gm).sum().backward()
    og = orc.backward(masked, with_mag=True)
    assert scale.grad is None
    for name, t in (("pos", pos), ("opacity", opacity), ("feat", feat)):
        w = grad_check(name, t.grad.cpu().numpy(), og[name].reshape(t.shape), og["mag"][name].reshape(t.shape))
        _log(f"  {name} worst={w:.3f}")
    for name, t in (("cam_R", cam_R), ("cam_t", cam_t)):
        assert t.grad is not None and t.grad.device.type == "cpu"
        w = grad_check(name, t.grad.numpy().reshape(-1), og[name].reshape(-1), og["mag"][name].reshape(-1))
        _log(f"  {name} worst={w:.3f}")
    # a render between a render and its backward leaves that backward nothing to use
    img1 = render(rz, pos=pos, opacity=opacity, feat=feat)
    render(rz, pos=pos, opacity=opacity, feat=feat)
    with pytest.raises(RuntimeError):
        img1.sum().backward()

    gs = S.gauss3d(seed=68, n=30_000, width=320, height=240)
    _log("[case] autograd: gauss3d 30k @320x240")
    rz = _rz(gs)
    ts = {k: rz.t[k].clone().requires_grad_(True) for k in ("pos", "scale", "rot", "opacity", "feat")}
    img = render(rz, **ts)
    orc = O.Oracle(gs)
    compare_forward(rz, orc)
    masked, _ = masked_grads(orc, S.upstream_grads(gs, 69))
    gm = torch.from_numpy(np.concatenate([m.reshape(-1) for m in masked])).cuda()
    (img * gm).sum().backward()
    og = orc.backward(masked, with_mag=True)
    for name, t in ts.items():
        w = grad_check(name, t.grad.cpu().numpy(), og[name].reshape(t.shape), og["mag"][name].reshape(t.shape))
        _log(f"  {name} worst={w:.3f}")


def test_spheres_two_views():
    """Spheres seen by two pinhole views: one backward call over both views
    (per-view camera reduction), and one call per view accumulating."""
    sc = S.pulsar_spheres(seed=17, n=60_000, width=256, height=192)
    c0 = sc.cams[0]
    R1 = S._rot_y(-12.0) @ np.asarray(c0.R)
    sc.cams = [c0, S.Camera(S.CAM_PINHOLE, 200, 160, R1, [0.4, 0.1, 0.5], fx=220.0, fy=230.0, cx=97.0, cy=83.0,
                            znear=1.0, zfar=21.0)]
    _log("[case] spheres, two views")
    rz = _rz(sc)
    rz.forward()
    orc = O.Oracle(sc)
    st = compare_forward(rz, orc)
    _log(f"  fwd ok img_err={st['img_err']:.2e} flagged={st['flag_frac']:.2e}")
    g = S.upstream_grads(sc, 31)
    bw = compare_backward(rz, orc, None, g)
    _log(f"  bwd (one call) worst={bw['worst']:.3f}")
    bw = compare_backward(rz, orc, None, g, view_groups=[(0, 1), (1, 1)])
    _log(f"  bwd (per view) worst={bw['worst']:.3f}")


def test_forward_clears_backward_sums():
    """A sphere forward handed the reverse pass's workspace clears the sums it
    accumulates into: with the workspace filled with NaN bytes before that forward,
    the reverse pass told so (sums_cleared) gives what a self-clearing reverse pass
    gave, for one view (camera R, t stored outright) and for two views (R, t zeroed
    and added); the reverse pass after it clears for itself again."""
    for views in (1, 2):
        sc = S.pulsar_spheres(seed=33, n=40_000, width=256, height=192)
        if views == 2:
            c0 = sc.cams[0]
            R1 = S._rot_y(8.0) @ np.asarray(c0.R)
            sc.cams = [c0, S.Camera(S.CAM_PINHOLE, 224, 176, R1, [0.2, -0.1, 0.3], fx=240.0, fy=236.0, cx=110.0,
                                    cy=90.0, znear=1.0, zfar=21.0)]
        _log(f"[case] forward-cleared reverse sums, {views} view(s)")
        rz = _rz(sc)
        rz.forward()
        assert not rz.sums_cleared                      # no workspace yet: the reverse pass clears
        dimg = torch.randn(rz.img.shape, generator=torch.Generator(device="cuda").manual_seed(7), device="cuda")
        want = ("pos", "scale", "opacity", "feat", "cam_R", "cam_t", "cam_K")
        ref = {k: v.clone() for k, v in rz.backward(dimg, want=want).items()}
        rz.bwd_ws.fill_(0xFF)                           # NaN in every fp64 sum
        rz.forward()
        assert rz.sums_cleared
        for rnd in range(2):                            # skipping the clearing, then clearing again
            got = rz.backward(dimg, want=want)
            torch.cuda.synchronize()
            assert not rz.sums_cleared
            for k in want:
                assert torch.isfinite(got[k]).all(), (views, rnd, k)
                torch.testing.assert_close(got[k], ref[k], rtol=1e-5, atol=1e-5 * float(ref[k].abs().max()) + 1e-12)


def test_sphere_overflow_after_clearing_forward():
    """A pair overflow makes the sphere forward write nothing, but its appended
    workgroups still clear the reverse pass's sums: the reverse pass told so then
    finds no stale sums of the step before, and every gradient is zero."""
    sc = S.pulsar_spheres(seed=35, n=20_000, width=128, height=96)
    _log("[case] sphere overflow after a clearing forward")
    rz = _rz(sc)
    rz.forward()
    dimg = torch.randn(rz.img.shape, generator=torch.Generator(device="cuda").manual_seed(9), device="cuda")
    want = ("pos", "scale", "opacity", "feat", "cam_R", "cam_t", "cam_K")
    g0 = rz.backward(dimg, want=want)                  # leaves non-zero sums in the workspace
    torch.cuda.synchronize()
    assert float(g0["pos"].abs().max()) > 0.0
    rz._alloc_pairs(100)
    rz.project()
    rz.bin_sort()
    rz.render_fwd()
    torch.cuda.synchronize()
    assert int(rz.overflow.item()) == 1 and rz.sums_cleared
    g = rz.backward(dimg, want=want)
    torch.cuda.synchronize()
    for k in want:
        assert torch.isfinite(g[k]).all() and float(g[k].abs().max()) == 0.0, k


def test_sphere_option_edges():
    """Option corners: closest-K with top_k 1 and 8; max-shift without early stop at
    gamma = 1/250; a pinhole and an orthographic view in one call with intrinsic
    gradients and normalisation (one call over both views)."""
    base = S.pulsar_spheres(seed=29, n=60_000, width=320, height=240)
    for k in (1, 8):
        sc = S.pulsar_spheres(seed=29, n=60_000, width=320, height=240)
        sc.params = S.Params(top_k=k, top_by_depth=1)
        _run(sc, 16 + k, f"spheres 60k @320x240 closest {k}")
    sc = S.pulsar_spheres(seed=30, n=60_000, width=320, height=240)
    sc.params = S.Params(gamma=0.004, tau=0.0, max_shift=1)
    _run(sc, 19, "spheres 60k @320x240 gamma 1/250 max-shifted, no early stop")
    sc = S.Scene(S.PRIM_SPHERE, base.n, 3, base.pos, base.scale, base.opacity, base.feat,
                 cams=[base.cams[0], S.Camera(S.CAM_ORTHO, 300, 220, base.cams[0].R, base.cams[0].t, fx=30.0,
                                              fy=28.0, cx=150.0, cy=110.0, znear=1.0, zfar=21.0)])
    _run(sc, 20, "spheres 60k: pinhole 320x240 + orthographic 300x220, normalised", normalize=True)


def test_all_culled_and_single():
    sc = TS.spheres([[0, 0, -5.0]], [0.5], [0.5], [[1, 0, 0]], [TS.pinhole(40, 30, 40.0, znear=1.0, zfar=21.0)])
    rz = _rz(sc)
    rz.forward()
    torch.cuda.synchronize()
    assert int(rz.num_pairs.item()) == 0
    assert float(rz.img.abs().max()) == 0.0
    assert torch.all(rz.norm == 1.0)
    # gamma = 1 keeps the single weight near 1; at gamma = 0.02 the colour saturates
    # (C = f to 1e-12) and every gradient falls below fp32 resolution
    sc1 = TS.spheres([[0.1, 0.05, 5.0]], [0.5], [0.7], [[0.2, 0.4, 0.6]], [TS.pinhole(40, 30, 40.0, znear=1.0, zfar=21.0)],
                     params=S.Params(gamma=1.0))
    _run(sc1, 3, "single sphere")
    sc2 = TS.scene2d([[20.3, 11.7]], [3.0], [0.8], [1.5], [[0.3, 0.9]], W=40, H=24)
    _run(sc2, 4, "single gaussian")


def test_empty_primitive_set():
    """No primitives: splat_project launches nothing, splat_bin_sort (the counting
    fallback with a zero record count) reports zero pairs, a clear overflow flag and
    empty ranges for every tile over pre-filled garbage, and the render calls reject
    n = 0 before any launch."""
    import ctypes as C
    from sphere_rasterization_amd import _lib as L
    from sphere_rasterization_amd.raster import make_cams, make_params
    _log("[case] empty primitive set: n=0, 1 view 128x96")
    sc = S.pulsar_spheres(n=10, width=128, height=96)
    cams = make_cams(sc.cams)
    prm, _ = make_params(sc.params, 3)
    pr = L.splat_prims()
    pr.kind, pr.n, pr.channels = S.PRIM_SPHERE, 0, 3
    lib = L.lib()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.splat_project(cams, 1, C.byref(pr), C.byref(prm), None, None, stream) == L.SPLAT_OK
    tiles = int(lib.splat_total_tiles(cams, 1))
    assert tiles == 8 * 6
    ranges = torch.full((tiles, 2), 7, dtype=torch.int32, device="cuda")
    num = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    of = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    ws_bytes = L.splat_sort_workspace_bytes(cams, 1, 0, 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    rc = lib.splat_bin_sort(cams, 1, 0, None, None, 0, None, None, ranges.data_ptr(), num.data_ptr(), of.data_ptr(),
                            ws.data_ptr(), ws_bytes, stream)
    assert rc == L.SPLAT_OK
    torch.cuda.synchronize()
    assert int(num.item()) == 0 and int(of.item()) == 0
    assert int(ranges.abs().sum().item()) == 0
    assert lib.splat_render_fwd(cams, 1, C.byref(pr), C.byref(prm), None, None, None, of.data_ptr(), None, None,
                                None, None, None, None, 0, stream) == L.SPLAT_ERR_INVALID_ARG


def test_overflow_then_regrow():
    sc = S.gauss3d(seed=5, n=20_000, width=256, height=256)
    _log("[case] overflow regrow")
    rz = _rz(sc, capacity=1000)
    rz.project()
    rz.bin_sort()
    torch.cuda.synchronize()
    need = int(rz.num_pairs.item())
    assert need > 1000 and int(rz.overflow.item()) == 1
    assert rz.ensure_capacity()
    rz.render_fwd()
    orc = O.Oracle(sc)
    compare_forward(rz, orc)


def test_forward_deterministic_and_null_grads():
    sc = S.pulsar_spheres(seed=21, n=50_000, width=256, height=256)
    rz = _rz(sc)
    a = rz.forward().clone()
    b = rz.forward().clone()
    assert torch.equal(a, b)
    dimg = torch.randn_like(rz.img)
    sentinel = torch.full((sc.n, 3), 7.0, device="cuda")
    grads = {"feat": torch.zeros(sc.n, 3, device="cuda"), "pos": sentinel.clone()}
    from sphere_rasterization_amd import _lib as L
    import ctypes as C
    g = L.splat_grads()
    g.feat = C.c_void_p(grads["feat"].data_ptr())
    rz.backward(dimg, grads={"feat": grads["feat"]})
    torch.cuda.synchronize()
    assert torch.equal(grads["pos"], sentinel)          # not requested: untouched
    g1 = rz.backward(dimg, want=("feat", "opacity"))
    g2 = rz.backward(dimg, want=("feat", "opacity"))
    torch.cuda.synchronize()
    # float atomics make the summation order (not the result) run-dependent
    from tests.parity import grad_check
    for k in g1:
        grad_check(k, g1[k].cpu().numpy(), g2[k].cpu().numpy())
    grad_check("feat", grads["feat"].cpu().numpy(), g1["feat"].cpu().numpy())


# The two largest workloads: full binning, image and gradient comparison (the
# oracle's reverse pass takes some tens of seconds on the host cores).
@pytest.mark.timeout(600)
def test_config4_driving_full():
    _run(S.driving(), S.CONFIGS[4]["grad_seed"], "gauss3d 2M @1920x1080 C=32")


@pytest.mark.timeout(600)
def test_config5_multisensor_full():
    # one backward call over the camera views and the lidar view, as timed
    _run(S.multisensor(), S.CONFIGS[5]["grad_seed"], "gauss3d 2M, 6 cameras 1280x720 + lidar 2048x64")


def test_graph_capture_replays():
    """One whole step (projection, binning, forward, reverse pass) captured in a HIP
    graph and replayed, with eager steps in between: every replay reproduces the
    eager outputs exactly. The path makes no host synchronisation or allocation, and
    the camera/lidar side-stream fork joins the capture."""
    sph = S.pulsar_spheres(seed=33, n=50_000, width=256, height=192)
    mv = S.gauss3d(seed=34, n=20_000)
    R1 = TS.rotation(np.random.default_rng(2))
    mv.cams = [mv.cams[0],
               S.Camera(S.CAM_PINHOLE, 320, 200, R1, [0.2, -0.1, 9.0], fx=300.0, fy=310.0, cx=160.0, cy=100.0,
                        znear=0.2, zfar=100.0),
               TS.lidar(512, 64, t=[0.0, 0.0, 0.0])]
    for name, sc in (("spheres", sph), ("2 pinhole + lidar", mv)):
        _log(f"[case] graph capture: {name}")
        rz = _rz(sc)
        rz.forward(check=True)
        dimg = torch.from_numpy(np.concatenate([g.reshape(-1) for g in S.upstream_grads(sc, 5)])).cuda()
        grads = rz.alloc_grads(("pos", "scale", "rot", "opacity", "feat", "cam_R", "cam_t"))

        def step():
            rz.project()
            rz.bin_sort()
            rz.render_fwd()
            rz.backward(dimg, grads=grads)

        for _ in range(2):
            step()
        torch.cuda.synchronize()
        ref_img = rz.img.clone()
        ref = {k: v.clone() for k, v in grads.items()}
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for r in range(3):
            rz.img.zero_()
            for v in grads.values():
                v.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(rz.img, ref_img), f"{name}: replay {r} image"
            for k in grads:
                # fp64 atomics sum in arrival order: equal to rounding of the fp32 outputs
                d = (grads[k] - ref[k]).abs().max().item()
                assert d <= 1e-5 * (ref[k].abs().max().item() + 1e-30), f"{name}: replay {r} {k} {d}"
            step()                                    # eager work between replays
            torch.cuda.synchronize()
        _log(f"  {name}: 3 replays ok")

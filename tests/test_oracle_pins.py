"""Pins of the CPU oracle against closed forms, invariants, brute force and
geometry computed independently of the oracle's own formulas (CPU only)."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from sphere_rasterization_amd import scenes as S
from tests import oracle_scenes as TS

A_MIN = float(np.float32(1 / 255))


def f64(x):
    return np.asarray(x, np.float32).astype(np.float64)


# ---------------------------------------------------------------- alpha path

def _closed_gauss2d(W, H, c, sig, o):
    ys, xs = np.mgrid[0:H, 0:W] + 0.5
    d2 = (xs - c[0]) ** 2 + (ys - c[1]) ** 2
    a = np.minimum(float(np.float32(0.99)), o * np.exp(-0.5 * d2 / sig ** 2))
    return np.where(a < A_MIN, 0.0, a)


def test_single_gaussian_closed_form():
    """One screen-space Gaussian: C = alpha*c with alpha = min(.99, o G), zero below 1/255."""
    c, sig, o, col = f64([13.3, 17.8]), f64(3.1), f64(0.7), f64([0.2, 0.5, 0.9])
    sc = TS.scene2d([c], [sig], [o], [2.0], [col])
    r = O.Oracle(sc).render_views()[0]
    a = _closed_gauss2d(32, 32, c, sig, o)
    np.testing.assert_allclose(r["img"], a[None] * col[:, None, None], atol=1e-13, rtol=0)
    np.testing.assert_allclose(r["T"], 1.0 - a, atol=1e-13, rtol=0)
    assert (r["ncontrib"] == (a > 0)).all()


def test_single_gaussian_clamps_at_099():
    c, sig, o = f64([10.5, 10.5]), f64(4.0), f64(1.0)
    sc = TS.scene2d([c], [sig], [o], [2.0], [[1.0]])
    r = O.Oracle(sc).render_views()[0]
    assert r["img"][0, 10, 10] == float(np.float32(0.99))
    np.testing.assert_allclose(r["img"][0], _closed_gauss2d(32, 32, c, sig, o), atol=1e-13)


def test_two_gaussians_front_to_back_order():
    """C = a1 c1 + (1 - a1) a2 c2; swapping the depths swaps the roles."""
    c1, c2 = f64([12.0, 14.0]), f64([16.0, 15.0])
    s1, s2, o1, o2 = f64(3.0), f64(4.0), f64(0.6), f64(0.8)
    col1, col2 = f64([1.0, 0.0]), f64([0.0, 1.0])
    a1 = _closed_gauss2d(32, 32, c1, s1, o1)
    a2 = _closed_gauss2d(32, 32, c2, s2, o2)
    for d1, d2 in ((1.0, 2.0), (2.0, 1.0)):
        sc = TS.scene2d([c1, c2], [s1, s2], [o1, o2], [d1, d2], [col1, col2])
        img = O.Oracle(sc).render_views()[0]["img"]
        if d1 < d2:
            exp = a1[None] * col1[:, None, None] + ((1 - a1) * a2)[None] * col2[:, None, None]
        else:
            exp = a2[None] * col2[:, None, None] + ((1 - a2) * a1)[None] * col1[:, None, None]
        np.testing.assert_allclose(img, exp, atol=1e-13, rtol=0)


def test_weights_sum_to_one_minus_T():
    """sum_k T_k alpha_k = 1 - T_final at every pixel (all features = 1)."""
    sc = S.tiny_2d()
    sc.feat = np.ones((sc.n, 1), np.float32)
    sc.channels = 1
    r = O.Oracle(sc).render_views()[0]
    np.testing.assert_allclose(r["img"][0], 1.0 - r["T"], atol=1e-12, rtol=0)
    assert (r["T"] >= 0).all() and (r["T"] <= 1).all()


def test_termination_stack_of_layers():
    """Identical centred layers with o = 0.8: alpha = 0.8 at the centre pixel, T after
    k layers = 0.2^k; T < 1e-4 first at k = 6 (6.4e-5; k = 5 gives 3.2e-4). With
    include-then-stop, layers 1..6 composite and layers 7, 8 get nothing."""
    n = 8
    o = float(np.float32(0.8))
    sc = TS.scene2d([[15.5, 15.5]] * n, [2.0] * n, [0.8] * n, np.arange(1, n + 1), np.ones((n, 1)))
    orc = O.Oracle(sc)
    r = orc.render_views()[0]
    assert r["ncontrib"][15, 15] == 6 and r["last"][15, 15] == 6
    assert r["T"][15, 15] == pytest.approx((1 - o) ** 6, rel=1e-12)
    g = np.zeros((1, 32, 32), np.float32)
    g[0, 15, 15] = 1.0
    gr = orc.backward([g])
    assert np.all(gr["opacity"][6:] == 0) and np.all(gr["feat"][6:] == 0)
    assert np.all(gr["feat"][:6, 0] > 0)
    # dC/dc_k = T_k alpha_k = 0.2^(k-1) * 0.8
    np.testing.assert_allclose(gr["feat"][:6, 0], [(1 - o) ** k * o for k in range(6)], rtol=1e-12)


def test_skip_below_alpha_min_is_strict():
    """A Gaussian whose peak alpha sits just under 1/255 contributes nothing."""
    o = float(np.nextafter(np.float32(A_MIN), np.float32(0)))
    sc = TS.scene2d([[8.5, 8.5]], [2.0], [o], [1.0], [[1.0]])
    r = O.Oracle(sc).render_views()[0]
    assert r["img"].max() == 0.0 and (r["T"] == 1.0).all()


# ---------------------------------------------------------------- EWA projection

def _quat_matrix_scipy(q):
    from scipy.spatial.transform import Rotation
    w, x, y, z = q
    return Rotation.from_quat([x, y, z, w]).as_matrix()


def test_ewa_isotropic_on_axis():
    """Isotropic Gaussian on the optical axis: Sigma2D = (f s / z)^2 I for any rotation."""
    rng = np.random.default_rng(7)
    f, z, s = 100.0, 5.0, f64(0.1)
    qs = rng.standard_normal((6, 4))
    sc = TS.scene3d(np.tile([0, 0, z], (6, 1)), np.full((6, 3), s), qs, np.full(6, 0.5),
                    np.ones((6, 1)), [TS.pinhole(32, 32, f)])
    pr = O.Oracle(sc).proj()
    np.testing.assert_allclose(pr["sxx"], (f * s / z) ** 2, rtol=1e-12)
    np.testing.assert_allclose(pr["syy"], (f * s / z) ** 2, rtol=1e-12)
    np.testing.assert_allclose(pr["sxy"], 0.0, atol=1e-12)
    np.testing.assert_allclose(pr["u"], 16.0, atol=1e-12)


@pytest.mark.parametrize("kind", ["pinhole", "spherical"])
def test_ewa_equals_numerical_jacobian(kind):
    """Sigma2D = J Sigma_world J^T with J = d(u,v)/d(mu) from central differences of the
    oracle's own projected means, and Sigma_world from scipy's quaternion rotation."""
    rng = np.random.default_rng(11)
    n = 12
    R = TS.rotation(rng)
    if kind == "pinhole":
        mu = np.stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), rng.uniform(3, 6, n)], 1)
        cam = S.Camera(S.CAM_PINHOLE, 64, 48, R, -R @ np.array([0.2, -0.1, 0.3]), fx=60.0, fy=55.0,
                       cx=31.0, cy=25.0, znear=0.2, zfar=100.0)
        mu = (R.T @ (mu.T)).T + np.array([0.2, -0.1, 0.3])
    else:
        az = rng.uniform(-np.pi, np.pi, n)
        el = rng.uniform(-0.3, 0.2, n)
        rr = rng.uniform(3, 8, n)
        loc = np.stack([rr * np.cos(el) * np.cos(az), rr * np.cos(el) * np.sin(az), rr * np.sin(el)], 1)
        cam = TS.lidar(128, 32, R=R, t=[0.1, 0.2, -0.3])
        mu = (R.T @ (loc - np.array([0.1, 0.2, -0.3])).T).T
    mu = f64(mu)
    s = f64(np.exp(rng.uniform(np.log(0.05), np.log(0.3), (n, 3))))
    q = f64(rng.standard_normal((n, 4)))
    sc = TS.scene3d(mu, s, q, np.full(n, 0.5), np.ones((n, 1)), [cam])
    base = O.Oracle(sc).proj()
    h = 1e-6
    J = np.zeros((n, 2, 3))
    for a in range(3):
        mp, mm = mu.copy(), mu.copy()
        mp[:, a] += h
        mm[:, a] -= h
        pp = O.Oracle(sc, pos=mp).proj()
        pm = O.Oracle(sc, pos=mm).proj()
        du = pp["u"] - pm["u"]
        if kind == "spherical":
            du = (du + 64) % 128 - 64
        J[:, 0, a] = du / (2 * h)
        J[:, 1, a] = (pp["v"] - pm["v"]) / (2 * h)
    for i in range(n):
        Rq = _quat_matrix_scipy(q[i] / np.linalg.norm(q[i]))
        Sw = Rq @ np.diag(s[i] ** 2) @ Rq.T
        S2 = J[i] @ Sw @ J[i].T
        np.testing.assert_allclose([base["sxx"][i], base["sxy"][i], base["syy"][i]],
                                   [S2[0, 0], S2[0, 1], S2[1, 1]], rtol=2e-6, atol=1e-9 * abs(S2).max())


def test_spherical_straight_ahead_closed_form():
    """A point straight ahead of the lidar (azimuth 0, elevation 0): u = W/2,
    v = el_max H / (el_max - el_min), Sigma2D = diag((a s / rho)^2, (b s / rho)^2)."""
    W, H = 128, 32
    rho, s = 5.0, f64(0.2)
    sc = TS.scene3d([[rho, 0, 0]], [[s, s, s]], [[1, 0, 0, 0]], [0.9], [[1.0]], [TS.lidar(W, H)])
    pr = O.Oracle(sc).proj()
    th_max, th_min = math.radians(15.0), math.radians(-25.0)
    a, b = W / (2 * math.pi), H / (th_max - th_min)
    assert pr["u"][0] == pytest.approx(W / 2, abs=1e-12)
    assert pr["v"][0] == pytest.approx(th_max * b, rel=1e-12)
    assert pr["sxx"][0] == pytest.approx((a * s / rho) ** 2, rel=1e-12)
    assert pr["syy"][0] == pytest.approx((b * s / rho) ** 2, rel=1e-12)
    assert pr["sxy"][0] == pytest.approx(0.0, abs=1e-12)
    assert pr["depth"][0] == pytest.approx(rho, rel=1e-15)


@pytest.mark.parametrize("behind", [False, True])
def test_lidar_single_gaussian_closed_form(behind):
    """Lidar image of one isotropic Gaussian: depth = alpha * range, opacity = alpha, with
    the horizontal offset wrapped around the seam (the 'behind' case straddles it)."""
    W, H = 128, 32
    rho, s, o = 4.0, f64(0.15), f64(0.8)
    m = [-rho, 0.0, 0.0] if behind else [rho, 0.0, 0.0]
    sc = TS.scene3d([m], [[s, s, s]], [[1, 0, 0, 0]], [o], [[1.0]], [TS.lidar(W, H)])
    r = O.Oracle(sc).render_views()[0]
    th_max, th_min = math.radians(15.0), math.radians(-25.0)
    a, b = W / (2 * math.pi), H / (th_max - th_min)
    u0 = 0.0 if behind else W / 2
    v0 = th_max * b
    ys, xs = np.mgrid[0:H, 0:W] + 0.5
    dx = (xs - u0 + W / 2) % W - W / 2
    dy = ys - v0
    al = np.minimum(float(np.float32(0.99)),
                    o * np.exp(-0.5 * ((dx / (a * s / rho)) ** 2 + (dy / (b * s / rho)) ** 2)))
    al = np.where(al < A_MIN, 0.0, al)
    np.testing.assert_allclose(r["img"][1], al, atol=1e-12)
    np.testing.assert_allclose(r["img"][0], al * rho, atol=1e-11)
    if behind:
        assert r["img"][1][:, 0].max() > 0.1 and r["img"][1][:, W - 1].max() > 0.1


# ---------------------------------------------------------------- sphere path

def _ray_dist(q, cam, W, H):
    """Orthogonal distance from q to every pixel ray, via the closest point on the ray."""
    ys, xs = np.mgrid[0:H, 0:W] + 0.5
    d = np.stack([(xs - cam.cx) / cam.fx, (ys - cam.cy) / cam.fy, np.ones_like(xs)], -1)
    tt = (d @ q) / np.einsum("hwk,hwk->hw", d, d)
    return np.linalg.norm(q[None, None, :] - tt[..., None] * d, axis=-1)


def test_sphere_single_closed_form():
    """One sphere: C = w f / (w + w_bg) with w = o (1 - dist^2/r^2) exp(o zhat / gamma)."""
    W = H = 32
    cam = TS.pinhole(W, H, 32.0, znear=1.0, zfar=21.0)
    prm = S.Params(gamma=1.0)
    q, r, o, f = f64([0.3, -0.2, 5.0]), f64(0.5), f64(0.6), f64([0.25, 0.75])
    sc = TS.spheres([q], [r], [o], [f], [cam], params=prm)
    res = O.Oracle(sc).render_views()[0]
    dist = _ray_dist(q, cam, W, H)
    D = np.clip(1 - dist ** 2 / r ** 2, 0, None)
    w = o * D * np.exp(o * ((21.0 - q[2]) / 20.0) / 1.0)
    exp = w[None] * f[:, None, None] / (w + 1.0)[None]
    np.testing.assert_allclose(res["img"], exp, atol=1e-12)
    np.testing.assert_allclose(res["N"], 1.0 + w, rtol=1e-12)
    assert ((res["top"][..., 0] == 0) == (D > 0)).all()


def test_sphere_blend_is_commutative():
    """Blending does not depend on sphere order (Pulsar appendix A), tau = 0."""
    rng = np.random.default_rng(5)
    sc = TS.random_spheres(rng, 300, 48, 48, 48.0, rmin=0.05, rmax=0.4)
    sc.params = S.Params(tau=0.0, gamma=0.05)
    base = O.Oracle(sc).render_views()[0]
    perm = rng.permutation(sc.n)
    sp = S.subset(sc, perm)
    sp.params = sc.params
    other = O.Oracle(sp).render_views()[0]
    np.testing.assert_allclose(other["img"], base["img"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(other["N"], base["N"], rtol=1e-12)


def _sphere_walk_inputs(sc):
    """Per sphere, from the raw inputs: sensor centre q, drawn radius r_eff, the
    stop bound b = exp(zhat(fp32 front depth) / gamma) and the exponent of the
    depth factor o zhat(qz) / gamma (Pulsar sec. 3.2 and appendix A), written
    here from the definitions, not taken from the oracle's projection."""
    cam, prm = sc.cams[0], sc.params
    R, t = f64(cam.R), f64(cam.t)
    q = f64(sc.pos) @ R.T + t
    r, o = f64(sc.scale), f64(sc.opacity)
    fmin = min(float(cam.fx), float(cam.fy))
    ortho = cam.kind == S.CAM_ORTHO
    rfl = np.full_like(r, 0.75 / fmin) if ortho else 0.75 * q[:, 2] / fmin
    re = np.maximum(r, rfl)
    front32 = (q[:, 2] - re).astype(np.float32).astype(np.float64)
    span = float(cam.zfar) - float(cam.znear)
    g = float(prm.gamma)
    b = np.exp((float(cam.zfar) - front32) / span / g)
    ex = o * (float(cam.zfar) - q[:, 2]) / span / g
    return q, re, o, b, ex


def _pixel_rays(cam, xs, ys):
    x, y = (xs + 0.5 - float(cam.cx)) / float(cam.fx), (ys + 0.5 - float(cam.cy)) / float(cam.fy)
    if cam.kind == S.CAM_ORTHO:
        org = np.stack([x, y, np.zeros_like(x)], -1)
        d = np.tile([0.0, 0.0, 1.0], (len(x), 1))
    else:
        org = np.zeros((len(x), 3))
        d = np.stack([x, y, np.ones_like(x)], -1)
    return org, d


def _stop_walk(sc, orc):
    """For every pixel, walk its tile's list (the oracle's sorted lists, pinned
    by the lexsort and brute-force tile-list tests) with the stop rule of
    Pulsar sec. 3.2 / Figure 3 and sec. B.1.3: stop at the first entry whose
    bound b < tau * N, N = bg_weight + the weights composited so far.
    Returns per pixel (row-major): the expected processed count, whether the
    rule fired, N at the end,
    the largest weight of any hitting sphere at or after the stop, and the
    smallest relative gap |b - tau N| / (tau N) over the entries it tested."""
    cam, prm = sc.cams[0], sc.params
    W, H = cam.width, cam.height
    q, re, o, b, ex = _sphere_walk_inputs(sc)
    _, vals, ranges = orc.pairs()
    tau, bgw = float(prm.tau), float(prm.bg_weight)
    proc = np.zeros(W * H, np.int64)
    fired = np.zeros(W * H, bool)
    Nend = np.zeros(W * H)
    wmax_after = np.zeros(W * H)
    gap = np.full(W * H, np.inf)
    for ty in range(cam.tiles_y):
        for tx in range(cam.tiles_x):
            s0, e0 = ranges[ty * cam.tiles_x + tx]
            ys, xs = np.mgrid[ty * 16:min(ty * 16 + 16, H), tx * 16:min(tx * 16 + 16, W)]
            xs, ys = xs.reshape(-1).astype(np.float64), ys.reshape(-1).astype(np.float64)
            pix = (ys * W + xs).astype(np.int64)
            ids = vals[s0:e0].astype(np.int64)
            L = len(ids)
            if L == 0:
                proc[pix], Nend[pix] = 0, bgw
                continue
            org, d = _pixel_rays(cam, xs, ys)
            e = q[ids][None, :, :] - org[:, None, :]
            ed = np.einsum("plk,pk->pl", e, d)
            dist2 = np.einsum("plk,plk->pl", e, e) - ed ** 2 / np.einsum("pk,pk->p", d, d)[:, None]
            r2 = re[ids] ** 2
            hit = dist2 < r2[None]
            w = np.where(hit, o[ids][None] * (1.0 - dist2 / r2[None]) * np.exp(ex[ids])[None], 0.0)
            Npre = np.cumsum(np.concatenate([np.full((len(pix), 1), bgw), w], 1), axis=1)[:, :L]
            lim = tau * Npre
            stop = b[ids][None] < lim
            has = stop.any(1)
            si = np.where(has, np.argmax(stop, 1), L)
            proc[pix] = np.where(has, si + 1, L)
            fired[pix] = has
            Nend[pix] = np.where(has, Npre[np.arange(len(pix)), np.minimum(si, L - 1)], Npre[:, -1] + w[:, -1])
            after = np.arange(L)[None] >= si[:, None]
            wmax_after[pix] = np.where(after, w, 0.0).max(1)
            tested = np.arange(L)[None] <= si[:, None]
            rel = np.abs(b[ids][None] - lim) / lim
            gap[pix] = np.where(tested, rel, np.inf).min(1)
    return proc, fired, Nend, wmax_after, gap


@pytest.mark.parametrize("camera", ["pinhole", "orthographic"])
def test_sphere_stop_rule_bruteforce(camera):
    """The oracle stops every pixel exactly where the rule b < tau N first holds
    (every entry before it had b >= tau N at its turn), and the rule is sound:
    every sphere at or after the stop weighs less than tau N_stop at that pixel
    (Pulsar sec. 3.2, Figure 3: the aggregated weight bounds the remainder).
    Dense scene with spheres behind the far plane too, so that many pixels stop
    with spheres close behind the stopping one."""
    rng = np.random.default_rng(61)
    W = H = 48
    if camera == "pinhole":
        cam = TS.pinhole(W, H, 48.0, znear=1.0, zfar=21.0)
        sc = TS.random_spheres(rng, 6000, W, H, 48.0, zmin=2.0, zmax=30.0, rmin=0.05, rmax=0.6, cam=cam)
    else:
        cam = _ortho_cam(W, H)
        sc = _ortho_spheres(rng, 6000, W, H, rmin=0.2, rmax=1.5)
        sc.pos[:, 2] = rng.uniform(2.0, 30.0, sc.n).astype(np.float32)
    orc = O.Oracle(sc)
    res = orc.render_views()[0]
    proc, fired, Nend, wmax_after, gap = _stop_walk(sc, orc)
    got_proc = res["processed"].reshape(-1)
    got_N = res["N"].reshape(-1)
    clear = gap > 1e-9                      # no bound within rounding of tau N
    assert clear.mean() > 0.999
    np.testing.assert_array_equal(got_proc[clear], proc[clear])
    np.testing.assert_allclose(got_N[clear], Nend[clear], rtol=1e-10)
    tau = float(sc.params.tau)
    assert (wmax_after < tau * got_N).all(), "a sphere dropped by the stop outweighs tau * N"
    # the rule fires at most pixels, with spheres close behind the stopping one:
    # a bound 20x too small would drop a sphere of weight >= tau N somewhere
    assert fired.mean() > 0.5
    assert (wmax_after > 0.05 * tau * got_N).sum() > 10


def test_sphere_stop_position_hand_built():
    """Four spheres on the ray of pixel (7, 7), each hit at its centre (D = 1).
    With gamma = 0.02, tau = 1e-5, znear 1, zfar 21, the weights are
    w = exp((21 - z) / 20 / 0.02) and the bounds b = exp((21 - (z - r)) / 20 / 0.02).
    A (z = 2) makes N ~ 4.3e20; B (z = 6.2) has b/(tau N) ~ 9.6: it is drawn;
    C (z = 8) has b/(tau N) ~ 0.11: the pixel stops there, so C and D are not
    composited. A bound off by a factor of 5 either way moves the stop."""
    W = H = 16
    cam = TS.pinhole(W, H, 16.0, znear=1.0, zfar=21.0)
    d = np.array([(7.5 - 8.0) / 16.0, (7.5 - 8.0) / 16.0, 1.0])
    zs = [2.0, 6.2, 8.0, 9.0]
    p = np.stack([z * d for z in zs])
    r = [0.5] * 4
    f = [[1.0, 0.0], [0.0, 1.0], [0.5, 0.5], [0.25, 0.75]]
    sc = TS.spheres(p, r, [1.0] * 4, f, [cam])
    prm = sc.params
    g, tau = float(prm.gamma), float(prm.tau)
    P = f64(sc.pos)
    zq = P[:, 2]
    front = (zq - f64(sc.scale)).astype(np.float32).astype(np.float64)
    w = np.exp((21.0 - zq) / 20.0 / g)
    b = np.exp((21.0 - front) / 20.0 / g)
    N = [1.0]
    for k in range(4):
        N.append(N[-1] + w[k])
    ratios = [b[k] / (tau * N[k]) for k in range(4)]
    assert ratios[0] > 1e10 and 5 < ratios[1] < 20 and 0.05 < ratios[2] < 0.2
    res = O.Oracle(sc).render_views()[0]
    assert res["processed"][7, 7] == 3 and res["ncontrib"][7, 7] == 2
    np.testing.assert_allclose(res["N"][7, 7], N[2], rtol=1e-9)
    col = (w[0] * f64(f[0]) + w[1] * f64(f[1])) / N[2]
    np.testing.assert_allclose(res["img"][:, 7, 7], col, rtol=1e-9)
    assert list(res["top"][7, 7, :3]) == [0, 1, -1]
    # tau = 0 never stops: all four are composited
    sc.params = S.Params(tau=0.0)
    res0 = O.Oracle(sc).render_views()[0]
    assert res0["processed"][7, 7] == 4 and res0["ncontrib"][7, 7] == 4
    np.testing.assert_allclose(res0["N"][7, 7], N[4], rtol=1e-9)


def test_spheres_behind_the_far_plane_are_culled():
    """A sphere whose fp32 front depth is not below zfar is culled: there the
    normalised depth is negative, a smaller opacity weighs more, and the stop
    bound would not hold. A bound exp(zhat(front)/gamma) of 3.7e-6 (front at
    zfar + span/4) would otherwise stop a background-only pixel (tau N = 1e-5)
    ahead of a sphere of opacity 0.1 weighing ~0.03. A sphere straddling zfar
    (front in front of it) is drawn."""
    W = H = 16
    cam = TS.pinhole(W, H, 16.0, znear=1.0, zfar=21.0)
    d = np.array([(7.5 - 8.0) / 16.0, (7.5 - 8.0) / 16.0, 1.0])
    # E: front 26 = zfar + span/4; F: o = 0.1 behind it; G: straddles zfar
    p = np.stack([26.5 * d, 27.0 * d, 21.3 * d])
    sc = TS.spheres(p, [0.5, 0.5, 0.5], [1.0, 0.1, 0.8], [[1.0], [0.5], [0.25]], [cam])
    orc = O.Oracle(sc)
    pr = orc.proj()
    assert list(pr["valid"]) == [0, 0, 1] and list(pr["ntiles"]) == [0, 0, 1]
    res = orc.render_views()[0]
    zq = f64(sc.pos)[2, 2]
    g = float(sc.params.gamma)
    D = 1.0 - _ray_dist(f64(sc.pos)[2], cam, W, H)[7, 7] ** 2 / 0.25
    w = float(np.float32(0.8)) * D * np.exp(float(np.float32(0.8)) * (21.0 - zq) / 20.0 / g)
    np.testing.assert_allclose(res["img"][0, 7, 7], w * 0.25 / (1.0 + w), rtol=1e-9)
    # the key depth decides: a front just below zfar in double that rounds to
    # zfar in fp32 is culled as well
    hit = None
    for r32 in np.float32(2.0) + np.arange(64, dtype=np.float32) * np.float32(1e-5):
        z = np.float32(21.0) + r32
        for _ in range(8):
            re = max(float(r32), 0.75 * float(z) / 16.0)
            zf = float(z) - re
            if zf < 21.0 and float(np.float32(zf)) == 21.0:
                hit = (z, r32)
                break
            z = np.nextafter(z, np.float32(0.0), dtype=np.float32)
        if hit:
            break
    assert hit is not None
    one = TS.spheres(np.array([[0.0, 0.0, float(hit[0])]]), [float(hit[1])], [1.0], [[1.0]], [cam])
    assert O.Oracle(one).proj()["valid"][0] == 0


def test_tangent_box_contains_every_hit_pixel():
    """Brute-force ray test over all pixels for 1000 spheres: every pixel with
    dist < r_eff lies inside the projected box; every sphere whose centre projects
    into the image gets at least one such pixel (Pulsar B.1.1)."""
    rng = np.random.default_rng(9)
    W = H = 64
    cam = S.Camera(S.CAM_PINHOLE, W, H, np.eye(3), [0.05, -0.02, 0.1], fx=64.0, fy=60.0, cx=31.5, cy=33.0,
                   znear=1.0, zfar=21.0)
    sc = TS.random_spheres(rng, 1000, W, H, 64.0, rmin=0.003, rmax=0.6, cam=cam)
    pr = O.Oracle(sc).proj()
    for i in range(sc.n):
        if not pr["valid"][i]:
            continue
        q = np.array([pr["m0"][i], pr["m1"][i], pr["m2"][i]])
        d = _ray_dist(q, cam, W, H)
        ys, xs = np.nonzero(d < pr["r_eff"][i])
        if len(xs):
            assert xs.min() >= pr["x0"][i] and xs.max() <= pr["x1"][i]
            assert ys.min() >= pr["y0"][i] and ys.max() <= pr["y1"][i]
        u = cam.fx * q[0] / q[2] + cam.cx
        v = cam.fy * q[1] / q[2] + cam.cy
        if 0 <= u < W and 0 <= v < H:
            assert d[int(v), int(u)] < pr["r_eff"][i]


# ------------------------------------------------ orthographic sphere camera

def _ortho_cam(W, H, fx=8.0, fy=7.5, cx=None, cy=None, t=(0.0, 0.0, 0.0)):
    return S.Camera(S.CAM_ORTHO, W, H, np.eye(3), t, fx=fx, fy=fy, cx=W / 2 if cx is None else cx,
                    cy=H / 2 if cy is None else cy, znear=1.0, zfar=21.0)


def _ortho_spheres(rng, n, W, H, rmin=0.01, rmax=0.6):
    cam = _ortho_cam(W, H)
    u, v = rng.uniform(-2, W + 2, n), rng.uniform(-2, H + 2, n)
    p = np.stack([(u - cam.cx) / cam.fx, (v - cam.cy) / cam.fy, rng.uniform(2, 20, n)], 1)
    r = np.exp(rng.uniform(math.log(rmin), math.log(rmax), n))
    return TS.spheres(p, r, rng.uniform(0.1, 1.0, n), rng.uniform(0, 1, (n, 3)), [cam])


def _ortho_dist(q, cam, W, H):
    """Distance of q from each pixel's ray, a line parallel to the optical axis
    through ((px - cx)/fx, (py - cy)/fy) in the sensor frame."""
    ys, xs = np.mgrid[0:H, 0:W] + 0.5
    return np.hypot((xs - cam.cx) / cam.fx - q[0], (ys - cam.cy) / cam.fy - q[1])


def test_ortho_sphere_single_closed_form():
    """One sphere seen by an orthographic camera: C = w f / (w + w_bg) with
    w = o (1 - dist^2/r^2) exp(o zhat / gamma), dist the offset from the axis-parallel ray."""
    W, H = 40, 32
    cam = _ortho_cam(W, H, t=(0.1, -0.2, 0.5))
    prm = S.Params(gamma=1.0)
    p, r, o, f = f64([0.3, -0.2, 5.0]), f64(1.5), f64(0.6), f64([0.25, 0.75])
    sc = TS.spheres([p], [r], [o], [f], [cam], params=prm)
    res = O.Oracle(sc).render_views()[0]
    q = p + f64(cam.t)
    dist = _ortho_dist(q, cam, W, H)
    D = np.clip(1 - dist ** 2 / r ** 2, 0, None)
    w = o * D * np.exp(o * ((21.0 - q[2]) / 20.0) / 1.0)
    exp = w[None] * f[:, None, None] / (w + 1.0)[None]
    np.testing.assert_allclose(res["img"], exp, atol=1e-12)
    np.testing.assert_allclose(res["N"], 1.0 + w, rtol=1e-12)
    # the disc covers about pi (fx r)(fy r) pixel centres
    assert abs((D > 0).sum() - math.pi * cam.fx * r * cam.fy * r) < 0.1 * math.pi * cam.fx * r * cam.fy * r


def test_ortho_depth_moves_only_the_weight():
    """Orthographic projection: moving a sphere along the optical axis keeps its
    footprint; with no background weight a lone sphere's colour is its feature."""
    W, H = 24, 24
    cam = _ortho_cam(W, H)
    prm = S.Params(gamma=1.0, bg_weight=0.0, tau=0.0)
    out = []
    for z in (3.0, 11.0):
        sc = TS.spheres([[0.2, -0.3, z]], [1.0], [0.7], [[0.4, 0.9]], [cam], params=prm)
        out.append(O.Oracle(sc).render_views()[0])
    np.testing.assert_array_equal(out[0]["ncontrib"], out[1]["ncontrib"])
    hit = out[0]["ncontrib"] > 0
    assert hit.sum() > 20
    np.testing.assert_allclose(out[0]["img"][:, hit], np.array([[0.4], [0.9]]) * np.ones(hit.sum()), rtol=1e-6)


def test_ortho_box_contains_every_hit_pixel():
    """Brute-force ray test over all pixels for 600 spheres under the orthographic
    camera: every pixel within r_eff of its ray lies inside the box; every sphere
    whose centre projects into the image keeps at least one pixel (one-pixel floor)."""
    rng = np.random.default_rng(19)
    W, H = 64, 56
    sc = _ortho_spheres(rng, 600, W, H, rmin=0.003, rmax=1.2)
    cam = sc.cams[0]
    pr = O.Oracle(sc).proj()
    nfloor = 0
    for i in range(sc.n):
        if not pr["valid"][i]:
            continue
        q = np.array([pr["m0"][i], pr["m1"][i], pr["m2"][i]])
        d = _ortho_dist(q, cam, W, H)
        ys, xs = np.nonzero(d < pr["r_eff"][i])
        if len(xs):
            assert xs.min() >= pr["x0"][i] and xs.max() <= pr["x1"][i]
            assert ys.min() >= pr["y0"][i] and ys.max() <= pr["y1"][i]
        u = cam.fx * q[0] + cam.cx
        v = cam.fy * q[1] + cam.cy
        if 0 <= u < W and 0 <= v < H:
            assert d[int(v), int(u)] < pr["r_eff"][i]
        nfloor += int(pr["floored"][i])
    assert nfloor > 10


# ---------------------------------------------------------------- tiles and sort

def _lexsort_pairs(orc):
    pr = orc.proj()
    tiles, bits, ids = [], [], []
    for k in np.nonzero(pr["valid"])[0]:
        v = k // orc.n
        c = orc.cams[v]
        toff = sum(cc.tiles_x * cc.tiles_y for cc in orc.cams[:v])
        for ty in range(pr["ty0"][k], pr["ty1"][k] + 1):
            for a in range(pr["ntx"][k]):
                tx = (pr["tx0"][k] + a) % c.tiles_x
                tiles.append(toff + ty * c.tiles_x + tx)
                bits.append(pr["key_bits"][k])
                ids.append(k)
    tiles, bits, ids = map(np.asarray, (tiles, bits, ids))
    order = np.lexsort((ids, bits, tiles))
    return (tiles[order].astype(np.uint64) << np.uint64(32)) | bits[order].astype(np.uint64), ids[order]


@pytest.mark.parametrize("which", ["2d", "3d", "sphere", "ortho", "lidar"])
def test_sort_order_equals_lexsort(which):
    rng = np.random.default_rng(3)
    if which == "2d":
        sc = S.tiny_2d(n=600)
    elif which == "3d":
        sc = S.gauss3d(n=20000, width=96, height=80)
    elif which == "sphere":
        sc = TS.random_spheres(rng, 3000, 80, 64, 70.0, rmin=0.01, rmax=0.2)
    elif which == "ortho":
        sc = _ortho_spheres(rng, 3000, 80, 64)
    else:
        sc = S.gauss3d(n=2000)
        sc.cams = [TS.lidar(256, 32, t=[0.0, 0.0, 0.0])]
    orc = O.Oracle(sc)
    keys, vals, ranges = orc.pairs()
    k2, v2 = _lexsort_pairs(orc)
    assert len(keys) > 1000
    np.testing.assert_array_equal(keys, k2)
    np.testing.assert_array_equal(vals, v2)
    t = (keys >> np.uint64(32)).astype(np.int64)
    for tile in np.unique(t)[:50]:
        sel = np.nonzero(t == tile)[0]
        assert ranges[tile, 0] == sel[0] and ranges[tile, 1] == sel[-1] + 1


@pytest.mark.parametrize("which", ["2d", "3d", "sphere", "ortho", "lidar"])
def test_tile_lists_equal_bruteforce(which):
    """Compositing over each tile's list equals compositing over every primitive in
    global (depth bits, id) order with no tiles at all, bit for bit."""
    rng = np.random.default_rng(4)
    if which == "2d":
        sc = S.tiny_2d()
    elif which == "3d":
        sc = S.gauss3d(n=20000, width=96, height=80)
    elif which == "sphere":
        sc = TS.random_spheres(rng, 3000, 80, 64, 70.0, rmin=0.01, rmax=0.2)
    elif which == "ortho":
        sc = _ortho_spheres(rng, 3000, 80, 64)
    else:
        sc = S.gauss3d(n=3000)
        sc.cams = [TS.lidar(256, 32)]
    orc = O.Oracle(sc)
    a = orc.render_views()[0]
    b = orc.render_bruteforce(0)
    np.testing.assert_array_equal(a["img"], b["img"])
    if sc.kind == S.PRIM_SPHERE:
        np.testing.assert_array_equal(a["N"], b["N"])
        np.testing.assert_array_equal(a["top"], b["top"])
    else:
        np.testing.assert_array_equal(a["T"], b["T"])


# ------------------------------------- closest-K recording (Pulsar B.1.3, B.1.4)

def _entry_depths(pr, cam, W, H, ortho):
    """Per pixel and sphere: sensor depth where the pixel's ray enters the sphere
    (inf if it misses), from the closest-approach point minus the half chord."""
    ys, xs = np.mgrid[0:H, 0:W] + 0.5
    x = ((xs - cam.cx) / cam.fx).reshape(-1, 1)
    y = ((ys - cam.cy) / cam.fy).reshape(-1, 1)
    q = np.stack([pr["m0"], pr["m1"], pr["m2"]], 1)[None]           # [1, n, 3]
    r = pr["r_eff"][None]
    if ortho:
        dist2 = (q[..., 0] - x) ** 2 + (q[..., 1] - y) ** 2
        z = q[..., 2] - np.sqrt(np.maximum(r ** 2 - dist2, 0.0))
    else:
        d = np.stack([x, y, np.ones_like(x)], -1)                    # [pix, 1, 3]
        dn = np.linalg.norm(d, axis=-1)
        cross = np.cross(q, d)
        dist2 = (cross ** 2).sum(-1) / dn ** 2
        s_c = (q * d).sum(-1) / dn ** 2                               # closest approach
        z = s_c - np.sqrt(np.maximum(r ** 2 - dist2, 0.0)) / dn      # d_z = 1: s is the depth
    return np.where((dist2 < r ** 2) & pr["valid"].astype(bool)[None], z, np.inf)


@pytest.mark.parametrize("ortho", [False, True])
def test_closest_k_by_entry_depth_bruteforce(ortho):
    """With no early stop every hit contributes, so the recorded spheres are the K
    hits of smallest entry depth (list order breaks ties), reported in list order."""
    rng = np.random.default_rng(31 + ortho)
    W, H, K = 40, 32, 5
    if ortho:
        sc = _ortho_spheres(rng, 400, W, H, rmin=0.3, rmax=2.0)
    else:
        sc = TS.random_spheres(rng, 400, W, H, 40.0, rmin=0.1, rmax=0.8)
    sc.params = S.Params(tau=0.0, top_k=K, top_by_depth=1)
    orc = O.Oracle(sc)
    r = orc.render_views()[0]
    assert (r["flags"] == 0).mean() > 0.99
    pr = orc.proj()
    z = _entry_depths(pr, sc.cams[0], W, H, ortho)
    order = np.lexsort((np.arange(sc.n), pr["key_bits"]))              # list order of the spheres
    rank = np.empty(sc.n, np.int64)
    rank[order] = np.arange(sc.n)
    top = r["top"].reshape(-1, K)
    ok = (r["flags"].reshape(-1) == 0)
    nhit_many = 0
    for p in np.nonzero(ok)[0]:
        hits = np.nonzero(np.isfinite(z[p]))[0]
        sel = hits[np.lexsort((rank[hits], z[p, hits]))][:K]
        want = sel[np.argsort(rank[sel])]
        got = top[p][top[p] >= 0]
        np.testing.assert_array_equal(got, want, err_msg=f"pixel {p}")
        nhit_many += len(hits) > K
    assert nhit_many > 200                                              # selection actually matters


def test_closest_k_equals_first_k_when_all_fit():
    """When no pixel has more than K hits both recording rules keep every hit."""
    rng = np.random.default_rng(35)
    sc = TS.random_spheres(rng, 60, 40, 32, 40.0, rmin=0.05, rmax=0.3)
    sc.params = S.Params(tau=0.0, top_k=8)
    a = O.Oracle(sc).render_views()[0]
    assert a["ncontrib"].max() <= 8 and a["ncontrib"].max() >= 2
    sc.params = S.Params(tau=0.0, top_k=8, top_by_depth=1)
    b = O.Oracle(sc).render_views()[0]
    np.testing.assert_array_equal(a["top"], b["top"])
    np.testing.assert_array_equal(a["img"], b["img"])


# ---------------------------------------------- max-shifted sphere normalisation

def test_max_shift_single_sphere_small_gamma():
    """gamma = 1/200: the weight o D exp(o zhat / gamma) reaches e^100 and more. With
    the shift m = ln o + o zhat / gamma the reported normalisation is D + exp(-m)
    where the sphere is hit (w_bg = 1) and exp(0) = 1 elsewhere, T carries m (0 where
    nothing contributes), and the colour is the plain w f / (w + 1)."""
    W = H = 32
    cam = TS.pinhole(W, H, 32.0, znear=1.0, zfar=21.0)
    prm = S.Params(gamma=0.005, max_shift=1, tau=0.0)
    q, r, o, f = f64([0.3, -0.2, 5.0]), f64(0.5), f64(0.6), f64([0.25, 0.75])
    sc = TS.spheres([q], [r], [o], [f], [cam], params=prm)
    res = O.Oracle(sc).render_views()[0]
    gam = f64(float(np.float32(0.005)))
    lam = math.log(o) + o * ((21.0 - q[2]) / 20.0) / gam
    assert lam > 88.0
    D = np.clip(1 - _ray_dist(q, cam, W, H) ** 2 / r ** 2, 0, None)
    hit = D > 0
    np.testing.assert_allclose(res["N"][hit], D[hit] + math.exp(-lam), rtol=1e-12)
    np.testing.assert_allclose(res["N"][~hit], 1.0, rtol=0)
    np.testing.assert_allclose(res["T"][hit], lam, rtol=1e-12)
    assert (res["T"][~hit] == 0).all()
    w_rel = D[hit]                                           # w exp(-lam)
    np.testing.assert_allclose(res["img"][:, hit], f[:, None] * (w_rel / (w_rel + math.exp(-lam)))[None],
                               rtol=1e-12)


def test_max_shift_only_rescales_the_normalisation():
    """At gamma = 0.02 (no overflow either way) the shifted run gives the same image,
    top-K and gradients; its N times exp(T) is the unshifted N, and T is the largest
    log-weight of the pixel's hits, or 0 (brute force over the spheres, tau = 0)."""
    rng = np.random.default_rng(37)
    W, H = 40, 32
    sc = TS.random_spheres(rng, 300, W, H, 40.0, rmin=0.05, rmax=0.5)
    sc.params = S.Params(tau=0.0)
    a = O.Oracle(sc)
    ra = a.render_views()[0]
    sc.params = S.Params(tau=0.0, max_shift=1)
    b = O.Oracle(sc)
    rb = b.render_views()[0]
    np.testing.assert_array_equal(ra["img"], rb["img"])
    np.testing.assert_array_equal(ra["top"], rb["top"])
    np.testing.assert_allclose(rb["N"] * np.exp(rb["T"]), ra["N"], rtol=1e-12)
    pr = a.proj()
    lam = np.log(pr["opac"]) + pr["opac"] * pr["zhat"] / float(np.float32(0.02))
    cam = sc.cams[0]
    want = np.zeros((H, W))
    for i in np.nonzero(pr["valid"])[0]:
        q = np.array([pr["m0"][i], pr["m1"][i], pr["m2"][i]])
        d = _ray_dist(q, cam, W, H)
        want = np.where(d < pr["r_eff"][i], np.maximum(want, lam[i]), want)
    np.testing.assert_allclose(rb["T"], want, rtol=1e-12, atol=0)
    g = [np.random.default_rng(3).standard_normal((3, H, W)).astype(np.float32)]
    ga, gb = a.backward(g), b.backward(g)
    for k in ("pos", "scale", "opacity", "feat", "cam_R", "cam_t"):
        np.testing.assert_array_equal(ga[k], gb[k])


def test_lidar_half_turn_scene_reaches_the_antipode():
    """The lidar half-turn parity scene lists entries centred within 8 columns of
    the half turn from their tile's centre, and for some of them pixels of the
    tile lie more than half a turn from the centre's image nearest the tile
    centre: the case the per-pixel column wrap exists for."""
    sc = TS.lidar_half_turn()
    orc = O.Oracle(sc)
    pr = orc.proj()
    keys, vals, _ = orc.pairs()
    W = sc.cams[0].width
    TW = (W + 15) // 16
    tile = (keys >> np.uint64(32)).astype(np.int64)
    u = pr["u"][vals.astype(np.int64)]
    tx = tile % TW
    du = np.mod(u - (16 * tx + 8) + W / 2, W) - W / 2       # nearest image, from the tile centre
    near = np.abs(du) >= W / 2 - 8
    assert near.sum() >= 50
    # pixel columns of those tiles that lie more than W/2 from that image
    px = np.arange(16)[None, :] + 0.5 - 8.0                  # from the tile centre
    off = px - du[near][:, None]
    assert ((off >= W / 2) | (off < -W / 2)).sum() >= 100
    orc.close()

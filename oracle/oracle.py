"""ctypes wrapper around the C oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg import this module; the library never does. It shares no code
with the HIP path. Inputs are promoted to float64 before the call.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "splat_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

CAM_STRIDE = 24
NPD, NPI = 17, 13
G_OFF = 8

FLAG_ALPHA_MIN, FLAG_T_STOP, FLAG_CLAMP, FLAG_SPH_EDGE, FLAG_SPH_STOP = 1, 2, 4, 8, 16
FLAG_SPH_ZTIE = 32          # closest-K recording: K-th and next entry depth nearly equal
FLAG_UNRESOLVED = 64        # more near-tie decisions along one outcome than render_alts enumerates
# near-tie decisions whose two outcomes render_alts enumerates (both are correct)
DECISION_FLAGS = FLAG_ALPHA_MIN | FLAG_T_STOP | FLAG_SPH_EDGE | FLAG_SPH_STOP
IMAGE_FLAGS = DECISION_FLAGS
MAX_TIES = 3
EPS_ALPHA = 1.5e-6          # relative error bound of an fp32 alpha (see the C source)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (double precision, no FP contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = C.CDLL(_SO)
        vp, dp, ip = C.c_void_p, C.POINTER(C.c_double), C.c_int
        L.or_create.restype = vp
        L.or_create.argtypes = [ip, ip, ip, dp, dp, dp, dp, dp, dp, ip, dp, dp]
        L.or_destroy.argtypes = [vp]
        L.or_total_tiles.restype = C.c_longlong
        L.or_total_tiles.argtypes = [vp]
        L.or_total_pix.restype = C.c_longlong
        L.or_total_pix.argtypes = [vp]
        L.or_get_proj.argtypes = [vp, vp, vp]
        L.or_bin.restype = C.c_longlong
        L.or_bin.argtypes = [vp]
        L.or_get_pairs.argtypes = [vp, vp, vp, vp]
        L.or_render.argtypes = [vp, C.c_longlong, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.or_render_alts.argtypes = [vp, C.c_longlong, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.or_set_branches.argtypes = [vp, vp]
        L.or_threads.restype = C.c_int
        L.or_threads.argtypes = [C.c_int]
        L.or_render_bruteforce.argtypes = [vp, ip, vp, vp, vp, vp]
        L.or_backward.argtypes = [vp] * 11 + [C.c_int]
        L.or_backward_mag.argtypes = [vp] * 19 + [C.c_int]
        _lib = L
    return _lib


def threads(n: int = 0) -> int:
    """Threads of the oracle's parallel loops; n > 0 sets them first."""
    return int(lib().or_threads(int(n)))


def _d(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(C.POINTER(C.c_double))


def _vp(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


def pack_cams(cams) -> np.ndarray:
    out = np.zeros((len(cams), CAM_STRIDE), dtype=np.float64)
    for v, c in enumerate(cams):
        out[v, 0] = c.kind
        out[v, 1] = c.width
        out[v, 2] = c.height
        out[v, 3:12] = np.asarray(c.R, dtype=np.float64).reshape(9)
        out[v, 12:15] = np.asarray(c.t, dtype=np.float64)
        out[v, 15:23] = [c.fx, c.fy, c.cx, c.cy, c.el_min_deg, c.el_max_deg, c.znear, c.zfar]
    return out


def pack_params(params, channels) -> np.ndarray:
    bg = np.zeros(channels) if params.background is None else np.asarray(params.background, np.float64)
    head = [params.alpha_min, params.alpha_max, params.T_min, params.gamma, params.bg_weight,
            params.tau, params.top_k, params.top_by_depth, getattr(params, "max_shift", 0)]
    return np.ascontiguousarray(np.concatenate([np.asarray(head, np.float64), bg]))


class Oracle:
    """Projection, binning, compositing and gradients of one scene in float64.

    Arrays may be float32 (promoted exactly) or float64 (for finite differences).
    """

    def __init__(self, scene, pos=None, scale=None, rot=None, opacity=None, feat=None,
                 depth=None, cams=None, params=None, packed_cams=None):
        s = scene
        self.kind, self.n, self.C = s.kind, s.n, s.channels
        self.cams = list(cams if cams is not None else s.cams)
        self.V = len(self.cams)
        if s.kind != 2 and any(c.kind == 2 for c in self.cams):
            raise ValueError("orthographic views are defined for spheres only")
        if s.kind == 2 and any(not c.zfar > c.znear for c in self.cams):
            raise ValueError("sphere views need zfar > znear (the normalised depth divides by the span)")
        self.params = params if params is not None else s.params
        self.K = self.params.top_k
        pick = lambda a, b: _d(a if a is not None else b)
        self._keep = [pick(pos, s.pos), pick(scale, s.scale), pick(rot, s.rot),
                      pick(opacity, s.opacity), pick(depth, s.depth), pick(feat, s.feat),
                      pack_cams(self.cams) if packed_cams is None else _d(packed_cams),
                      pack_params(self.params, self.C)]
        a = self._keep
        self.h = lib().or_create(self.kind, self.n, self.C, _p(a[0]), _p(a[1]), _p(a[2]), _p(a[3]),
                                 _p(a[4]), _p(a[5]), self.V, _p(a[6]), _p(a[7]))
        self.total_tiles = lib().or_total_tiles(self.h)
        self.total_pix = lib().or_total_pix(self.h)
        self.npairs = None

    def close(self):
        if self.h:
            lib().or_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- projection -----------------------------------------------------
    def proj(self) -> dict:
        NV = self.V * self.n
        d = np.zeros((NV, NPD), np.float64)
        i = np.zeros((NV, NPI), np.int64)
        lib().or_get_proj(self.h, _vp(d), _vp(i))
        names_d = ["u", "v", "sxx", "sxy", "syy", "ca", "cb", "cc", "depth", "m0", "m1", "m2",
                   "r_eff", "e", "b", "zhat", "opac"]
        names_i = ["valid", "x0", "x1", "y0", "y1", "tx0", "ntx", "ty0", "ty1", "ntiles",
                   "key_bits", "floored", "gated"]
        out = {k: d[:, j] for j, k in enumerate(names_d)}
        out.update({k: i[:, j] for j, k in enumerate(names_i)})
        return out

    # ---- binning --------------------------------------------------------
    def bin(self) -> int:
        self.npairs = lib().or_bin(self.h)
        return self.npairs

    def pairs(self):
        if self.npairs is None:
            self.bin()
        keys = np.zeros(self.npairs, np.uint64)
        vals = np.zeros(self.npairs, np.uint32)
        ranges = np.zeros((self.total_tiles, 2), np.uint32)
        lib().or_get_pairs(self.h, _vp(keys), _vp(vals), _vp(ranges))
        return keys, vals, ranges

    # ---- forward --------------------------------------------------------
    def render(self, pix=None) -> dict:
        """Composite the given global pixel ids (default: every pixel of every view)."""
        if self.npairs is None:
            self.bin()
        if pix is not None:
            pix = np.ascontiguousarray(np.asarray(pix, dtype=np.int64))
            cnt = len(pix)
        else:
            cnt = self.total_pix
        Cm = max(self.C, 2)
        img = np.zeros((cnt, Cm))
        T = np.zeros(cnt)
        last = np.zeros(cnt, np.int64)
        N = np.zeros(cnt)
        top = np.zeros((cnt, max(self.K, 1)), np.int32)
        flags = np.zeros(cnt, np.int32)
        proc = np.zeros(cnt, np.int64)
        ncon = np.zeros(cnt, np.int64)
        errb = np.zeros(cnt)
        lib().or_render(self.h, cnt, _vp(pix), _vp(img), _vp(T), _vp(last), _vp(N), _vp(top),
                        _vp(flags), _vp(proc), _vp(ncon), _vp(errb))
        return dict(img=img, T=T, last=last, N=N, top=top[:, :self.K], flags=flags,
                    processed=proc, ncontrib=ncon, errb=errb)

    def render_alts(self, pix) -> dict:
        """Every outcome of the given pixels over their near-tie decisions (both
        outcomes of each of the first MAX_TIES ties met are correct). Arrays
        [npix, 2^MAX_TIES, ...]; slots a >= nalt[q] are unused; mask[q, a] is the
        flip mask that gives outcome a (0: the default outcome)."""
        if self.npairs is None:
            self.bin()
        pix = np.ascontiguousarray(np.asarray(pix, dtype=np.int64))
        cnt, NA, Cm, K = len(pix), 1 << MAX_TIES, max(self.C, 2), max(self.K, 1)
        nalt = np.zeros(cnt, np.int32)
        mask = np.zeros((cnt, NA), np.int32)
        img = np.zeros((cnt, NA, Cm))
        T = np.zeros((cnt, NA))
        last = np.zeros((cnt, NA), np.int64)
        N = np.zeros((cnt, NA))
        top = np.zeros((cnt, NA, K), np.int32)
        unres = np.zeros(cnt, np.int32)
        if cnt:
            lib().or_render_alts(self.h, cnt, _vp(pix), _vp(nalt), _vp(mask), _vp(img), _vp(T), _vp(last),
                                 _vp(N), _vp(top), _vp(unres))
        return dict(nalt=nalt, mask=mask, img=img, T=T, last=last, N=N, top=top[:, :, :self.K],
                    unresolved=unres.astype(bool))

    def set_branches(self, branch):
        """Per global pixel, the flip mask (render_alts) the reverse pass follows;
        None: the default outcome everywhere."""
        if branch is None:
            self._branch = None
            lib().or_set_branches(self.h, None)
            return
        b = np.ascontiguousarray(np.asarray(branch, dtype=np.int32))
        assert b.shape == (self.total_pix,)
        self._branch = b
        lib().or_set_branches(self.h, _vp(b))

    def render_views(self) -> list:
        """Full images per view as dicts of [C,H,W] / [H,W] arrays."""
        r = self.render()
        out, off = [], 0
        for c in self.cams:
            hw = c.width * c.height
            sl = slice(off, off + hw)
            Cv = 2 if c.kind == 1 else self.C
            out.append(dict(img=r["img"][sl, :Cv].T.reshape(Cv, c.height, c.width),
                            T=r["T"][sl].reshape(c.height, c.width),
                            last=r["last"][sl].reshape(c.height, c.width),
                            N=r["N"][sl].reshape(c.height, c.width),
                            top=r["top"][sl].reshape(c.height, c.width, self.K),
                            flags=r["flags"][sl].reshape(c.height, c.width),
                            processed=r["processed"][sl].reshape(c.height, c.width),
                            ncontrib=r["ncontrib"][sl].reshape(c.height, c.width)))
            off += hw
        return out

    def render_bruteforce(self, view=0) -> dict:
        if self.params.top_by_depth:
            raise ValueError("the brute-force renderer records the first top_k contributions only")
        c = self.cams[view]
        hw = c.width * c.height
        Cm = max(self.C, 2)
        img = np.zeros((hw, Cm))
        T = np.zeros(hw)
        N = np.zeros(hw)
        top = np.zeros((hw, max(self.K, 1)), np.int32)
        lib().or_render_bruteforce(self.h, view, _vp(img), _vp(T), _vp(N), _vp(top))
        Cv = 2 if c.kind == 1 else self.C
        return dict(img=img[:, :Cv].T.reshape(Cv, c.height, c.width), T=T.reshape(c.height, c.width),
                    N=N.reshape(c.height, c.width), top=top[:, :self.K].reshape(c.height, c.width, self.K))

    # ---- backward -------------------------------------------------------
    def backward(self, dimg_views, with_mag: bool = False, normalize: bool = False) -> dict:
        """dimg_views: list of [Cv,H,W] arrays (one per view). Returns float64 grads.

        normalize (spheres): sphere gradients averaged over their contributing pixels,
        camera contributions divided by projected area and 1e-3 (Pulsar B.2).

        with_mag adds "mag": for every gradient the sum of the magnitudes of the
        terms that make it up (a bound for what rounding in the terms can do to
        the sum; it is not part of the gradient).
        """
        if self.npairs is None:
            self.bin()
        g = np.ascontiguousarray(np.concatenate([np.asarray(a, np.float32).reshape(-1)
                                                 for a in dimg_views]))
        n, Cc = self.n, self.C
        pd = 2 if self.kind == 0 else 3
        sd = 3 if self.kind == 1 else 1

        def outs():
            return dict(pos=np.zeros((n, pd)), scale=np.zeros((n, sd)) if sd > 1 else np.zeros(n),
                        rot=np.zeros((n, 4)) if self.kind == 1 else None, opacity=np.zeros(n),
                        feat=np.zeros((n, Cc)) if Cc > 0 else None, cam_R=np.zeros((self.V, 3, 3)),
                        cam_t=np.zeros((self.V, 3)), cam_K=np.zeros((self.V, 4)))

        o = outs()
        acc = np.zeros((self.V * n, G_OFF + Cc))
        args = [self.h, _vp(g)] + [_vp(o[k]) for k in ("pos", "scale", "rot", "opacity", "feat", "cam_R", "cam_t")]
        args.append(_vp(acc))
        if with_mag:
            m = outs()
            lib().or_backward_mag(*args, *[_vp(m[k]) for k in ("pos", "scale", "rot", "opacity", "feat",
                                                               "cam_R", "cam_t")],
                                  _vp(o["cam_K"]), _vp(m["cam_K"]), int(normalize))
            o["mag"] = m
        else:
            lib().or_backward(*args, _vp(o["cam_K"]), int(normalize))
        o["acc"] = acc
        return o

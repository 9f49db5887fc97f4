"""Per-frame parameter assembly, plain float64 numpy (the oracle of splat_interpolate).

TEST INFRASTRUCTURE ONLY: the tests import this module; the library never does.
It shares no code with the HIP path.

NuRec's profiling page ("Profiling with Nsight Systems", "Fusing small kernels and
removing synchronizations") names a per-frame step, interpolate inside
collect_gaussian_parameters, that assembles the Gaussian parameters of one frame
before rendering, and fuses its many small kernels into one. The page does not
say what is interpolated. Reading used here: every primitive carries its centre
and its rotation quaternion at n_keys keyframe times t_0 < t_1 < ...; the frame at
time t takes the bracketing keyframes k, k + 1 (t_k <= t <= t_{k+1}; t outside
[t_0, t_last] clamps to the end frame) with w = (t - t_k) / (t_{k+1} - t_k) and
  centre   = (1 - w) c_k + w c_{k+1}
  rotation = (1 - w) q_k + w s q_{k+1},  s = -1 if q_k . q_{k+1} < 0 else 1
(normalised linear interpolation, the sign taking the shorter arc; the projection
normalises the quaternion). Scales, opacities and features do not change.
"""
from __future__ import annotations

import numpy as np


def bracket(key_times, t):
    """(k, k1, w) for time t: keyframe indices and the weight of k1."""
    kt = np.asarray(key_times, np.float64)
    n = len(kt)
    if n == 1 or t <= kt[0]:
        return 0, 0, 0.0
    if t >= kt[-1]:
        return n - 1, n - 1, 0.0
    k = int(np.searchsorted(kt, t, side="right")) - 1     # kt[k] <= t < kt[k+1]
    return k, k + 1, float((t - kt[k]) / (kt[k + 1] - kt[k]))


def interpolate(key_times, t, key_pos, key_rot):
    """key_pos [K][n][3], key_rot [K][n][4] -> pos [n][3], rot [n][4] (float64)."""
    k, k1, w = bracket(key_times, t)
    p0, p1 = np.asarray(key_pos[k], np.float64), np.asarray(key_pos[k1], np.float64)
    q0, q1 = np.asarray(key_rot[k], np.float64), np.asarray(key_rot[k1], np.float64)
    s = np.where((q0 * q1).sum(1) < 0.0, -1.0, 1.0)[:, None]
    return (1.0 - w) * p0 + w * p1, (1.0 - w) * q0 + w * s * q1


def interpolate_backward(key_times, t, key_rot, d_pos, d_rot):
    """Gradients w.r.t. key_pos and key_rot ([K][n][3], [K][n][4]) of a loss whose
    gradients w.r.t. the assembled pos and rot are d_pos, d_rot (the sign s is a
    discrete choice and carries no gradient)."""
    K = len(key_times)
    k, k1, w = bracket(key_times, t)
    d_pos = np.asarray(d_pos, np.float64)
    d_rot = np.asarray(d_rot, np.float64)
    n = d_pos.shape[0]
    gp = np.zeros((K, n, 3))
    gr = np.zeros((K, n, 4))
    q0, q1 = np.asarray(key_rot[k], np.float64), np.asarray(key_rot[k1], np.float64)
    s = np.where((q0 * q1).sum(1) < 0.0, -1.0, 1.0)[:, None]
    gp[k] += (1.0 - w) * d_pos
    gp[k1] += w * d_pos
    gr[k] += (1.0 - w) * d_rot
    gr[k1] += w * s * d_rot
    return gp, gr


def sign_ties(key_times, t, key_rot, rel=1e-6):
    """Primitives whose keyframe quaternions are nearly orthogonal: the shorter-arc
    sign is a near tie there (either choice is within rounding of correct)."""
    k, k1, _ = bracket(key_times, t)
    q0, q1 = np.asarray(key_rot[k], np.float64), np.asarray(key_rot[k1], np.float64)
    dot = (q0 * q1).sum(1)
    return np.abs(dot) <= rel * np.linalg.norm(q0, axis=1) * np.linalg.norm(q1, axis=1)

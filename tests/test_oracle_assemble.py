"""Pins of the parameter-assembly oracle (CPU only): keyframe and clamp cases,
the segment and the midpoint, the shorter-arc sign as a rotation identity, the
textbook slerp midpoint, and the backward against central differences."""
import math

import numpy as np
import pytest

from oracle import assemble as A


def _quat_to_mat(q):
    w, x, y, z = q / np.linalg.norm(q)
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                     [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                     [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def _keys(rng, K=4, n=50):
    times = np.cumsum(rng.uniform(0.1, 1.0, K))
    pos = rng.standard_normal((K, n, 3))
    rot = rng.standard_normal((K, n, 4))
    return times, pos, rot


def test_keyframes_and_clamping():
    rng = np.random.default_rng(1)
    times, pos, rot = _keys(rng)
    for k in range(len(times)):
        p, q = A.interpolate(times, times[k], pos, rot)
        np.testing.assert_array_equal(p, pos[k])
        s = np.sign((rot[k] * rot[k]).sum(1))[:, None]          # +1: q . q > 0
        np.testing.assert_array_equal(q, rot[k] * s)
    p, q = A.interpolate(times, times[0] - 5.0, pos, rot)
    np.testing.assert_array_equal(p, pos[0])
    p, q = A.interpolate(times, times[-1] + 5.0, pos, rot)
    np.testing.assert_array_equal(p, pos[-1])
    p, q = A.interpolate(times[:1], 3.0, pos[:1], rot[:1])
    np.testing.assert_array_equal(p, pos[0])


def test_centre_runs_along_the_segment():
    rng = np.random.default_rng(2)
    times, pos, rot = _keys(rng)
    t = 0.3 * times[1] + 0.7 * times[2]
    p, _ = A.interpolate(times, t, pos, rot)
    # p - c_1 is parallel to c_2 - c_1 with ratio 0.7
    np.testing.assert_allclose(p - pos[1], 0.7 * (pos[2] - pos[1]), rtol=1e-12, atol=1e-12)
    mid, _ = A.interpolate(times, 0.5 * (times[0] + times[1]), pos, rot)
    np.testing.assert_allclose(mid, 0.5 * (pos[0] + pos[1]), rtol=1e-12, atol=1e-15)


def test_rotation_midpoint_is_the_slerp_midpoint_on_the_shorter_arc():
    """For unit q0, q1 with q0.q1 >= 0 the slerp midpoint is (q0 + q1)/|q0 + q1|; the
    interpolated rotation equals it after normalisation, and flipping q1 to -q1 (the
    same rotation) changes nothing."""
    rng = np.random.default_rng(3)
    times = np.array([0.0, 2.0])
    n = 40
    q0 = rng.standard_normal((n, 4))
    q0 /= np.linalg.norm(q0, axis=1, keepdims=True)
    q1 = rng.standard_normal((n, 4))
    q1 /= np.linalg.norm(q1, axis=1, keepdims=True)
    q1 *= np.sign((q0 * q1).sum(1))[:, None]
    pos = np.zeros((2, n, 3))
    _, q = A.interpolate(times, 1.0, pos, np.stack([q0, q1]))
    # slerp at 1/2 from the angle between them
    om = np.arccos(np.clip((q0 * q1).sum(1), -1, 1))[:, None]
    slerp = (np.sin(0.5 * om) * q0 + np.sin(0.5 * om) * q1) / np.sin(om)
    np.testing.assert_allclose(q / np.linalg.norm(q, axis=1, keepdims=True), slerp, rtol=1e-10, atol=1e-12)
    _, qf = A.interpolate(times, 0.7, pos, np.stack([q0, -q1]))
    _, qp = A.interpolate(times, 0.7, pos, np.stack([q0, q1]))
    for i in range(n):
        np.testing.assert_allclose(_quat_to_mat(qf[i]), _quat_to_mat(qp[i]), atol=1e-12)


def test_backward_against_central_differences():
    rng = np.random.default_rng(4)
    times, pos, rot = _keys(rng, K=3, n=6)
    t = 0.25 * times[0] + 0.75 * times[1]
    gp = rng.standard_normal((6, 3))
    gq = rng.standard_normal((6, 4))

    def loss(kp, kr):
        p, q = A.interpolate(times, t, kp, kr)
        return float((p * gp).sum() + (q * gq).sum())

    dp, dq = A.interpolate_backward(times, t, rot, gp, gq)
    h = 1e-6
    for arr, grad in ((pos, dp), (rot, dq)):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            if arr is pos:
                fd[idx] = (loss(a1, rot) - loss(a2, rot)) / (2 * h)
            else:
                fd[idx] = (loss(pos, a1) - loss(pos, a2)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-7, atol=1e-8)
    assert np.abs(dp[2]).max() == 0.0 and np.abs(dq[2]).max() == 0.0     # frames not bracketing t

"""Pins of the oracle's EWA projection (orc_project, [gsplat-proj] gs_project_one) against what the mathematics
fixes: the closed form of an isotropic Gaussian on the optical axis, an independent float64 formulation of the
Jacobian projection (J W Sigma W^T J^T with the page's clipping) on random scenes, the orthographic closed form,
the conic as the inverse of the regularised covariance, the compensation as a determinant ratio, and the
visibility rules."""
import math

import numpy as np
import pytest

import oracle
from tile_binned_gaussian_amd import synth


def _cam(fx=1000.0, fy=900.0, cx=320.0, cy=240.0, R=None, t=(0.0, 0.0, 0.0)):
    v = np.eye(4, dtype=np.float32)
    if R is not None:
        v[:3, :3] = R
    v[:3, 3] = t
    K = np.array([[fx, 0, cx], [0, fy, cy], [0, 0, 1]], np.float32)
    return v[None], K[None]


def test_isotropic_on_axis_closed_form():
    z, s, eps = 5.0, 0.05, 0.3
    v, K = _cam()
    means = np.array([[0.0, 0.0, z]], np.float32)
    cov = (np.eye(3) * s * s).astype(np.float32)[None]
    pr = oracle.project(means, cov, v, K, 640, 480, eps2d=eps, compensation=True)
    fx, fy = 1000.0, 900.0
    c00, c11 = (fx / z) ** 2 * s * s, (fy / z) ** 2 * s * s
    np.testing.assert_allclose(pr.means2d[0, 0], [320.0, 240.0], rtol=0, atol=1e-4)
    assert pr.depths[0, 0] == np.float32(z)
    np.testing.assert_allclose(pr.conics[0, 0], [1 / (c00 + eps), 0.0, 1 / (c11 + eps)], rtol=1e-5, atol=1e-9)
    assert tuple(pr.radii[0, 0]) == (math.ceil(3.33 * math.sqrt(c00 + eps)), math.ceil(3.33 * math.sqrt(c11 + eps)))
    np.testing.assert_allclose(pr.compensations[0, 0], math.sqrt(c00 * c11 / ((c00 + eps) * (c11 + eps))), rtol=1e-5)


def test_orthographic_closed_form():
    v, K = _cam()
    rng = np.random.default_rng(3)
    means = rng.uniform(-1, 1, (50, 3)).astype(np.float32)
    means[:, 2] += 4.0
    A = rng.normal(size=(50, 3, 3)) * 0.05
    cov = (A @ np.transpose(A, (0, 2, 1))).astype(np.float32)
    pr = oracle.project(means, cov, v, K, 640, 480, eps2d=0.3, orthographic=True)
    fx, fy, cx, cy = 1000.0, 900.0, 320.0, 240.0
    np.testing.assert_allclose(pr.means2d[0, :, 0], means[:, 0].astype(np.float64) * fx + cx, rtol=1e-6, atol=1e-4)
    np.testing.assert_allclose(pr.means2d[0, :, 1], means[:, 1].astype(np.float64) * fy + cy, rtol=1e-6, atol=1e-4)
    c = cov.astype(np.float64)
    c00, c01, c11 = fx * fx * c[:, 0, 0] + 0.3, fx * fy * c[:, 0, 1], fy * fy * c[:, 1, 1] + 0.3
    det = c00 * c11 - c01 * c01
    np.testing.assert_allclose(pr.conics[0], np.stack([c11 / det, -c01 / det, c00 / det], -1), rtol=2e-4)


def _ewa64(sc, eps2d, near, far):
    """Float64 EWA projection written from the formula (independent of the oracle's loops)."""
    means, cov = sc.means.astype(np.float64), sc.covars.astype(np.float64)
    out = []
    for c in range(sc.C):
        V, K = sc.viewmats[c].astype(np.float64), sc.Ks[c].astype(np.float64)
        W, t = V[:3, :3], V[:3, 3]
        mc = means @ W.T + t
        cc = W[None] @ cov @ W.T[None]
        depth = mc[:, 2]
        z = np.where((depth <= near) | (depth >= far), 1.0, depth)
        fx, fy, cx, cy = K[0, 0], K[1, 1], K[0, 2], K[1, 2]
        lim_x = 0.15 * sc.width / fx
        lim_y = 0.15 * sc.height / fy
        tx = np.clip(mc[:, 0] / z, -cx / fx - lim_x, (sc.width - cx) / fx + lim_x) * z
        ty = np.clip(mc[:, 1] / z, -cy / fy - lim_y, (sc.height - cy) / fy + lim_y) * z
        J = np.zeros((len(z), 2, 3))
        J[:, 0, 0], J[:, 0, 2] = fx / z, -fx * tx / z ** 2
        J[:, 1, 1], J[:, 1, 2] = fy / z, -fy * ty / z ** 2
        c2 = J @ cc @ np.transpose(J, (0, 2, 1))
        det0 = c2[:, 0, 0] * c2[:, 1, 1] - c2[:, 0, 1] * c2[:, 1, 0]
        c2[:, 0, 0] += eps2d
        c2[:, 1, 1] += eps2d
        det = c2[:, 0, 0] * c2[:, 1, 1] - c2[:, 0, 1] * c2[:, 1, 0]
        p = np.stack([(K[0, 0] * mc[:, 0] + K[0, 1] * mc[:, 1] + K[0, 2] * z) / z,
                      (K[1, 0] * mc[:, 0] + K[1, 1] * mc[:, 1] + K[1, 2] * z) / z], -1)
        conic = np.stack([c2[:, 1, 1] / det, -c2[:, 0, 1] / det, c2[:, 0, 0] / det], -1)
        r = 3.33 * np.sqrt(np.maximum(np.stack([c2[:, 0, 0], c2[:, 1, 1]], -1), 0))
        out.append((p, depth, conic, r, np.sqrt(np.maximum(det0 / det, 0)), det))
    return out


@pytest.mark.parametrize("seed", [5, 6])
def test_matches_float64_formulation(seed):
    sc = synth.scene3d(seed, 3000, C=2, width=800, height=600)
    pr = oracle.project(sc.means, sc.covars, sc.viewmats, sc.Ks, sc.width, sc.height, eps2d=0.3,
                        near_plane=0.01, far_plane=1e10, compensation=True)
    for c, (p, depth, conic, r, comp, det) in enumerate(_ewa64(sc, 0.3, 0.01, 1e10)):
        front = depth > 0.2  # away from the camera plane, where float32 rounding is well conditioned
        np.testing.assert_allclose(pr.depths[c], depth, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(pr.means2d[c][front], p[front], rtol=1e-5, atol=2e-3)
        np.testing.assert_allclose(pr.conics[c][front], conic[front], rtol=2e-3, atol=1e-6)
        np.testing.assert_allclose(pr.compensations[c][front], comp[front], rtol=2e-3, atol=1e-5)
        # radii: ceil of the float64 value wherever it is not within rounding of an integer
        visible = pr.radii[c, :, 0] > 0
        ok = front & visible[:] & np.all(np.abs(r - np.round(r)) > 1e-3, axis=1)
        np.testing.assert_array_equal(pr.radii[c][ok], np.ceil(r[ok]).astype(np.int32))
    assert (pr.radii[..., 0] > 0).mean() > 0.2  # the scene exercises visible splats


def test_conic_inverts_regularised_covariance_and_visibility_rules():
    sc = synth.scene3d(7, 2000, C=1, width=640, height=480)
    eps, near, clip = 0.3, 0.5, 2.0
    pr = oracle.project(sc.means, sc.covars, sc.viewmats, sc.Ks, sc.width, sc.height, eps2d=eps, near_plane=near,
                        radius_clip=clip, compensation=True)
    (p, depth, conic, r, comp, det), = _ewa64(sc, eps, near, 1e10)
    vis = pr.radii[0, :, 0] > 0
    assert np.all(pr.radii[0][~vis] == 0)
    # every visible splat is in front of the near plane, larger than the clip radius and overlaps the image
    assert np.all(pr.depths[0][vis] > near)
    rr = pr.radii[0].astype(np.float64)
    assert np.all(np.maximum(rr[vis, 0], rr[vis, 1]) > clip)
    m = pr.means2d[0].astype(np.float64)
    assert np.all(m[vis, 0] + rr[vis, 0] > 0) and np.all(m[vis, 0] - rr[vis, 0] < sc.width)
    assert np.all(m[vis, 1] + rr[vis, 1] > 0) and np.all(m[vis, 1] - rr[vis, 1] < sc.height)
    # splats behind the near plane are never visible, and some exist in this scene
    assert np.any(pr.depths[0] <= near) and not np.any(vis & (pr.depths[0] <= near))
    # conic (a, b, c) is the inverse of [[c00, c01], [c01, c11]]: a c00 + b c01 = 1, b c00 + c c01 = 0 (float32)
    a, b, c = (pr.conics[0, :, i].astype(np.float64) for i in range(3))
    c00 = c / (a * c - b * b)
    c01 = -b / (a * c - b * b)
    np.testing.assert_allclose((a * c00 + b * c01)[vis], 1.0, rtol=1e-3)
    assert np.all(pr.compensations[0][vis] <= 1.0 + 1e-6) and np.all(pr.compensations[0] >= 0)


def test_degenerate_covariance_is_invisible_with_safe_conic():
    v, K = _cam()
    means = np.array([[0.0, 0.0, 3.0]], np.float32)
    cov = np.zeros((1, 3, 3), np.float32)  # a point: cov2d = eps I only
    pr = oracle.project(means, cov, v, K, 640, 480, eps2d=0.0, compensation=True)
    assert tuple(pr.radii[0, 0]) == (0, 0)  # det = 0 -> invisible
    np.testing.assert_array_equal(pr.conics[0, 0], np.float32([0.0, -0.0, 0.0]))  # divided by the 1e-10 floor
    assert pr.compensations[0, 0] == 0.0

"""GPU parity of the EWA projection (gs_project_fwd) with the oracle's orc_project on seeded 3D scenes: both evaluate
the page's float32 operations in the same order without contraction, so every output is compared bit for bit
(radii as integers, the float outputs by their bit patterns)."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, synth

from gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _compare(sc, **kw):
    o = oracle.project(sc.means, sc.covars, sc.viewmats, sc.Ks, sc.width, sc.height, **kw)
    g = binding.gs_project_fwd(dev(sc.means), dev(sc.covars), dev(sc.viewmats), dev(sc.Ks), sc.width, sc.height,
                               **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(g.radii), o.radii)
    for name in ("means2d", "depths", "conics"):
        np.testing.assert_array_equal(_bits(host(getattr(g, name))), _bits(getattr(o, name)), err_msg=name)
    if kw.get("compensation"):
        np.testing.assert_array_equal(_bits(host(g.compensations)), _bits(o.compensations))
    return g, o


CASES = {
    "one-camera": (lambda: synth.scene3d(11, 5000, C=1, width=800, height=600), {}),
    "four-cameras-compensation": (lambda: synth.scene3d(12, 3000, C=4, width=640, height=480),
                                  {"compensation": True}),
    "orthographic": (lambda: synth.scene3d(13, 2000, C=2, width=512, height=512),
                     {"orthographic": True, "compensation": True}),
    "near-far-clip": (lambda: synth.scene3d(14, 4000, C=2, width=700, height=500, behind_frac=0.2),
                      {"near_plane": 2.0, "far_plane": 9.0, "radius_clip": 3.0, "eps2d": 0.1}),
    "wide-spread": (lambda: synth.scene3d(15, 4000, C=3, width=300, height=200, spread=12.0, scale_sigma_ln=2.0),
                    {"compensation": True}),
    "ragged-count": (lambda: synth.scene3d(16, 257, C=1, width=100, height=80), {}),
    "empty": (lambda: synth.scene3d(17, 0, C=2, width=64, height=64), {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_projection_bit_exact(name):
    make, kw = CASES[name]
    _compare(make(), **kw)


def test_projection_degenerate_and_extreme_covariances():
    sc = synth.scene3d(18, 600, C=1, width=400, height=300)
    sc.covars[:100] = 0.0  # points: det from eps2d only
    sc.covars[100:200] *= 1e-12  # tiny
    sc.covars[200:300] *= 1e6  # huge: radii far beyond the image
    sc.covars[300:350, 0, 1] = sc.covars[300:350, 1, 0] = 10.0  # indefinite
    _compare(sc, eps2d=0.0, compensation=True)
    _compare(sc, eps2d=0.3, compensation=True)


def test_projection_one_million_bit_exact():
    sc = synth.scene3d(19, 1_000_000, C=1, width=1920, height=1080)
    g, o = _compare(sc, compensation=True)
    assert (o.radii[..., 0] > 0).mean() > 0.2

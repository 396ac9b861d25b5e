"""GPU parity of the composite's backward (gs_rasterize_bwd) against the oracle's orc_rasterize_bwd on the same
seeded inputs and the same forward outputs.

Each gradient term is computed by both sides with the same float32 operations in the same order; only the order in
which a splat's terms are summed differs (the oracle sums them exactly in double; the GPU sums each 16-lane row of a
wavefront with a 4-level tree, adds the row sums into a per-tile LDS accumulator, then adds one partial sum per
(splat, tile) with float atomics). Float summation of terms t_i with at most L additions on any path errs by at
most L * 2^-24 * sum|t_i|, so each entry is checked against |gpu - oracle| <= (6 + A + 2) * 2^-24 * sum|t_i|, with
A = 4 x (wavefronts per tile) x (the splat's tile count) partial sums that can reach the entry, and sum|t_i| from
the oracle."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, synth

from gpu_util import dev, gpu_frame, host, require_gpu
from test_gpu_parity import SCENES

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _grads_in(scene, seed):
    rng = np.random.default_rng(seed)
    C, H, W, K = scene.C, scene.height, scene.width, scene.colors.shape[-1]
    return (rng.normal(size=(C, H, W, K)).astype(np.float32), rng.normal(size=(C, H, W)).astype(np.float32))


def _waves_per_tile(ts):
    return max(1, (ts * ts + 63) // 64)


def _assert_close(g, o, abs_sum, adds, what):
    bound = (6.0 + adds + 2.0) * U * abs_sum + 1e-30
    err = np.abs(g.astype(np.float64) - o)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries off; worst err {err[bad].max():.3e} vs bound "
                           f"{bound[bad][np.argmax(err[bad])]:.3e}")


def run_and_compare(scene, seed=0, absgrad=True):
    fr = gpu_frame(scene)
    off, ids, n = fr.isect_offsets, fr.isect.flatten_ids, fr.isect.n_isects
    gc, ga = _grads_in(scene, seed)
    ras_a, last = host(fr.render.render_alphas), host(fr.render.last_ids)
    o = oracle.rasterize_bwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                             scene.width, scene.height, scene.tile_size, host(off), host(ids), n,
                             scene.alpha_cutoff, scene.alpha_clamp, ras_a, last, gc, ga)
    m = lambda a: dev(a)  # noqa: E731
    g = binding.gs_rasterize_bwd(m(scene.means2d), m(scene.conics), m(scene.colors), m(scene.opacities),
                                 None if scene.backgrounds is None else m(scene.backgrounds), scene.width,
                                 scene.height, scene.tile_size, off, ids, fr.render.render_alphas,
                                 fr.render.last_ids, m(gc), m(ga), n_isects=n, alpha_cutoff=scene.alpha_cutoff,
                                 alpha_clamp=scene.alpha_clamp, absgrad=absgrad)
    torch.cuda.synchronize()
    tiles = host(fr.isect.tiles_per_gauss).astype(np.float64)
    adds = tiles * 4 * _waves_per_tile(scene.tile_size)
    _assert_close(host(g.means2d), o.means2d, o.abs_means2d, adds[..., None], "means2d")
    _assert_close(host(g.conics), o.conics, o.abs_conics, adds[..., None], "conics")
    _assert_close(host(g.colors), o.colors, o.abs_colors, adds[..., None], "colors")
    _assert_close(host(g.opacities), o.opacities, o.abs_opacities, adds, "opacities")
    if scene.backgrounds is not None:
        pixels_adds = scene.tile_width * scene.tile_height * _waves_per_tile(scene.tile_size)
        _assert_close(host(g.backgrounds), o.backgrounds, o.abs_backgrounds, pixels_adds, "backgrounds")
    if absgrad:
        _assert_close(host(g.means2d_abs), o.means2d_abs, o.means2d_abs, adds[..., None], "means2d_abs")
    # the gradients are not trivially zero where the oracle's are not
    assert (np.abs(o.means2d) > 0).sum() == 0 or (np.abs(host(g.means2d)) > 0).any()
    return g, o


BWD_SCENES = ["tiny", "tiny-aniso", "cull-edges", "multicam-ragged-elliptical", "ts8-margin", "ts32-ppt4", "ts1",
              "dense-early-out", "deep-tiles", "single-tile", "all-equal-keys", "zero-radius", "one-isect", "empty",
              "K1", "K2", "K4"]


@pytest.mark.parametrize("name", BWD_SCENES)
def test_backward_matches_oracle(name):
    run_and_compare(SCENES[name](), seed=len(name))


def test_backward_config2_full():
    run_and_compare(synth.config2(), seed=2)


def test_backward_without_background_gradient_or_abs():
    s = SCENES["multicam-ragged-elliptical"]()
    fr = gpu_frame(s)
    gc, ga = _grads_in(s, 5)
    m = lambda a: dev(a)  # noqa: E731
    full = binding.gs_rasterize_bwd(m(s.means2d), m(s.conics), m(s.colors), m(s.opacities), m(s.backgrounds),
                                    s.width, s.height, s.tile_size, fr.isect_offsets, fr.isect.flatten_ids,
                                    fr.render.render_alphas, fr.render.last_ids, m(gc), m(ga), absgrad=True)
    lean = binding.gs_rasterize_bwd(m(s.means2d), m(s.conics), m(s.colors), m(s.opacities), m(s.backgrounds),
                                    s.width, s.height, s.tile_size, fr.isect_offsets, fr.isect.flatten_ids,
                                    fr.render.render_alphas, fr.render.last_ids, m(gc), m(ga),
                                    grad_backgrounds=False)
    torch.cuda.synchronize()
    assert lean.backgrounds is None and lean.means2d_abs is None
    # same terms, same per-wave sums: only the atomics' order may differ between the two launches
    for a, b in [(full.means2d, lean.means2d), (full.conics, lean.conics), (full.colors, lean.colors),
                 (full.opacities, lean.opacities)]:
        torch.testing.assert_close(a, b, rtol=1e-5, atol=1e-6)
    # written, not accumulated: a second launch into the same arrays gives the same values
    again = binding.gs_rasterize_bwd(m(s.means2d), m(s.conics), m(s.colors), m(s.opacities), m(s.backgrounds),
                                     s.width, s.height, s.tile_size, fr.isect_offsets, fr.isect.flatten_ids,
                                     fr.render.render_alphas, fr.render.last_ids, m(gc), m(ga), absgrad=True,
                                     out=full)
    torch.cuda.synchronize()
    torch.testing.assert_close(again.means2d, lean.means2d, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("name", ["multicam-ragged-elliptical", "ts8-margin", "ts32-ppt4"])
def test_masked_backward_matches_oracle(name):
    scene = SCENES[name]()
    fr = gpu_frame(scene)
    off, ids, n = fr.isect_offsets, fr.isect.flatten_ids, fr.isect.n_isects
    masks = (np.random.default_rng(len(name) + 7).uniform(size=tuple(off.shape)) < 0.6).astype(np.int32)
    m = lambda a: dev(a)  # noqa: E731
    bg = None if scene.backgrounds is None else m(scene.backgrounds)
    ren = binding.gs_rasterize_fwd(m(scene.means2d), m(scene.conics), m(scene.colors), m(scene.opacities), bg,
                                   scene.width, scene.height, scene.tile_size, off, ids, n, scene.alpha_cutoff,
                                   scene.alpha_clamp, scene.transmittance_threshold, masks=m(masks))
    gc, ga = _grads_in(scene, 9)
    o = oracle.rasterize_bwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                             scene.width, scene.height, scene.tile_size, host(off), host(ids), n,
                             scene.alpha_cutoff, scene.alpha_clamp, host(ren.render_alphas), host(ren.last_ids), gc,
                             ga, masks=masks)
    g = binding.gs_rasterize_bwd(m(scene.means2d), m(scene.conics), m(scene.colors), m(scene.opacities), bg,
                                 scene.width, scene.height, scene.tile_size, off, ids, ren.render_alphas,
                                 ren.last_ids, m(gc), m(ga), n_isects=n, alpha_cutoff=scene.alpha_cutoff,
                                 alpha_clamp=scene.alpha_clamp, masks=m(masks))
    torch.cuda.synchronize()
    adds = host(fr.isect.tiles_per_gauss).astype(np.float64) * 4 * _waves_per_tile(scene.tile_size)
    _assert_close(host(g.means2d), o.means2d, o.abs_means2d, adds[..., None], "means2d")
    _assert_close(host(g.conics), o.conics, o.abs_conics, adds[..., None], "conics")
    _assert_close(host(g.opacities), o.opacities, o.abs_opacities, adds, "opacities")
    if scene.backgrounds is not None:
        pixels_adds = scene.tile_width * scene.tile_height * _waves_per_tile(scene.tile_size)
        _assert_close(host(g.backgrounds), o.backgrounds, o.abs_backgrounds, pixels_adds, "backgrounds")

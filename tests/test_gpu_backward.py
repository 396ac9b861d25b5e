"""GPU parity of the composite's backward (gs_rasterize_bwd) against the oracle's exact gradient.

Both sides start from the same seeded scene and output gradients, and each from its own forward: the GPU backward
reads the GPU forward's render_alphas and last_ids, the oracle's backward the oracle forward's (the two forwards are
checked equal bit for bit first). The oracle evaluates the exact gradient in double (front-to-back transmittances,
suffix sums); the GPU evaluates the backward page's float32 recurrence (gsplat 1.0.0 raster_backward.c,
gs_raster_backward_pixel: transmittance rebuilt back to front from 1 - render_alpha by divisions) and sums each
splat's terms over 16-lane rows, LDS accumulators per tile and one float atomic per (splat, tile). The bar per
entry is the oracle's derived bound: err (the float32 recurrence's rounding of every term, phi = (8 L + K + 12) u +
u / T_final per pixel) plus (D + 2) u times the sum of the terms' magnitudes for a float sum of depth
D = 6 + 4 x (wavefronts per tile) x (the splat's tile count), widened by 2%."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, synth

from gpu_util import assert_raster_equal, dev, gpu_frame, host, oracle_frame, oracle_lists, require_gpu
from test_gpu_parity import SCENES

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def grads_in(scene, seed):
    rng = np.random.default_rng(seed)
    C, H, W, K = scene.C, scene.height, scene.width, scene.colors.shape[-1]
    return (rng.normal(size=(C, H, W, K)).astype(np.float32), rng.normal(size=(C, H, W)).astype(np.float32))


def waves_per_tile(ts):
    return max(1, (ts * ts + 63) // 64)


def summation_depth(scene, it_o):
    """Additions on any path of one splat's float sum on the GPU (per [C, N] splat)."""
    return 6.0 + 4.0 * waves_per_tile(scene.tile_size) * it_o.tiles_per_gauss.astype(np.float64)


def assert_within(g, o, field, adds):
    """|GPU - exact| within the oracle's derived bound for one gradient output."""
    gpu = host(getattr(g, field)).astype(np.float64)
    want = getattr(o, field)
    a = np.asarray(adds, np.float64)
    while a.ndim < want.ndim:
        a = a[..., None]
    if field == "means2d_abs":
        bound = 1.02 * (o.err_means2d + (a + 2.0) * U * o.means2d_abs) + 1e-30
    else:
        bound = o.bound(field, a)
    err = np.abs(gpu - want)
    bad = err > bound
    assert not bad.any(), (f"{field}: {int(bad.sum())} entries off; worst err {err[bad].max():.3e} vs bound "
                           f"{bound[bad][np.argmax(err[bad])]:.3e}")
    return float((err / bound).max()) if err.size else 0.0


def _gpu_bwd(scene, fr, gc, ga, absgrad=True, masks=None, ren=None):
    ren = ren if ren is not None else fr.render
    bg = None if scene.backgrounds is None else dev(scene.backgrounds)
    g = binding.gs_rasterize_bwd(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities), bg,
                                 scene.width, scene.height, scene.tile_size, fr.isect_offsets, fr.isect.flatten_ids,
                                 ren.render_alphas, ren.last_ids, dev(gc), dev(ga), n_isects=fr.isect.n_isects,
                                 alpha_cutoff=scene.alpha_cutoff, alpha_clamp=scene.alpha_clamp, absgrad=absgrad,
                                 masks=None if masks is None else dev(masks))
    torch.cuda.synchronize()
    return g


def _check_all(scene, g, o, it_o, absgrad=True):
    adds = summation_depth(scene, it_o)
    worst = 0.0
    for field in ("means2d", "conics", "colors", "opacities"):
        worst = max(worst, assert_within(g, o, field, adds))
    if scene.backgrounds is not None:
        worst = max(worst, assert_within(g, o, "backgrounds",
                                         6.0 + scene.tile_width * scene.tile_height * waves_per_tile(scene.tile_size)))
    if absgrad:
        worst = max(worst, assert_within(g, o, "means2d_abs", adds))
    return worst


def run_and_compare(scene, seed=0, absgrad=True):
    it_o, off_o, ras_o = oracle_frame(scene)
    fr = gpu_frame(scene)
    assert_raster_equal(scene, fr, ras_o, it_o.flatten_ids)
    gc, ga = grads_in(scene, seed)
    o = oracle.rasterize_bwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                             scene.width, scene.height, scene.tile_size, off_o, it_o.flatten_ids, it_o.n_isects,
                             scene.alpha_cutoff, scene.alpha_clamp, ras_o.render_alphas, ras_o.last_ids, gc, ga)
    g = _gpu_bwd(scene, fr, gc, ga, absgrad)
    _check_all(scene, g, o, it_o, absgrad)
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
    gc, ga = grads_in(s, 5)
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


def _masked_compare(scene, masks, seed):
    it_o, off_o, ras_o = oracle_frame(scene, masks=masks)
    fr = gpu_frame(scene)
    bg = None if scene.backgrounds is None else dev(scene.backgrounds)
    ren = binding.gs_rasterize_fwd(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities), bg,
                                   scene.width, scene.height, scene.tile_size, fr.isect_offsets, fr.isect.flatten_ids,
                                   fr.isect.n_isects, scene.alpha_cutoff, scene.alpha_clamp,
                                   scene.transmittance_threshold, masks=dev(masks))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ren.render_colors), ras_o.render_colors)
    np.testing.assert_array_equal(host(ren.render_T), ras_o.render_T)
    gc, ga = grads_in(scene, seed)
    o = oracle.rasterize_bwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                             scene.width, scene.height, scene.tile_size, off_o, it_o.flatten_ids, it_o.n_isects,
                             scene.alpha_cutoff, scene.alpha_clamp, ras_o.render_alphas, ras_o.last_ids, gc, ga,
                             masks=masks)
    g = _gpu_bwd(scene, fr, gc, ga, True, masks=masks, ren=ren)
    return _check_all(scene, g, o, it_o), o


@pytest.mark.parametrize("name", ["multicam-ragged-elliptical", "ts8-margin", "ts32-ppt4"])
def test_masked_backward_matches_oracle(name):
    scene = SCENES[name]()
    shape = (scene.C, scene.tile_height, scene.tile_width)
    masks = (np.random.default_rng(len(name) + 7).uniform(size=shape) < 0.6).astype(np.int32)
    _masked_compare(scene, masks, 9)


def test_backward_1m_splats_1080p_on_masked_tiles():
    """The 1M-splat 1920x1080 frame, restricted on both sides (the page's per-tile masks) to a seeded 2% of the
    tiles plus the 16 with the longest lists, so that the single-threaded oracle stays quick; every gradient entry
    of every splat is compared (splats outside the kept tiles get exactly zero on both sides)."""
    scene = synth.config3()
    it_o, off_o = oracle_lists(scene)
    flat = off_o.reshape(-1).astype(np.int64)
    lengths = np.diff(np.append(flat, it_o.n_isects))
    rng = np.random.default_rng(103)
    keep = rng.uniform(size=flat.size) < 0.02
    keep[np.argsort(-lengths, kind="stable")[:16]] = True
    masks = keep.reshape(off_o.shape).astype(np.int32)
    print(f"\n1M backward: {int(keep.sum())} of {keep.size} tiles kept", flush=True)
    worst, o = _masked_compare(scene, masks, 104)
    assert (np.abs(o.means2d) > 0).sum() > 10_000  # a real share of the splats is compared
    print(f"worst error / bound: {worst:.3g}", flush=True)

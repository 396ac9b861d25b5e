"""Pins of the oracle's composite backward (orc_rasterize_bwd, [gsplat-bwd] gs_raster_backward_pixel) against what
the mathematics fixes: closed-form gradients for one and two splats at one pixel, central finite differences of an
independent float64 forward on small scenes (away from the cutoff, clamp and early-out events, where the composite is
smooth), and the background gradient's closed form."""
import math

import numpy as np
import pytest

import oracle
from tile_binned_gaussian_amd import synth

CUT = float(np.float32(1.0) / np.float32(255.0))


def _one_pixel_scene(means, conics, colors, opacities, depths, background, K=3):
    n = len(opacities)
    s = synth.random_scene(0, 1, n, 1, 1, 16, channels=K, background=True)
    s.means2d[0] = np.float32(means)
    s.conics[0] = np.float32(conics)
    s.colors[0] = np.float32(colors)
    s.opacities[0] = np.float32(opacities)
    s.depths[0] = np.float32(depths)
    s.radii[0] = np.float32(8.0)
    s.backgrounds[0] = np.float32(background)
    return s


def _run(scene, gc, ga):
    it, off, ras = oracle.scene_pipeline(scene)
    return oracle.rasterize_bwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                                scene.width, scene.height, scene.tile_size, off, it.flatten_ids, it.n_isects,
                                scene.alpha_cutoff, scene.alpha_clamp, ras.render_alphas, ras.last_ids, gc, ga), ras


def _alpha_terms(mean, conic, opacity):
    """Double-precision alpha and its partial derivatives at the pixel centre (0.5, 0.5)."""
    dx, dy = float(np.float32(mean[0])) - 0.5, float(np.float32(mean[1])) - 0.5
    a, b, c = (float(np.float32(v)) for v in conic)
    o = float(np.float32(opacity))
    sigma = 0.5 * (a * dx * dx + c * dy * dy) + b * dx * dy
    e = math.exp(-sigma)
    alpha = o * e
    # d alpha / d(param): alpha depends on mean through sigma, d sigma/d mean = (a dx + b dy, c dy + b dx)
    d = {"o": e, "mx": -alpha * (a * dx + b * dy), "my": -alpha * (c * dy + b * dx),
         "a": -alpha * 0.5 * dx * dx, "b": -alpha * dx * dy, "c": -alpha * 0.5 * dy * dy}
    return alpha, d


def test_one_splat_closed_form():
    rng = np.random.default_rng(5)
    mean, conic, col, o = [0.9, 0.1], [0.8, 0.15, 0.6], rng.uniform(0, 1, 3), 0.7
    bg = rng.uniform(0, 1, 3)
    s = _one_pixel_scene([mean], [conic], [col], [o], [2.0], bg)
    gc = rng.normal(size=(1, 1, 1, 3)).astype(np.float32)
    ga = rng.normal(size=(1, 1, 1)).astype(np.float32)
    g, ras = _run(s, gc, ga)
    alpha, d = _alpha_terms(mean, conic, o)
    gcv, gav = gc.reshape(3).astype(np.float64), float(ga.reshape(()))
    colv = np.float32(col).astype(np.float64)
    bgv = np.float32(bg).astype(np.float64)
    # C = alpha col + (1 - alpha) bg, A = alpha
    dl_dalpha = float(gcv @ (colv - bgv)) + gav
    np.testing.assert_allclose(g.colors[0, 0], gcv * alpha, rtol=2e-5, atol=1e-7)
    np.testing.assert_allclose(g.backgrounds[0], gcv * (1 - alpha), rtol=2e-5, atol=1e-7)
    np.testing.assert_allclose(g.opacities[0, 0], dl_dalpha * d["o"], rtol=2e-5, atol=1e-7)
    np.testing.assert_allclose(g.means2d[0, 0], [dl_dalpha * d["mx"], dl_dalpha * d["my"]], rtol=2e-5, atol=1e-7)
    np.testing.assert_allclose(g.conics[0, 0], [dl_dalpha * d["a"], dl_dalpha * d["b"], dl_dalpha * d["c"]],
                               rtol=2e-5, atol=1e-7)
    np.testing.assert_allclose(g.means2d_abs[0, 0], np.abs(g.means2d[0, 0]), rtol=1e-12)


def test_two_splats_closed_form():
    rng = np.random.default_rng(6)
    means, conics = [[0.3, 0.9], [1.4, -0.2]], [[0.5, -0.1, 0.9], [1.2, 0.3, 0.4]]
    cols, ops = rng.uniform(0, 1, (2, 3)), [0.6, 0.8]
    bg = rng.uniform(0, 1, 3)
    s = _one_pixel_scene(means, conics, cols, ops, [1.0, 3.0], bg)  # splat 0 in front
    gc = rng.normal(size=(1, 1, 1, 3)).astype(np.float32)
    ga = rng.normal(size=(1, 1, 1)).astype(np.float32)
    g, ras = _run(s, gc, ga)
    a1, d1 = _alpha_terms(means[0], conics[0], ops[0])
    a2, d2 = _alpha_terms(means[1], conics[1], ops[1])
    c1, c2 = (np.float32(c).astype(np.float64) for c in cols)
    bgv = np.float32(bg).astype(np.float64)
    gcv, gav = gc.reshape(3).astype(np.float64), float(ga.reshape(()))
    # C = a1 c1 + (1 - a1) a2 c2 + (1 - a1)(1 - a2) bg,  A = 1 - (1 - a1)(1 - a2)
    dl_da1 = float(gcv @ (c1 - a2 * c2 - (1 - a2) * bgv)) + gav * (1 - a2)
    dl_da2 = float(gcv @ ((1 - a1) * c2 - (1 - a1) * bgv)) + gav * (1 - a1)
    np.testing.assert_allclose(g.colors[0, 0], gcv * a1, rtol=2e-5, atol=1e-7)
    np.testing.assert_allclose(g.colors[0, 1], gcv * (1 - a1) * a2, rtol=2e-5, atol=1e-7)
    np.testing.assert_allclose(g.backgrounds[0], gcv * (1 - a1) * (1 - a2), rtol=2e-5, atol=1e-7)
    for j, (dl, d) in enumerate([(dl_da1, d1), (dl_da2, d2)]):
        np.testing.assert_allclose(g.opacities[0, j], dl * d["o"], rtol=5e-5, atol=1e-7)
        np.testing.assert_allclose(g.means2d[0, j], [dl * d["mx"], dl * d["my"]], rtol=5e-5, atol=1e-7)
        np.testing.assert_allclose(g.conics[0, j], [dl * d["a"], dl * d["b"], dl * d["c"]], rtol=5e-5, atol=1e-7)


def _smooth_scene(seed, n=6, W=20, H=18, ts=8, K=3):
    """Splats with moderate opacity and sizes, so that no alpha sits near the cutoff or the clamp and no pixel
    reaches the transmittance threshold (the composite is smooth in every parameter there)."""
    rng = np.random.default_rng(seed)
    s = synth.random_scene(seed, 1, n, W, H, ts, channels=K, background=True)
    s.means2d[0] = rng.uniform([2, 2], [W - 2, H - 2], (n, 2)).astype(np.float32)
    l1 = rng.uniform(4.0, 16.0, n)
    l2 = l1 * rng.uniform(0.4, 1.0, n)
    th = rng.uniform(0, np.pi, n)
    cs, sn = np.cos(th), np.sin(th)
    sxx, syy, sxy = l1 * cs * cs + l2 * sn * sn, l1 * sn * sn + l2 * cs * cs, (l1 - l2) * cs * sn
    det = l1 * l2
    s.conics[0] = np.stack([syy / det, -sxy / det, sxx / det], -1).astype(np.float32)
    s.radii[0] = np.float32(40.0)  # every splat touches every tile: lists do not depend on the means
    s.opacities[0] = rng.uniform(0.3, 0.7, n).astype(np.float32)
    s.depths[0] = rng.permutation(n).astype(np.float32) + 1
    return s


def _forward64(s, lists, params, max_steps=None):
    """Independent float64 forward over fixed per-tile lists: returns colour [C,H,W,K] and alpha [C,H,W].
    max_steps: stop each pixel after that many composited splats."""
    means, conics, colors, ops, bg = params
    C, H, W, K, ts = s.C, s.height, s.width, s.colors.shape[-1], s.tile_size
    out = np.zeros((C, H, W, K))
    alp = np.zeros((C, H, W))
    for y in range(H):
        for x in range(W):
            t = (y // ts) * s.tile_width + x // ts
            T, acc, steps = 1.0, np.zeros(K), 0
            for g in lists[t]:
                if max_steps is not None and steps >= max_steps:
                    break
                dx, dy = means[0, g, 0] - (x + 0.5), means[0, g, 1] - (y + 0.5)
                a, b, c = conics[0, g]
                sigma = 0.5 * (a * dx * dx + c * dy * dy) + b * dx * dy
                if sigma < 0:
                    continue
                al = min(s.alpha_clamp, ops[0, g] * math.exp(-sigma))
                if al < CUT:
                    continue
                tn = T * (1 - al)
                if tn <= s.transmittance_threshold:
                    break
                acc += colors[0, g] * al * T
                T = tn
                steps += 1
            out[0, y, x] = acc + T * bg[0]
            alp[0, y, x] = 1 - T
    return out, alp


@pytest.mark.parametrize("seed", [11, 12])
def test_finite_differences(seed):
    s = _smooth_scene(seed)
    it, off, ras = oracle.scene_pipeline(s)
    flat = off.reshape(-1).astype(np.int64)
    ends = np.append(flat[1:], it.n_isects)
    lists = [it.flatten_ids[flat[t]:ends[t]] for t in range(flat.size)]
    rng = np.random.default_rng(seed + 100)
    gc = rng.normal(size=ras.render_colors.shape).astype(np.float32)
    ga = rng.normal(size=ras.render_alphas.shape).astype(np.float32)
    g = oracle.rasterize_bwd(s.means2d, s.conics, s.colors, s.opacities, s.backgrounds, s.width, s.height,
                             s.tile_size, off, it.flatten_ids, it.n_isects, s.alpha_cutoff, s.alpha_clamp,
                             ras.render_alphas, ras.last_ids, gc, ga)
    base = [s.means2d.astype(np.float64), s.conics.astype(np.float64), s.colors.astype(np.float64),
            s.opacities.astype(np.float64), s.backgrounds.astype(np.float64)]
    out, alp = _forward64(s, lists, base)
    assert alp.max() < 1 - 1e-3  # far from the early-out threshold
    # the float64 forward reproduces the oracle's float32 forward closely (same lists, same rule)
    np.testing.assert_allclose(out, ras.render_colors, atol=1e-5)

    def loss(params):
        o, a = _forward64(s, lists, params)
        return float((gc * o).sum() + (ga * a).sum())

    grads = [g.means2d, g.conics, g.colors, g.opacities, g.backgrounds]
    for which, grad in enumerate(grads):
        fd = np.zeros_like(base[which])
        for idx in np.ndindex(base[which].shape):
            h = 1e-5 * max(1.0, abs(base[which][idx]))
            up = [p.copy() for p in base]
            dn = [p.copy() for p in base]
            up[which][idx] += h
            dn[which][idx] -= h
            fd[idx] = (loss(up) - loss(dn)) / (2 * h)
        scale = np.abs(fd).max()
        np.testing.assert_allclose(grad, fd, rtol=2e-3, atol=2e-4 * scale, err_msg=f"parameter group {which}")


def test_background_gradient_is_sum_of_transmittance():
    s = synth.random_scene(21, 2, 300, 40, 30, 16, background=True)
    rng = np.random.default_rng(22)
    it, off, ras = oracle.scene_pipeline(s)
    gc = rng.normal(size=ras.render_colors.shape).astype(np.float32)
    ga = rng.normal(size=ras.render_alphas.shape).astype(np.float32)
    g = oracle.rasterize_bwd(s.means2d, s.conics, s.colors, s.opacities, s.backgrounds, s.width, s.height,
                             s.tile_size, off, it.flatten_ids, it.n_isects, s.alpha_cutoff, s.alpha_clamp,
                             ras.render_alphas, ras.last_ids, gc, ga)
    # dL/d bg = sum over pixels of g * T_final; the forward's float32 T agrees with the exact product of
    # (1 - alpha) within the oracle's own error bound for that term
    T = ras.render_T.astype(np.float64)
    terms = gc.astype(np.float64) * T[..., None]
    want = terms.sum(axis=(1, 2))
    assert (np.abs(g.backgrounds - want) <= g.bound("backgrounds", 0)).all()
    np.testing.assert_allclose(g.abs_backgrounds, np.abs(terms).sum(axis=(1, 2)), rtol=1e-5)
    # not trivially loose: the bound is a small fraction of the magnitude
    assert (g.err_backgrounds < 1e-3 * g.abs_backgrounds).all()


def test_uncovered_pixels_and_untouched_splats_give_nothing():
    s = synth.random_scene(23, 1, 40, 64, 64, 16, background=False)
    s.radii[0, :20] = 0  # no tiles: never composited
    it, off, ras = oracle.scene_pipeline(s)
    rng = np.random.default_rng(24)
    gc = rng.normal(size=ras.render_colors.shape).astype(np.float32)
    ga = rng.normal(size=ras.render_alphas.shape).astype(np.float32)
    g = oracle.rasterize_bwd(s.means2d, s.conics, s.colors, s.opacities, None, s.width, s.height, s.tile_size,
                             off, it.flatten_ids, it.n_isects, s.alpha_cutoff, s.alpha_clamp, ras.render_alphas,
                             ras.last_ids, gc, ga)
    assert g.backgrounds is None
    for arr in (g.means2d, g.conics, g.colors, g.opacities, g.abs_means2d):
        assert np.all(arr[0, :20] == 0)
    # where nothing was composited the pixel contributes nothing: zero its gradients and compare
    gc2, ga2 = gc.copy(), ga.copy()
    empty = ras.last_ids < 0
    gc2[empty] = 0
    ga2[empty] = 0
    g2 = oracle.rasterize_bwd(s.means2d, s.conics, s.colors, s.opacities, None, s.width, s.height, s.tile_size,
                              off, it.flatten_ids, it.n_isects, s.alpha_cutoff, s.alpha_clamp, ras.render_alphas,
                              ras.last_ids, gc2, ga2)
    for a, b in [(g.means2d, g2.means2d), (g.conics, g2.conics), (g.colors, g2.colors),
                 (g.opacities, g2.opacities)]:
        np.testing.assert_array_equal(a, b)


def test_clamped_splat_has_no_shape_or_opacity_gradient():
    """alpha = clamp does not depend on opacity, mean or conic: only colour and background receive gradient
    (C = clamp col + (1 - clamp) bg)."""
    rng = np.random.default_rng(7)
    col, bg = rng.uniform(0, 1, 3), rng.uniform(0, 1, 3)
    s = _one_pixel_scene([[0.5, 0.5]], [[0.4, 0.05, 0.3]], [col], [1.0], [1.5], bg)  # raw alpha = 1 > 0.99
    gc = rng.normal(size=(1, 1, 1, 3)).astype(np.float32)
    ga = rng.normal(size=(1, 1, 1)).astype(np.float32)
    g, ras = _run(s, gc, ga)
    clamp = float(np.float32(0.99))
    assert ras.render_alphas.reshape(()) == np.float32(clamp)
    gcv = gc.reshape(3).astype(np.float64)
    np.testing.assert_allclose(g.colors[0, 0], gcv * clamp, rtol=1e-6)
    np.testing.assert_allclose(g.backgrounds[0], gcv * float(np.float32(1) - np.float32(clamp)), rtol=1e-5)
    assert np.all(g.opacities == 0) and np.all(g.means2d == 0) and np.all(g.conics == 0)


def test_masked_tiles_finite_differences_and_forward():
    """Per-tile masks: a masked tile composites nothing (background, T = 1, no last id) in the forward, and in the
    backward adds only its background terms; checked against finite differences of the float64 forward with the
    same masks applied, and the forward against the unmasked run on the other tiles."""
    s = _smooth_scene(31, W=24, H=16, ts=8)
    it, off, ras = oracle.scene_pipeline(s)
    masks = np.ones_like(off)
    masks.reshape(-1)[[0, 4]] = 0  # two of the six tiles
    rm = oracle.rasterize_fwd(s.means2d, s.conics, s.colors, s.opacities, s.backgrounds, s.width, s.height,
                              s.tile_size, off, it.flatten_ids, it.n_isects, s.alpha_cutoff, s.alpha_clamp,
                              s.transmittance_threshold, masks=masks)
    ty, tx = np.divmod(np.arange(s.height * s.width).reshape(s.height, s.width), s.width)
    tile = (ty // s.tile_size) * s.tile_width + (tx // s.tile_size)
    masked_px = masks.reshape(-1)[tile] == 0
    assert masked_px.any() and not masked_px.all()
    np.testing.assert_array_equal(rm.render_T[0][masked_px], 1.0)
    np.testing.assert_array_equal(rm.last_ids[0][masked_px], -1)
    np.testing.assert_array_equal(rm.render_colors[0][masked_px],
                                  np.broadcast_to(s.backgrounds[0], (masked_px.sum(), 3)))
    for a, b in [(rm.render_colors, ras.render_colors), (rm.render_T, ras.render_T), (rm.last_ids, ras.last_ids)]:
        np.testing.assert_array_equal(a[0][~masked_px], b[0][~masked_px])

    flat = off.reshape(-1).astype(np.int64)
    ends = np.append(flat[1:], it.n_isects)
    lists = [it.flatten_ids[flat[t]:ends[t]] if masks.reshape(-1)[t] else it.flatten_ids[:0]
             for t in range(flat.size)]
    rng = np.random.default_rng(32)
    gc = rng.normal(size=rm.render_colors.shape).astype(np.float32)
    ga = rng.normal(size=rm.render_alphas.shape).astype(np.float32)
    g = oracle.rasterize_bwd(s.means2d, s.conics, s.colors, s.opacities, s.backgrounds, s.width, s.height,
                             s.tile_size, off, it.flatten_ids, it.n_isects, s.alpha_cutoff, s.alpha_clamp,
                             rm.render_alphas, rm.last_ids, gc, ga, masks=masks)
    base = [s.means2d.astype(np.float64), s.conics.astype(np.float64), s.colors.astype(np.float64),
            s.opacities.astype(np.float64), s.backgrounds.astype(np.float64)]

    def loss(params):
        o, a = _forward64(s, lists, params)
        return float((gc * o).sum() + (ga * a).sum())

    for which, grad in enumerate([g.means2d, g.opacities, g.backgrounds]):
        idx_group = [0, 3, 4][which]
        fd = np.zeros_like(base[idx_group])
        for idx in np.ndindex(base[idx_group].shape):
            h = 1e-5 * max(1.0, abs(base[idx_group][idx]))
            up = [p.copy() for p in base]
            dn = [p.copy() for p in base]
            up[idx_group][idx] += h
            dn[idx_group][idx] -= h
            fd[idx] = (loss(up) - loss(dn)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=2e-3, atol=2e-4 * np.abs(fd).max())

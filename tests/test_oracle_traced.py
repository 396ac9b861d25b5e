"""Pins of the oracle's traced forward (orc_rasterize_fwd_traced, [rlx-metal] training_forward_metal_traced with
max_splat_steps and max_list_entries) against what the definition fixes independently of its code:

* a float64 brute force of which splats each pixel composites (the trace), away from the cutoff and early-out
  decisions;
* with no caps, the traced forward is the untraced forward to the bit;
* the list cap equals the untraced forward over lists physically cut to their first entries;
* the step cap equals the untraced composite over the pixel's list cut right after its capped last step, and the
  capped trace is a prefix of the uncapped one;
* compositing a pixel over its trace alone gives its colour and transmittance to the bit (the trace holds every
  splat that changed the pixel, and only those);
* the composite's backward evaluated on a capped forward's outputs matches finite differences of a capped float64
  forward (the trace carries nothing the range walk up to the last id does not recompute)."""
import math

import numpy as np
import pytest

import oracle
from tile_binned_gaussian_amd import synth

from test_oracle_backward import _forward64, _smooth_scene


def _traced(scene, it, off, S, L=-1, masks=None):
    return oracle.rasterize_fwd_traced(scene.means2d, scene.conics, scene.colors, scene.opacities,
                                       scene.backgrounds, scene.width, scene.height, scene.tile_size, off,
                                       it.flatten_ids, it.n_isects, scene.alpha_cutoff, scene.alpha_clamp,
                                       scene.transmittance_threshold, S, max_list_entries=L, masks=masks)


def _untraced(scene, off, ids, n):
    return oracle.rasterize_fwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                                scene.width, scene.height, scene.tile_size, off, ids, n, scene.alpha_cutoff,
                                scene.alpha_clamp, scene.transmittance_threshold)


def _tile_lists(scene, it, off):
    flat = off.reshape(-1).astype(np.int64)
    ends = np.append(flat[1:], it.n_isects)
    return flat, ends


def _pixel_tile(scene, c, y, x):
    return (c * scene.tile_height + y // scene.tile_size) * scene.tile_width + x // scene.tile_size


def test_brute_force_trace_on_a_small_scene():
    """Float64 evaluation of every (pixel, listed splat): the composited set and order, skipping pixels where any
    decision (sigma sign, cutoff, early-out) lies within a relative 1e-4 of its boundary."""
    s = synth.random_scene(41, 2, 120, 40, 28, 8, channels=3, background=True)
    it, off, _ = oracle.scene_pipeline(s)
    S = 64
    tr = _traced(s, it, off, S)
    flat, ends = _tile_lists(s, it, off)
    checked = 0
    for c in range(s.C):
        for y in range(s.height):
            for x in range(s.width):
                t = _pixel_tile(s, c, y, x)
                T, want, clear = 1.0, [], True
                for i in range(flat[t], ends[t]):
                    g = int(it.flatten_ids[i])
                    m = s.means2d.reshape(-1, 2)[g].astype(np.float64)
                    a, b, cc = s.conics.reshape(-1, 3)[g].astype(np.float64)
                    dx, dy = m[0] - (x + 0.5), m[1] - (y + 0.5)
                    sigma = 0.5 * (a * dx * dx + cc * dy * dy) + b * dx * dy
                    if abs(sigma) < 1e-4:
                        clear = False
                    if sigma < 0:
                        continue
                    al = min(float(s.alpha_clamp), float(s.opacities.reshape(-1)[g]) * math.exp(-sigma))
                    if abs(al - s.alpha_cutoff) < 1e-4 * s.alpha_cutoff:
                        clear = False
                    if al < s.alpha_cutoff:
                        continue
                    tn = T * (1 - al)
                    if abs(tn - s.transmittance_threshold) < 1e-4 * max(s.transmittance_threshold, 1e-6):
                        clear = False
                    if tn <= s.transmittance_threshold or len(want) == S:
                        break
                    want.append(g)
                    T = tn
                if not clear:
                    continue
                n = int(tr.trace_counts[c, y, x])
                assert n == len(want), (c, y, x)
                np.testing.assert_array_equal(tr.trace_ids[c, y, x, :n], want)
                checked += 1
    assert checked > 0.9 * s.C * s.height * s.width
    assert tr.trace_counts.max() > 5  # the scene stacks several splats on a pixel


@pytest.mark.parametrize("seed", [42, 43])
def test_uncapped_trace_is_the_untraced_forward(seed):
    s = synth.random_scene(seed, 2, 40, 50, 37, 16, channels=3, background=True)
    it, off, ras = oracle.scene_pipeline(s)
    big = int(np.diff(np.append(off.reshape(-1), it.n_isects)).max()) + 1
    tr = _traced(s, it, off, big)
    for name in ("render_colors", "render_alphas", "render_T", "last_ids"):
        np.testing.assert_array_equal(getattr(tr, name), getattr(ras, name), err_msg=name)
    assert tr.n_eval == ras.n_eval
    # the last traced splat sits at the last id; nothing composited means no trace
    has = tr.trace_counts > 0
    assert has.any() and (~has).any()
    last_ids = it.flatten_ids[ras.last_ids[has]]
    idx = tr.trace_counts[has] - 1
    np.testing.assert_array_equal(tr.trace_ids[has][np.arange(idx.size), idx], last_ids)
    np.testing.assert_array_equal(ras.last_ids[~has], -1)
    # entries past a pixel's count are left as they were (the wrapper pre-fills -2)
    past = np.arange(big)[None, None, None, :] >= tr.trace_counts[..., None]
    assert (tr.trace_ids[past] == -2).all() and (tr.trace_ids[~past] >= 0).all()


def test_early_out_pixels_trace_only_what_they_composited():
    """Dense opaque splats: most pixels stop at the transmittance threshold; the stopping splat is not traced."""
    s = synth.random_scene(50, 1, 600, 32, 32, 16, channels=3, background=True)
    s.opacities[:] = np.float32(0.97)
    it, off, ras = oracle.scene_pipeline(s)
    S = 512
    tr = _traced(s, it, off, S)
    flat, ends = _tile_lists(s, it, off)
    ty = np.arange(s.height)[:, None] // s.tile_size
    tx = np.arange(s.width)[None, :] // s.tile_size
    t = ty * s.tile_width + tx
    # pixels whose last id is before the end of a list with more splats behind it stopped early
    early = ras.last_ids[0] + 1 < ends[t]
    assert early.mean() > 0.5
    past = np.arange(S)[None, None, None, :] >= tr.trace_counts[..., None]
    assert (tr.trace_ids[past] == -2).all()


def test_trace_alone_reproduces_the_pixel():
    s = synth.random_scene(44, 1, 200, 33, 30, 16, channels=2, background=True)
    it, off, _ = oracle.scene_pipeline(s)
    tr = _traced(s, it, off, 256)
    for y in range(0, s.height, 3):
        for x in range(0, s.width, 2):
            n = int(tr.trace_counts[0, y, x])
            acc, T, last, _, trace = oracle.composite_pixel_traced(
                s.means2d, s.conics, s.colors, s.opacities, tr.trace_ids[0, y, x, :n], x, y, s.alpha_cutoff,
                s.alpha_clamp, s.transmittance_threshold, -1)
            assert T == tr.render_T[0, y, x]
            np.testing.assert_array_equal(acc + np.float32(T) * s.backgrounds[0], tr.render_colors[0, y, x])
            np.testing.assert_array_equal(trace, tr.trace_ids[0, y, x, :n])  # every traced splat composites


@pytest.mark.parametrize("S", [0, 1, 3, 7])
def test_step_cap_is_the_composite_cut_after_the_last_step(S):
    s = synth.random_scene(45, 2, 400, 40, 35, 16, channels=3, background=True)
    it, off, _ = oracle.scene_pipeline(s)
    flat, ends = _tile_lists(s, it, off)
    full = _traced(s, it, off, 4096)
    cap = _traced(s, it, off, S)
    assert (cap.trace_counts == np.minimum(full.trace_counts, S)).all()
    if S == 0:
        assert (cap.render_T == 1).all() and (cap.last_ids == -1).all()
        np.testing.assert_array_equal(cap.render_colors, np.broadcast_to(s.backgrounds[:, None, None],
                                                                          cap.render_colors.shape))
        return
    for c in range(s.C):
        for y in range(0, s.height, 2):
            for x in range(s.width):
                n = int(cap.trace_counts[c, y, x])
                np.testing.assert_array_equal(cap.trace_ids[c, y, x, :n], full.trace_ids[c, y, x, :n])
                t = _pixel_tile(s, c, y, x)
                # the untraced composite over the list cut right after the capped last step
                cut = ends[t] if n < S else cap.last_ids[c, y, x] + 1
                lst = it.flatten_ids[flat[t]:cut]
                acc, T, last, _ = oracle.composite_pixel(s.means2d, s.conics, s.colors, s.opacities, lst, x, y,
                                                         s.alpha_cutoff, s.alpha_clamp, s.transmittance_threshold)
                assert T == cap.render_T[c, y, x]
                np.testing.assert_array_equal(acc + np.float32(T) * s.backgrounds[c], cap.render_colors[c, y, x])
                assert (last + flat[t] if last >= 0 else -1) == cap.last_ids[c, y, x]
    assert (full.trace_counts > S).any()  # the cap bites somewhere


@pytest.mark.parametrize("L", [0, 1, 5, 40])
def test_list_cap_is_the_forward_over_cut_lists(L):
    s = synth.random_scene(46, 2, 500, 48, 40, 16, channels=3, background=True)
    it, off, _ = oracle.scene_pipeline(s)
    flat, ends = _tile_lists(s, it, off)
    keep = np.minimum(ends - flat, L)
    new_off = np.concatenate([[0], np.cumsum(keep)[:-1]]).astype(np.int32).reshape(off.shape)
    new_ids = np.concatenate([it.flatten_ids[f:f + k] for f, k in zip(flat, keep)]).astype(np.int32)
    ref = _untraced(s, new_off, new_ids, new_ids.size)
    tr = _traced(s, it, off, 4096, L=L)
    for name in ("render_colors", "render_alphas", "render_T"):
        np.testing.assert_array_equal(getattr(tr, name), getattr(ref, name), err_msg=name)
    # last ids are global intersection indices: map the cut lists' positions back to the original ones
    ty = np.arange(s.height)[:, None] // s.tile_size
    tx = np.arange(s.width)[None, :] // s.tile_size
    for c in range(s.C):
        t = (c * s.tile_height + ty) * s.tile_width + tx
        mapped = np.where(ref.last_ids[c] >= 0, ref.last_ids[c] - new_off.reshape(-1)[t] + flat[t], -1)
        np.testing.assert_array_equal(tr.last_ids[c], mapped)
    assert (ends - flat).max() > L  # the cap bites


def test_capped_forward_backward_matches_finite_differences():
    """The range backward on a step-capped forward's outputs is the gradient of the capped forward."""
    s = _smooth_scene(47, n=7)
    it, off, _ = oracle.scene_pipeline(s)
    S = 3
    tr = _traced(s, it, off, S)
    assert (tr.trace_counts == S).any() and (tr.trace_counts < S).any()
    flat, ends = _tile_lists(s, it, off)
    lists = [it.flatten_ids[flat[t]:ends[t]] for t in range(flat.size)]
    rng = np.random.default_rng(48)
    gc = rng.normal(size=tr.render_colors.shape).astype(np.float32)
    ga = rng.normal(size=tr.render_alphas.shape).astype(np.float32)
    g = oracle.rasterize_bwd(s.means2d, s.conics, s.colors, s.opacities, s.backgrounds, s.width, s.height,
                             s.tile_size, off, it.flatten_ids, it.n_isects, s.alpha_cutoff, s.alpha_clamp,
                             tr.render_alphas, tr.last_ids, gc, ga)
    base = [s.means2d.astype(np.float64), s.conics.astype(np.float64), s.colors.astype(np.float64),
            s.opacities.astype(np.float64), s.backgrounds.astype(np.float64)]
    out, _ = _forward64(s, lists, base, max_steps=S)
    np.testing.assert_allclose(out, tr.render_colors, atol=1e-5)

    def loss(params):
        o, a = _forward64(s, lists, params, max_steps=S)
        return float((gc * o).sum() + (ga * a).sum())

    for which, grad in enumerate([g.means2d, g.conics, g.colors, g.opacities, g.backgrounds]):
        fd = np.zeros_like(base[which])
        for idx in np.ndindex(base[which].shape):
            h = 1e-5 * max(1.0, abs(base[which][idx]))
            up = [p.copy() for p in base]
            dn = [p.copy() for p in base]
            up[which][idx] += h
            dn[which][idx] -= h
            fd[idx] = (loss(up) - loss(dn)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=2e-3, atol=2e-4 * np.abs(fd).max(), err_msg=f"group {which}")


def test_trace_needs_a_row_length():
    s = synth.random_scene(49, 1, 10, 16, 16, 16, channels=3)
    it, off, _ = oracle.scene_pipeline(s)
    with pytest.raises(ValueError):
        _traced(s, it, off, -1)

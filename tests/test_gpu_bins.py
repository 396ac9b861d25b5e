"""GPU parity of the fixed-capacity bins (gs_bin_tiles) and compositing over them (gs_rasterize_fwd_bins) with the
oracle's orc_bin_tiles / orc_rasterize_bins on the same seeded inputs: bins, counts, colours, alphas, T and last ids
exactly; under overflow the counts exactly and the kept entries checked for validity (a sorted subset of the tile's
list, since which ones a full bin keeps is not specified); sentinels anywhere in a bin; and the 1080p, 1M-splat frame
against the sorted intersection path."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, synth

from gpu_util import dev, gpu_frame, host, oracle_frame, require_gpu
from test_gpu_parity import SCENES

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _gpu_bins(scene, capacity):
    b = binding.gs_bin_tiles(dev(scene.means2d), dev(scene.radii), dev(scene.depths), scene.tile_size,
                             scene.tile_width, scene.tile_height, capacity)
    torch.cuda.synchronize()
    return b


def _oracle_bins(scene, capacity):
    return oracle.bin_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                            scene.tile_height, capacity)


def _largest(scene):
    return max(1, _oracle_bins(scene, 1).largest)


def _gpu_composite(scene, bins):
    bg = None if scene.backgrounds is None else dev(scene.backgrounds)
    r = binding.gs_rasterize_fwd_bins(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities),
                                      bg, scene.width, scene.height, scene.tile_size, bins.bin_ids, bins.bin_counts,
                                      scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold)
    torch.cuda.synchronize()
    return r


def _oracle_composite(scene, bin_ids):
    return oracle.rasterize_bins(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                                 scene.width, scene.height, scene.tile_size, bin_ids, scene.alpha_cutoff,
                                 scene.alpha_clamp, scene.transmittance_threshold)


def _assert_render_equal(g, o):
    np.testing.assert_array_equal(host(g.render_colors), o.render_colors)
    np.testing.assert_array_equal(host(g.render_alphas), o.render_alphas)
    np.testing.assert_array_equal(host(g.render_T), o.render_T)
    np.testing.assert_array_equal(host(g.last_ids), o.last_ids)


NAMES = ["tiny", "tiny-aniso", "cull-edges", "multicam-ragged-elliptical", "ts8-margin", "ts32-ppt4", "ts1",
         "dense-early-out", "deep-tiles", "single-tile", "all-equal-keys", "zero-radius", "one-isect", "empty", "K1",
         "K2", "K4"]


@pytest.mark.parametrize("name", NAMES)
def test_bins_and_bin_composite_match_oracle(name):
    scene = SCENES[name]()
    cap = _largest(scene) + 3
    g = _gpu_bins(scene, cap)
    o = _oracle_bins(scene, cap)
    np.testing.assert_array_equal(host(g.bin_counts), o.bin_counts)
    np.testing.assert_array_equal(host(g.bin_ids), o.bin_ids)
    _assert_render_equal(_gpu_composite(scene, g), _oracle_composite(scene, o.bin_ids))


@pytest.mark.parametrize("name,cap", [("multicam-ragged-elliptical", 4), ("deep-tiles", 50), ("ts8-margin", 1),
                                      ("all-equal-keys", 7)])
def test_overflowing_bins_keep_counts_and_a_sorted_subset(name, cap):
    scene = SCENES[name]()
    g = _gpu_bins(scene, cap)
    full = _oracle_bins(scene, _largest(scene))
    counts = full.bin_counts.reshape(-1)
    np.testing.assert_array_equal(host(g.bin_counts).reshape(-1), counts)
    assert (counts > cap).any()
    gb = host(g.bin_ids).reshape(counts.size, cap)
    fb = full.bin_ids.reshape(counts.size, -1)
    for t in range(counts.size):
        k = min(int(counts[t]), cap)
        assert (gb[t, k:] == -1).all()
        kept = gb[t, :k]
        rank = {int(v): i for i, v in enumerate(fb[t, :counts[t]])}  # positions in the tile's full list
        ranks = np.array([rank.get(int(v), -1) for v in kept])
        assert (ranks >= 0).all(), f"tile {t}: kept ids outside the tile's list"
        assert (np.diff(ranks) > 0).all(), f"tile {t}: kept ids out of (depth, id) order"


def test_sentinels_anywhere_in_a_bin_are_skipped():
    scene = SCENES["multicam-ragged-elliptical"]()
    cap = _largest(scene)
    o = _oracle_bins(scene, cap)
    T = o.bin_counts.size
    rng = np.random.default_rng(71)
    wide = np.full((T, 3 * cap), -1, np.int32)
    for t in range(T):
        n = int(o.bin_counts.reshape(-1)[t])
        wide[t, np.sort(rng.choice(3 * cap, size=n, replace=False))] = o.bin_ids.reshape(T, cap)[t, :n]
    wide = wide.reshape(o.bin_ids.shape[:3] + (3 * cap,))
    counts = np.full(o.bin_counts.shape, 3 * cap, np.int32)  # read every slot
    g = _gpu_composite(scene, binding.Bins(dev(wide), dev(counts)))
    _assert_render_equal(g, _oracle_composite(scene, wide))


def test_bins_1m_splats_1080p_match_the_sorted_path():
    """At 1M splats the bins equal the oracle's sorted tile lists and their composite the oracle's frame."""
    scene = synth.config3()
    it_o, off_o, ras_o = oracle_frame(scene, openmp=True)
    cap = 8192
    g = _gpu_bins(scene, cap)
    off = off_o.reshape(-1).astype(np.int64)
    ids = it_o.flatten_ids
    ends = np.append(off[1:], it_o.n_isects)
    counts = host(g.bin_counts).reshape(-1)
    np.testing.assert_array_equal(counts, ends - off)
    assert counts.max() <= cap
    gb = host(g.bin_ids).reshape(counts.size, cap)
    for t in range(counts.size):
        np.testing.assert_array_equal(gb[t, :counts[t]], ids[off[t]:ends[t]], err_msg=f"tile {t}")
    assert (gb[np.arange(cap)[None, :] >= counts[:, None]] == -1).all()
    r = _gpu_composite(scene, g)
    np.testing.assert_array_equal(host(r.render_colors), ras_o.render_colors)
    np.testing.assert_array_equal(host(r.render_T), ras_o.render_T)
    lb = host(r.last_ids).astype(np.int64)
    t = np.maximum(lb, 0) // cap
    mapped = np.where(lb >= 0, off[t] + lb % cap, -1)
    np.testing.assert_array_equal(mapped, ras_o.last_ids)


def test_bins_with_more_tiles_than_the_lds_counters():
    """Above 32768 tiles the fill takes one global atomic per (splat, tile) instead of the LDS-aggregated path."""
    scene = synth.random_scene(72, 1, 400, 256, 160, 1, r_range=(0.3, 4.0))
    assert scene.tile_width * scene.tile_height > 32768
    cap = _largest(scene) + 1
    g = _gpu_bins(scene, cap)
    o = _oracle_bins(scene, cap)
    np.testing.assert_array_equal(host(g.bin_counts), o.bin_counts)
    np.testing.assert_array_equal(host(g.bin_ids), o.bin_ids)
    _assert_render_equal(_gpu_composite(scene, g), _oracle_composite(scene, o.bin_ids))

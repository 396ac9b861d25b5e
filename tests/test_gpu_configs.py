"""GPU parity at the five workload sizes, in the launch configuration the benchmark times.

tiny and the 200k-splat 800x800 scene: every output against the oracle's full run. The 1M-splat 1080p scene:
intersections, sorted keys and tile ranges against the full oracle run; the composite on sampled tiles (the
heaviest plus a seeded random set), each composited by the oracle from its own per-tile list. The 4-camera 3M and
the 6M 4K scenes: counts, offsets, unsorted keys and tile ranges against the oracle in full; the sorted order by
properties that fix it uniquely at any size (strictly increasing (key, id), every pair a real intersection, and
per-tile counts equal to the oracle's); and sampled tiles as above."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, synth

from gpu_util import (assert_isect_equal, assert_raster_equal, check_tiles_against_oracle, gpu_frame, gpu_isect,
                      host, keys_u64, require_gpu, sampled_tiles)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_tiny_full():
    s = synth.tiny()
    it_o, off_o, ras_o = oracle.scene_pipeline(s)
    fr = gpu_frame(s)
    assert_isect_equal(s, fr.isect, it_o, True)
    np.testing.assert_array_equal(host(fr.isect_offsets), off_o)
    assert_raster_equal(s, fr, ras_o, it_o.flatten_ids)


def test_config2_full():
    s = synth.config2()
    it_o, off_o, ras_o = oracle.scene_pipeline(s)
    fr = gpu_frame(s)
    assert_isect_equal(s, fr.isect, it_o, True)
    np.testing.assert_array_equal(host(fr.isect_offsets), off_o)
    assert_raster_equal(s, fr, ras_o, it_o.flatten_ids)
    it_u = oracle.isect_tiles(s.means2d, s.radii, s.depths, 16, s.tile_width, s.tile_height, sort=False)
    assert_isect_equal(s, gpu_isect(s, False), it_u, False)


def test_config3_isect_sort_ranges_full_and_sampled_composite():
    s = synth.config3()
    it_o = oracle.isect_tiles(s.means2d, s.radii, s.depths, 16, s.tile_width, s.tile_height, sort=True)
    off_o = oracle.tile_offsets(it_o.keys, 1, s.tile_width, s.tile_height)
    assert 10_000_000 <= it_o.n_isects <= 20_000_000
    fr = gpu_frame(s)
    assert_isect_equal(s, fr.isect, it_o, True)
    np.testing.assert_array_equal(host(fr.isect_offsets), off_o)
    tiles = sampled_tiles(off_o, it_o.n_isects, 64, seed=3)
    check_tiles_against_oracle(s, fr, tiles)


def _check_sorted_by_properties(s, it_g, off_o, rects):
    keys = keys_u64(it_g.isect_ids)
    ids = host(it_g.flatten_ids).astype(np.int64)
    n = keys.size
    # strictly increasing (key, id): sorted, stable for equal keys, and no repeated pair
    dk = keys[1:] > keys[:-1]
    eq = keys[1:] == keys[:-1]
    assert (dk | (eq & (ids[1:] > ids[:-1]))).all()
    # every pair is a real intersection of its splat
    tb = oracle.bits_for(s.tile_width * s.tile_height)
    upper = keys >> np.uint64(32)
    cam = (upper >> np.uint64(tb)).astype(np.int64)
    tile = (upper & np.uint64((1 << tb) - 1)).astype(np.int64)
    np.testing.assert_array_equal(cam, ids // s.N)
    np.testing.assert_array_equal((keys & np.uint64(0xFFFFFFFF)).astype(np.uint32),
                                  s.depths.reshape(-1).view(np.uint32)[ids])
    ty, tx = tile // s.tile_width, tile % s.tile_width
    r = rects[ids]
    assert ((tx >= r[:, 0]) & (tx < r[:, 2]) & (ty >= r[:, 1]) & (ty < r[:, 3])).all()
    del r, ty, tx, upper
    # per-tile counts equal the oracle's: with the above, each tile holds exactly its true splat set
    gt = cam * (s.tile_width * s.tile_height) + tile
    counts = np.bincount(gt, minlength=off_o.size)
    np.testing.assert_array_equal(np.concatenate([[0], np.cumsum(counts)[:-1]]), off_o.reshape(-1))
    assert counts.sum() == n


@pytest.mark.parametrize("make", [synth.config4, synth.config5], ids=["config4", "config5"])
def test_large_configs(make):
    s = make()
    print(f"\n{s.name}: C={s.C} N={s.N}", flush=True)
    it_u = oracle.isect_tiles(s.means2d, s.radii, s.depths, 16, s.tile_width, s.tile_height, sort=False)
    off_o = oracle.tile_offsets(it_u.keys, s.C, s.tile_width, s.tile_height)
    print(f"oracle n_isects={it_u.n_isects}", flush=True)
    g_u = gpu_isect(s, False)
    assert_isect_equal(s, g_u, it_u, False)
    del g_u
    torch.cuda.empty_cache()
    rects = oracle.rects(s.means2d, s.radii, 16, s.tile_width, s.tile_height)
    del it_u
    fr = gpu_frame(s)
    np.testing.assert_array_equal(host(fr.isect_offsets), off_o)
    _check_sorted_by_properties(s, fr.isect, off_o, rects)
    tiles = sampled_tiles(off_o, fr.isect.n_isects, 24, seed=5)
    check_tiles_against_oracle(s, fr, tiles)
    if "config5" in s.name:
        assert fr.isect.n_isects > 150_000_000
    if "config4" in s.name:
        tp = host(fr.isect.tiles_per_gauss)
        assert (tp == 0).sum() >= 4 * 30_000

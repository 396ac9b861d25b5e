"""Pins for the oracle's intersection step (tile rectangles, counts, key emission), CPU only.

Definitions: gsplat 1.0.0 native extension, intersections.c (gs_tile_bits, gs_bounds, gs_isect_tiles).
The pins are independent of the oracle's code: a hand-worked example, an interval-overlap enumeration of
tiles (a different formulation from floor/ceil), and decoding of every emitted key.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from tile_binned_gaussian_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex(v):
    return np.array([int(x, 16) for x in v], dtype=np.uint64)


def test_hand_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "isect_hand_example.json")))
    m = np.array(g["means2d"], np.float32)
    r = np.array(g["radii"], np.float32)
    d = np.array(g["depths"], np.float32)
    ts, tw, th = g["tile_size"], g["tile_width"], g["tile_height"]
    it = orc.isect_tiles(m, r, d, ts, tw, th, sort=False)
    assert it.n_isects == g["n_isects"]
    np.testing.assert_array_equal(it.tiles_per_gauss, np.array(g["tiles_per_gauss"]))
    np.testing.assert_array_equal(it.keys, _hex(g["keys_emitted"]))
    np.testing.assert_array_equal(it.flatten_ids, np.array(g["ids_emitted"]))
    its = orc.isect_tiles(m, r, d, ts, tw, th, sort=True)
    np.testing.assert_array_equal(its.keys, _hex(g["keys_sorted"]))
    np.testing.assert_array_equal(its.flatten_ids, np.array(g["ids_sorted"]))
    off = orc.tile_offsets(its.keys, 2, tw, th)
    np.testing.assert_array_equal(off, np.array(g["isect_offsets"]))


@pytest.mark.parametrize("count", list(range(1, 70)) + [1000, 1024, 1025, 8160, 32400, 26800, 2 ** 20 + 1])
def test_bits_for_is_ceil_log2(orc, count):
    b = orc.bits_for(count)
    assert (1 << b) >= count
    assert b == 0 or (1 << (b - 1)) < count
    assert b == (0 if count == 1 else math.ceil(math.log2(count)))


def brute_tiles(mx, my, rx, ry, ts, tw, th):
    """Tiles whose cell [tx*ts, (tx+1)*ts) x [ty*ts, (ty+1)*ts) meets the open box (m - r, m + r).

    The box edges are the float32 values fl(m - r), fl(m + r) the definition divides; the cell test is exact
    in float64. For a power-of-two tile size this is the floor/ceil rectangle of the definition:
    tx >= floor(lo/ts) <=> (tx+1) ts > lo, and tx < ceil(hi/ts) <=> tx ts < hi."""
    mx, my, rx, ry = (np.float32(v) for v in (mx, my, rx, ry))
    if not (rx > 0 and ry > 0):
        return []
    lox, hix = float(mx - rx), float(mx + rx)
    loy, hiy = float(my - ry), float(my + ry)
    out = []
    for ty in range(th):
        if not ((ty + 1) * ts > loy and ty * ts < hiy):
            continue
        for tx in range(tw):
            if (tx + 1) * ts > lox and tx * ts < hix:
                out.append(ty * tw + tx)
    return out


def check_against_brute(orc, scene, sort=False):
    ts, tw, th = scene.tile_size, scene.tile_width, scene.tile_height
    it = orc.isect_tiles(scene.means2d, scene.radii, scene.depths, ts, tw, th, sort=sort)
    C, N = scene.C, scene.N
    tile_bits = orc.bits_for(tw * th)
    rad = scene.radii.reshape(C * N, scene.radii_per_gauss)
    mm = scene.means2d.reshape(C * N, 2)
    dbits = scene.depths.reshape(-1).view(np.uint32)
    expected = []
    for i in range(C * N):
        rx = rad[i, 0]
        ry = rad[i, 1] if rad.shape[1] == 2 else rx
        expected.append(brute_tiles(mm[i, 0], mm[i, 1], rx, ry, ts, tw, th))
    counts = np.array([len(e) for e in expected], dtype=np.int64)
    np.testing.assert_array_equal(it.tiles_per_gauss.reshape(-1), counts)
    assert it.n_isects == counts.sum()
    np.testing.assert_array_equal(it.gauss_offsets, np.concatenate([[0], np.cumsum(counts)[:-1]]) if C * N else [])
    # decode every key: camera, tile and depth bits
    k = it.keys
    upper = k >> np.uint64(32)
    cam = (upper >> np.uint64(tile_bits)).astype(np.int64)
    tile = (upper & np.uint64((1 << tile_bits) - 1)).astype(np.int64)
    low = (k & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    ids = it.flatten_ids.astype(np.int64)
    np.testing.assert_array_equal(cam, ids // max(N, 1))
    np.testing.assert_array_equal(low, dbits[ids])
    if not sort:
        # emission order: ascending flat id, and each splat's tiles in row-major order, each once
        exp_ids = np.repeat(np.arange(C * N), counts)
        np.testing.assert_array_equal(ids, exp_ids)
        np.testing.assert_array_equal(tile, np.array([t for e in expected for t in e], dtype=np.int64))
    else:
        pairs = sorted(zip(ids.tolist(), tile.tolist()))
        assert pairs == sorted((i, t) for i, e in enumerate(expected) for t in e)
    return it


@pytest.mark.parametrize("make", [lambda: synth.tiny(), lambda: synth.tiny(anisotropic=True),
                                  lambda: synth.random_scene(5, 2, 300, 130, 90, 16, elliptical=True,
                                                             zero_radius_frac=0.1),
                                  lambda: synth.random_scene(6, 3, 200, 77, 41, 8, r_range=(0.1, 30.0),
                                                             margin=0.5, zero_radius_frac=0.05),
                                  lambda: synth.random_scene(7, 1, 150, 40, 40, 32, elliptical=True)])
def test_counts_and_keys_vs_brute_force(orc, make):
    check_against_brute(orc, make(), sort=False)


def test_sorted_isect_is_a_permutation_of_brute_force(orc):
    check_against_brute(orc, synth.random_scene(8, 2, 250, 100, 60, 16, elliptical=True, dup_depth_frac=0.3),
                        sort=True)


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.sampled_from([1, 2, 4, 8, 16, 32]), st.integers(1, 9), st.integers(1, 9),
       st.integers(1, 3), st.integers(0, 12), st.booleans())
def test_random_grids_vs_brute_force(orc, seed, ts, tw, th, C, N, elliptical):
    rng = np.random.default_rng(seed)
    W, H = tw * ts, th * ts
    means = rng.uniform(-0.5 * W, 1.5 * W, size=(C, N, 2)).astype(np.float32)
    means[..., 1] = rng.uniform(-0.5 * H, 1.5 * H, size=(C, N))
    shape = (C, N, 2) if elliptical else (C, N)
    radii = rng.choice([0.0, -1.0, 0.25, 1.0, 3.5, 16.0, 40.0], size=shape).astype(np.float32)
    radii = np.where(rng.uniform(size=shape) < 0.5, rng.uniform(0, 2 * ts, size=shape), radii).astype(np.float32)
    depths = rng.uniform(0.1, 5.0, size=(C, N)).astype(np.float32)
    ts_scene = synth.Scene("h", C, N, W, H, ts, means, radii, depths, np.zeros((C, N, 3), np.float32),
                           np.zeros((C, N, 3), np.float32), np.zeros((C, N), np.float32))
    check_against_brute(orc, ts_scene, sort=bool(seed & 1))


def test_degenerate_bounds(orc):
    # zero / negative radius -> empty; a splat entirely left of or below the grid -> empty
    assert orc.bounds(10, 10, 0, 5, 16, 4, 4) == (0, 0, 0, 0)
    assert orc.bounds(10, 10, 5, -1, 16, 4, 4) == (0, 0, 0, 0)
    x0, y0, x1, y1 = orc.bounds(-20, 10, 3, 3, 16, 4, 4)
    assert (x1 - x0) == 0
    # covering everything clamps to the grid
    assert orc.bounds(32, 32, 1000, 1000, 16, 4, 4) == (0, 0, 4, 4)
    # a mean exactly on a tile edge with a tiny radius touches both neighbouring tiles
    assert orc.bounds(16, 16, 0.5, 0.5, 16, 4, 4) == (0, 0, 2, 2)
    # non-finite input yields no tiles (documented reading of the float-to-int step)
    x0, y0, x1, y1 = orc.bounds(float("nan"), 10, 3, 3, 16, 4, 4)
    assert (x1 - x0) * (y1 - y0) == 0


def test_single_tile_grid_has_zero_tile_bits(orc):
    m = np.array([[[3.0, 4.0], [9.0, 9.0]]], np.float32)
    r = np.array([[2.0, 50.0]], np.float32)
    d = np.array([[1.0, 0.5]], np.float32)
    it = orc.isect_tiles(m, r, d, 16, 1, 1, sort=True)
    assert orc.bits_for(1) == 0
    assert it.n_isects == 2
    assert [int(k >> np.uint64(32)) for k in it.keys] == [0, 0]
    assert it.flatten_ids.tolist() == [1, 0]  # 0.5 sorts before 1.0


def test_empty_inputs(orc):
    m = np.zeros((1, 0, 2), np.float32)
    it = orc.isect_tiles(m, np.zeros((1, 0), np.float32), np.zeros((1, 0), np.float32), 16, 4, 4)
    assert it.n_isects == 0
    off = orc.tile_offsets(it.keys, 1, 4, 4)
    assert (off == 0).all()

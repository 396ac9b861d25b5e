"""GPU edge cases and property tests of the intersection, sort and range path (and the composite where the grid
fits an image), each against the oracle.

- The key-width limit: camera bits + tile bits = 32 (gsplat 1.0.0 intersections.c, gs_isect_tiles packs
  ((camera << tile_bits) | tile) << 32 | depth bits), so the frame's tile sort runs four 8-bit passes over bits
  [32, 64) and the last camera's keys have bit 63 set; the ranges (gs_offset_encode's [C, th, tw] offsets) of such a
  grid, and the rejection of a grid of 2^32 tiles.
- Random small grids drawn by hypothesis with a fixed example budget (derandomized): tile sizes 1..32, grids not
  tied to an image, up to 3 cameras, radii <= 0, means off the image, duplicated depths, n = 0 and n = 1 intersections
  and all-equal keys; sorted and unsorted emission, ranges and, on image-shaped grids, the composite."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from tile_binned_gaussian_amd import binding, frame, synth

from gpu_util import assert_isect_equal, assert_raster_equal, dev, gpu_frame, gpu_isect, host, keys_u64, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _grid_scene(seed, C, N, tw, th, ts, r_max=3.0):
    """C cameras of N splats each over a tw x th grid of ts-pixel tiles (image tw*ts x th*ts)."""
    rng = np.random.default_rng(seed)
    W, H = tw * ts, th * ts
    M = C * N
    means = np.stack([rng.uniform(-2, W + 2, M), rng.uniform(-2, H + 2, M)], -1).astype(np.float32)
    radii = rng.uniform(0.3, r_max, M).astype(np.float32)
    radii[rng.uniform(size=M) < 0.05] = 0.0
    depths = rng.uniform(0.5, 10.0, M).astype(np.float32)
    z = np.zeros((C, N, 3), np.float32)
    return synth.Scene(f"grid-{C}x{N}-{tw}x{th}-ts{ts}", C, N, W, H, ts, means.reshape(C, N, 2),
                       radii.reshape(C, N), depths.reshape(C, N), z, z, np.zeros((C, N), np.float32))


def test_key_width_limit_frame_path():
    s = _grid_scene(201, 32769, 2, 10923, 3, 1)
    tb, cb = oracle.bits_for(s.tile_width * s.tile_height), oracle.bits_for(s.C)
    assert (tb, cb) == (16, 16)
    print(f"\nkey-width limit: C={s.C} grid {s.tile_width}x{s.tile_height}", flush=True)
    it_o = oracle.isect_tiles(s.means2d, s.radii, s.depths, 1, s.tile_width, s.tile_height, sort=True)
    assert (it_o.keys >> np.uint64(63)).any(), "the last camera's keys carry bit 63"
    g = gpu_isect(s, True)
    assert_isect_equal(s, g, it_o, True)
    off_o = oracle.tile_offsets(it_o.keys, s.C, s.tile_width, s.tile_height)
    off_g = binding.gs_tile_ranges(g.isect_ids, s.C, s.tile_width, s.tile_height, validate=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(off_g), off_o)
    # the frame plan sorts the tile bits in 4 passes
    assert (32 + tb + cb - 32 + 7) // 8 == 4


def test_key_width_limit_of_2_to_32_tiles_sorts_and_rejects_ranges():
    s = _grid_scene(202, 65536, 2, 256, 256, 1)
    assert oracle.bits_for(s.tile_width * s.tile_height) + oracle.bits_for(s.C) == 32
    it_o = oracle.isect_tiles(s.means2d, s.radii, s.depths, 1, s.tile_width, s.tile_height, sort=True)
    assert (it_o.keys >> np.uint64(63)).any()
    g = gpu_isect(s, True)
    assert_isect_equal(s, g, it_o, True)
    with pytest.raises(binding.GsError) as e:
        binding.gs_tile_ranges(g.isect_ids, s.C, s.tile_width, s.tile_height)
    assert e.value.status == binding.GS_ERR_INVALID_ARG


@st.composite
def _grids(draw):
    ts = draw(st.sampled_from([1, 2, 4, 8, 16, 32]))
    tw, th = draw(st.integers(1, 9)), draw(st.integers(1, 9))
    C = draw(st.integers(1, 3))
    N = draw(st.sampled_from([0, 1, 2, 5, 17, 60]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    image = draw(st.booleans())  # the grid is ceil(W / ts) x ceil(H / ts) of a ragged image
    equal_keys = draw(st.booleans())
    return ts, tw, th, C, N, seed, image, equal_keys


@settings(max_examples=60, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(_grids())
def test_random_small_grids_against_oracle(g):
    ts, tw, th, C, N, seed, image, equal_keys = g
    rng = np.random.default_rng(seed)
    W = tw * ts - (int(rng.integers(0, ts)) if image else 0)
    H = th * ts - (int(rng.integers(0, ts)) if image else 0)
    s = synth.random_scene(seed, C, N, max(W, 1), max(H, 1), ts, elliptical=bool(seed & 1), margin=0.5,
                           r_range=(0.25, 2.5 * ts), zero_radius_frac=0.2, dup_depth_frac=0.5, background=True)
    if equal_keys and C * N > 0:
        # every splat on one tile with one depth: all keys equal, the order is the ids'
        s.means2d[...] = np.float32(0.5 * ts)
        s.radii[...] = np.float32(0.25 * ts)
        s.depths[...] = np.float32(2.0)
    assert (s.tile_width, s.tile_height) == (tw, th)
    for sort in (False, True):
        it_o = oracle.isect_tiles(s.means2d, s.radii, s.depths, ts, tw, th, sort=sort)
        it_g = gpu_isect(s, sort)
        assert_isect_equal(s, it_g, it_o, sort)
    off_o = oracle.tile_offsets(it_o.keys, C, tw, th)
    if it_o.n_isects > 0:
        off_g = binding.gs_tile_ranges(it_g.isect_ids, C, tw, th, validate=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(off_g), off_o)
    ras_o = oracle.rasterize_fwd(s.means2d, s.conics, s.colors, s.opacities, s.backgrounds, s.width, s.height, ts,
                                 off_o, it_o.flatten_ids, it_o.n_isects, s.alpha_cutoff, s.alpha_clamp,
                                 s.transmittance_threshold)
    fr = gpu_frame(s)
    assert_raster_equal(s, fr, ras_o, it_o.flatten_ids)

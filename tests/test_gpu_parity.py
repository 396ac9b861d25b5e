"""GPU parity on small scenes and edge cases: every step through the C ABI against the CPU oracle, on the same
seeded inputs. Integer outputs (counts, offsets, keys, ids, tile ranges) must match bit for bit; colours and
transmittance are compared bit for bit as well (the composite's float32 operation order and exponential are fixed),
and within the 1e-4 absolute bar."""
import numpy as np
import pytest
import torch

import oracle
from tile_binned_gaussian_amd import binding, synth

from gpu_util import (assert_isect_equal, assert_raster_equal, dev, gpu_frame, gpu_isect, host, keys_u64,
                      require_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _single_tile():
    s = synth.random_scene(31, 1, 40, 13, 11, 16, r_range=(1.0, 9.0))
    return s


def _all_equal_keys():
    # 300 identical splats: one key value repeated, the sort must keep ascending ids
    s = synth.random_scene(32, 1, 300, 48, 48, 16)
    s.means2d[:] = np.float32([20.0, 21.0])
    s.radii[:] = np.float32(2.0)
    s.depths[:] = np.float32(1.25)
    return s


def _zero_radius():
    s = synth.random_scene(33, 2, 50, 64, 64, 16)
    s.radii[:] = 0
    return s


def _one_isect():
    s = synth.random_scene(34, 1, 3, 64, 64, 16)
    s.radii[:] = np.float32([0.0, 0.0, 1.5])
    s.means2d[0, 2] = np.float32([40.0, 40.0])
    return s


def _cull_edges():
    # opacities just above the cutoff, strongly anisotropic conics and means on quadrant borders: the cases where a
    # conservative per-region cull of the composite would be wrong if its margins were
    rng = np.random.default_rng(44)
    s = synth.random_scene(44, 1, 1500, 48, 48, 16, r_range=(1.0, 14.0))
    cut = np.float32(1.0) / np.float32(255.0)
    n = s.N
    s.opacities[0] = np.where(rng.uniform(size=n) < 0.5, cut * rng.uniform(1.0, 1.3, n),
                              rng.uniform(0.5, 1.0, n)).astype(np.float32)
    s.opacities[0, :20] = cut
    edges = np.array([7.5, 8.0, 8.5, 15.5, 16.0, 16.5, 23.5, 24.0, 24.5, 31.5, 32.0, 32.5], np.float32)
    s.means2d[0, : n // 3] = rng.choice(edges, size=(n // 3, 2))
    l1 = rng.uniform(0.5, 40.0, n)
    l2 = l1 / rng.uniform(1.0, 250.0, n)
    th = rng.uniform(0, np.pi, n)
    cs, sn = np.cos(th), np.sin(th)
    sxx, syy, sxy = l1 * cs * cs + l2 * sn * sn, l1 * sn * sn + l2 * cs * cs, (l1 - l2) * cs * sn
    det = l1 * l2
    s.conics[0] = np.stack([syy / det, -sxy / det, sxx / det], -1).astype(np.float32)
    s.radii[0] = (3.0 * np.sqrt(l1)).astype(np.float32)
    return s


def _step_mix():
    # splats outside the composite's short step beside ordinary ones, so that some batches of a wave take the full
    # step and others the short one: ill-conditioned conics (axis ratio 2000-5000), indefinite conics (sigma < 0 in
    # places), opacities above 1e6, and infinite or NaN colour channels
    rng = np.random.default_rng(45)
    s = synth.random_scene(45, 1, 3000, 96, 64, 16, r_range=(1.0, 16.0), background=True)
    n = s.N
    pick = lambda frac: rng.uniform(size=n) < frac  # noqa: E731
    ill = pick(0.08)
    l1 = rng.uniform(1.0, 30.0, n)
    l2 = l1 / rng.uniform(2000.0, 5000.0, n)
    th = rng.uniform(0, np.pi, n)
    cs, sn = np.cos(th), np.sin(th)
    sxx, syy, sxy = l1 * cs * cs + l2 * sn * sn, l1 * sn * sn + l2 * cs * cs, (l1 - l2) * cs * sn
    det = l1 * l2
    ill_conic = np.stack([syy / det, -sxy / det, sxx / det], -1).astype(np.float32)
    s.conics[0][ill] = ill_conic[ill]
    indef = pick(0.04)
    a = rng.uniform(0.05, 0.5, n)
    s.conics[0][indef] = np.stack([a, 1.5 * a, a], -1).astype(np.float32)[indef]
    s.opacities[0][pick(0.02)] = np.float32(2.0e6)
    s.colors[0][pick(0.02), 1] = np.float32(np.inf)
    s.colors[0][pick(0.01), 2] = np.float32(np.nan)
    return s


def _cutoff(value):
    s = synth.random_scene(46, 1, 800, 80, 48, 16, r_range=(1.0, 14.0))
    s.alpha_cutoff = float(value)
    return s


SCENES = {
    "cull-edges": _cull_edges,
    "step-mix": _step_mix,
    "cutoff-zero": lambda: _cutoff(0.0),
    "cutoff-1e-20": lambda: _cutoff(np.float32(1e-20)),
    "tiny": lambda: synth.tiny(),
    "tiny-aniso": lambda: synth.tiny(anisotropic=True),
    "multicam-ragged-elliptical": lambda: synth.random_scene(35, 3, 700, 150, 90, 16, elliptical=True,
                                                              zero_radius_frac=0.05, dup_depth_frac=0.2,
                                                              background=True),
    "ts8-margin": lambda: synth.random_scene(36, 2, 500, 70, 45, 8, r_range=(0.3, 20.0), margin=0.5),
    "ts32-ppt4": lambda: synth.random_scene(37, 1, 900, 100, 70, 32, r_range=(2.0, 30.0), background=True),
    "ts1": lambda: synth.random_scene(38, 1, 60, 9, 7, 1, r_range=(0.2, 3.0)),
    "dense-early-out": lambda: synth.random_scene(22, 1, 600, 32, 32, 16, r_range=(3.0, 12.0)),
    "deep-tiles": lambda: synth.random_scene(39, 1, 6000, 64, 48, 16, r_range=(4.0, 24.0)),
    "single-tile": _single_tile,
    "all-equal-keys": _all_equal_keys,
    "zero-radius": _zero_radius,
    "one-isect": _one_isect,
    "empty": lambda: synth.random_scene(40, 1, 0, 32, 32, 16),
    "K1": lambda: synth.random_scene(41, 2, 400, 64, 40, 16, channels=1, background=True),
    "K2": lambda: synth.random_scene(42, 1, 400, 64, 40, 16, channels=2),
    "K4": lambda: synth.random_scene(43, 1, 400, 64, 40, 16, channels=4, background=True),
}


@pytest.mark.parametrize("name", list(SCENES))
def test_isect_unsorted_and_sorted(name):
    scene = SCENES[name]()
    for sort in (False, True):
        it_o = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                                  scene.tile_height, sort=sort)
        it_g = gpu_isect(scene, sort)
        assert_isect_equal(scene, it_g, it_o, sort)


def test_isect_rectangle_past_2_pow_22_tiles():
    # one splat whose rectangle covers a 2300 x 2000 grid of one-pixel tiles (4.6M > 2^22 tiles) among small ones:
    # the emission splits a slot's index in the rectangle into row and column with a float reciprocal below 2^22
    # and with the integer division from 2^22 on, so both ways meet in one rectangle
    s = synth.random_scene(45, 1, 40, 2300, 2000, 1, r_range=(0.5, 6.0))
    s.means2d[0, 0] = np.float32([1150.0, 1000.0])
    s.radii[0, 0] = np.float32(5000.0)
    for sort in (False, True):
        it_o = oracle.isect_tiles(s.means2d, s.radii, s.depths, s.tile_size, s.tile_width, s.tile_height, sort=sort)
        assert it_o.tiles_per_gauss[0, 0] == 2300 * 2000 > (1 << 22)
        assert_isect_equal(s, gpu_isect(s, sort), it_o, sort)


def _bit_pattern_depths(rng, m):
    """Depth bit patterns over the whole 32-bit range: negative floats, -0, infinities, NaN payloads and
    denormals beside ordinary positive depths, many sharing a top byte of 0xff (the last depth pass's largest
    digit) and many repeated exactly."""
    bits = rng.integers(0, 1 << 32, m, dtype=np.uint64).astype(np.uint32)
    kind = rng.integers(0, 6, m)
    bits = np.where(kind == 0, np.uint32(0xFF000000) | (bits & np.uint32(0x00FFFFFF)), bits)
    bits = np.where(kind == 1, np.float32(rng.uniform(0.5, 10.0, m)).view(np.uint32), bits)
    bits = np.where(kind == 2, bits & np.uint32(0x007FFFFF), bits)  # +0 and positive denormals
    special = np.array([0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFFFFFFF, 0x00000000], np.uint32)
    bits = np.where(kind == 3, special[rng.integers(0, len(special), m)], bits)
    dup = rng.uniform(size=m) < 0.2
    bits[dup] = bits[rng.integers(0, m, int(dup.sum()))]
    return bits.view(np.float32)


@pytest.mark.parametrize("n_per_camera", [1, 2047, 5000, 6144])
def test_isect_sorted_depth_bit_patterns(n_per_camera):
    # The depth sort orders the splats by the depths' bit patterns alone, over ragged partitions of 4096 splats
    # (2 cameras: 2, 4094, 10000 and 12288 splats); the last pass also scans the tile counts in that order, so
    # splats without tiles and the largest digit (top byte 0xff) next to the padding past the last splat are
    # covered. Keys, ids, counts and offsets must equal the oracle's bit for bit.
    rng = np.random.default_rng(n_per_camera)
    s = synth.random_scene(46 + n_per_camera, 2, n_per_camera, 96, 80, 16, r_range=(0.25, 20.0),
                           zero_radius_frac=0.25)
    s.depths[...] = _bit_pattern_depths(rng, s.C * s.N).reshape(s.C, s.N)
    s.depths[:, -min(n_per_camera, 64):] = np.uint32(0xFFFFFFF0).view(np.float32)
    it_o = oracle.isect_tiles(s.means2d, s.radii, s.depths, s.tile_size, s.tile_width, s.tile_height, sort=True)
    assert it_o.n_isects > 0
    assert_isect_equal(s, gpu_isect(s, True), it_o, True)


@pytest.mark.parametrize("name", list(SCENES))
def test_ranges_on_oracle_keys(name):
    scene = SCENES[name]()
    it_o = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                              scene.tile_height, sort=True)
    off_o = oracle.tile_offsets(it_o.keys, scene.C, scene.tile_width, scene.tile_height)
    keys = dev(it_o.keys.view(np.int64))
    for validate in (False, True):
        off_g = binding.gs_tile_ranges(keys, scene.C, scene.tile_width, scene.tile_height, validate=validate)
        np.testing.assert_array_equal(host(off_g), off_o)


@pytest.mark.parametrize("name", ["multicam-ragged-elliptical", "ts8-margin", "one-isect", "deep-tiles"])
def test_ranges_on_keys_not_16_byte_aligned(name):
    # keys one element into an allocation: 8-byte but not 16-byte aligned, which takes the scalar-load path
    scene = SCENES[name]()
    it_o = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                              scene.tile_height, sort=True)
    off_o = oracle.tile_offsets(it_o.keys, scene.C, scene.tile_width, scene.tile_height)
    padded = dev(np.concatenate([np.zeros(1, np.int64), it_o.keys.view(np.int64)]))
    keys = padded[1:]
    assert keys.data_ptr() % 16 == 8
    for validate in (False, True):
        off_g = binding.gs_tile_ranges(keys, scene.C, scene.tile_width, scene.tile_height, validate=validate)
        np.testing.assert_array_equal(host(off_g), off_o)


@pytest.mark.parametrize("name", list(SCENES))
def test_frame_end_to_end(name):
    scene = SCENES[name]()
    it_o, off_o, ras_o = oracle.scene_pipeline(scene)
    fr = gpu_frame(scene)
    np.testing.assert_array_equal(host(fr.isect_offsets), off_o)
    assert_raster_equal(scene, fr, ras_o, it_o.flatten_ids)


@pytest.mark.parametrize("name", ["multicam-ragged-elliptical", "tiny", "ts8-margin", "one-isect", "empty"])
def test_frame_plan_matches_oracle(name):
    """The preallocated frame path bench.py times: the count read back into page-locked memory (the depth order
    queued before the host waits), one intersection workspace shared by both phases and grown once, and repeated
    frames reusing every buffer."""
    from tile_binned_gaussian_amd import frame
    scene = SCENES[name]()
    it_o, off_o, ras_o = oracle.scene_pipeline(scene)
    plan = frame.FramePlan(frame.to_device(scene))
    for _ in range(3):
        n = plan.run()
        torch.cuda.synchronize()
        assert n == it_o.n_isects
        np.testing.assert_array_equal(keys_u64(plan.keys)[:n], it_o.keys)
        np.testing.assert_array_equal(host(plan.ids)[:n], it_o.flatten_ids)
        np.testing.assert_array_equal(host(plan.offsets), off_o)
        fr = frame.FrameResult(binding.Intersections(plan.tiles_per, plan.goff, plan.keys[:n], plan.ids[:n], n),
                               plan.offsets, plan.render)
        assert_raster_equal(scene, fr, ras_o, it_o.flatten_ids)


def test_count_into_pageable_and_pinned_memory_agree():
    """Phase 1 writes the same count through both readback paths (pageable: the copy waits; page-locked: the
    copy is asynchronous and the host waits on an event)."""
    import ctypes
    scene = SCENES["multicam-ragged-elliptical"]()
    lib = binding.load_library()
    m, r, d = dev(scene.means2d), dev(scene.radii), dev(scene.depths)
    C, N = scene.C, scene.N
    rpg = 2 if scene.radii.ndim == 3 else 1
    ws = torch.empty(lib.gs_isect_workspace_bytes(C, N, 0, scene.tile_width, scene.tile_height, 1),
                     dtype=torch.uint8, device="cuda")
    tpg = torch.empty((C, N), dtype=torch.int32, device="cuda")
    goff = torch.empty(C * N, dtype=torch.int32, device="cuda")
    s = binding._stream(None)
    pageable = ctypes.c_int64(-1)
    pinned = torch.full((1,), -1, dtype=torch.int64, pin_memory=True)
    for out in (ctypes.byref(pageable), binding._ptr(pinned)):
        binding._check(lib.gs_isect_tiles(binding._ptr(m), binding._ptr(r), rpg, binding._ptr(d), C, N,
                                          scene.tile_size, scene.tile_width, scene.tile_height, 1, binding._ptr(tpg),
                                          binding._ptr(goff), out, None, None, 0, binding._ptr(ws), ws.numel(), s))
    expected = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                                  scene.tile_height, sort=True).n_isects
    assert pageable.value == expected
    assert int(pinned[0]) == expected


@pytest.mark.parametrize("name", ["multicam-ragged-elliptical", "two-tile-passes"])
def test_isect_phase2_repeats_on_one_prefix(name):
    """Phase 2 run three times on the prefix one phase 1 left: the tile sort keeps its digit counts in that prefix
    and zeroes them as it reads them, so every run gives the oracle's sorted intersections."""
    import ctypes
    scene = (synth.random_scene(43, 3, 3000, 640, 360, 8, elliptical=True) if name == "two-tile-passes"
             else SCENES[name]())
    lib = binding.load_library()
    m, r, d = dev(scene.means2d), dev(scene.radii), dev(scene.depths)
    C, N = scene.C, scene.N
    rpg = 2 if scene.radii.ndim == 3 else 1
    expected = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                                  scene.tile_height, sort=True)
    n = expected.n_isects
    ws = torch.empty(lib.gs_isect_workspace_bytes(C, N, n, scene.tile_width, scene.tile_height, 1),
                     dtype=torch.uint8, device="cuda")
    tpg = torch.empty((C, N), dtype=torch.int32, device="cuda")
    goff = torch.empty(C * N, dtype=torch.int32, device="cuda")
    s = binding._stream(None)
    count = ctypes.c_int64(-1)
    binding._check(lib.gs_isect_tiles(binding._ptr(m), binding._ptr(r), rpg, binding._ptr(d), C, N, scene.tile_size,
                                      scene.tile_width, scene.tile_height, 1, binding._ptr(tpg), binding._ptr(goff),
                                      ctypes.byref(count), None, None, 0, binding._ptr(ws), ws.numel(), s))
    assert count.value == n
    for _ in range(3):
        keys = torch.full((n,), -1, dtype=torch.int64, device="cuda")
        ids = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        binding._check(lib.gs_isect_tiles(binding._ptr(m), binding._ptr(r), rpg, binding._ptr(d), C, N,
                                          scene.tile_size, scene.tile_width, scene.tile_height, 1, None,
                                          binding._ptr(goff), None, binding._ptr(keys), binding._ptr(ids), n,
                                          binding._ptr(ws), ws.numel(), s))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(keys_u64(keys), expected.keys)
        np.testing.assert_array_equal(host(ids), expected.flatten_ids)


def test_frame_is_deterministic():
    scene = SCENES["multicam-ragged-elliptical"]()
    a, b = gpu_frame(scene), gpu_frame(scene)
    for x, y in [(a.isect.isect_ids, b.isect.isect_ids), (a.isect.flatten_ids, b.isect.flatten_ids),
                 (a.isect_offsets, b.isect_offsets), (a.render.render_colors, b.render.render_colors),
                 (a.render.render_T, b.render.render_T), (a.render.last_ids, b.render.last_ids)]:
        assert torch.equal(x, y)


@pytest.mark.parametrize("n,end_bit,distinct", [(2, 64, 2), (100, 64, 7), (4095, 36, 50), (4096, 45, 4096),
                                                (4097, 64, 3), (14335, 40, 14335), (14336, 45, 14336),
                                                (14337, 64, 5), (28673, 47, 300), (70001, 17, 1000), (70001, 1, 2),
                                                (300000, 47, 20000), (1 << 20, 64, 1 << 20), (1000, 0, 5)])
def test_sort_keys_random(n, end_bit, distinct):
    rng = np.random.default_rng(n + end_bit)
    pool = rng.integers(0, 2 ** 63, size=distinct, dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, size=distinct).astype(np.uint64)
    keys = pool[rng.integers(0, distinct, size=n)]
    ids = rng.integers(-2 ** 31, 2 ** 31 - 1, size=n).astype(np.int32)
    mask = np.uint64((1 << end_bit) - 1) if end_bit < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
    # oracle: stable sort of the masked keys carrying positions -> the expected permutation
    _, perm = oracle.sort_pairs(keys & mask, np.arange(n, dtype=np.int32))
    kg, ig = dev(keys.view(np.int64)), dev(ids)
    binding.gs_sort_keys(kg, ig, end_bit=end_bit)
    np.testing.assert_array_equal(keys_u64(kg), keys[perm])
    np.testing.assert_array_equal(host(ig), ids[perm])


def test_ranges_validation_errors():
    # a key whose camera field is outside C, and keys out of tile order
    tw, th = 4, 4
    bad = np.array([0, (1 << 4) << 32], np.uint64)  # tile_bits 4: upper 16 -> camera 1 with C = 1
    with pytest.raises(binding.GsError) as e:
        binding.gs_tile_ranges(dev(bad.view(np.int64)), 1, tw, th, validate=True)
    assert e.value.status == binding.GS_ERR_OUT_OF_GRID
    unsorted = np.array([5 << 32, 2 << 32], np.uint64)
    with pytest.raises(binding.GsError) as e:
        binding.gs_tile_ranges(dev(unsorted.view(np.int64)), 1, tw, th, validate=True)
    assert e.value.status == binding.GS_ERR_INVALID_ARG
    # without validation the same input is accepted and the writes stay inside the offsets array
    binding.gs_tile_ranges(dev(bad.view(np.int64)), 1, tw, th, validate=False)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "dense-early-out", "ts32-ppt4", "multicam-ragged-elliptical", "K1",
                                  "cull-edges", "ts8-margin"])
def test_eval_counter_matches_oracle(name):
    # the composite's optional work counter: evaluations per pixel up to and including the stopping splat
    scene = SCENES[name]()
    it_o, off_o, ras_o = oracle.scene_pipeline(scene)
    from tile_binned_gaussian_amd import frame
    ds = frame.to_device(scene)
    it = binding.gs_isect_tiles(ds.means2d, ds.radii, ds.depths, ds.tile_size, ds.tile_width, ds.tile_height)
    off = binding.gs_tile_ranges(it.isect_ids, ds.C, ds.tile_width, ds.tile_height)
    counts = torch.zeros(5, dtype=torch.int64, device="cuda")
    ren = binding.gs_rasterize_fwd(ds.means2d, ds.conics, ds.colors, ds.opacities, ds.backgrounds, ds.width,
                                   ds.height, ds.tile_size, off, it.flatten_ids, it.n_isects, eval_counts=counts)
    c = host(counts)
    assert c[0] == ras_o.n_eval
    assert c[0] >= c[1] >= c[2]
    assert c[0] >= c[3] >= c[1]  # the kernel never evaluates more than the definition, nor skips a contributor
    assert c[4] <= it.n_isects
    # every pixel with a last id composited at least one splat
    assert c[2] >= int((host(ren.last_ids) >= 0).sum())
    np.testing.assert_array_equal(host(ren.render_T), ras_o.render_T)


@pytest.mark.parametrize("name", ["multicam-ragged-elliptical", "dense-early-out", "ts8-margin", "ts32-ppt4", "K1"])
def test_masked_composite_matches_oracle(name):
    """Per-tile masks: masked tiles composite nothing, the rest is unchanged (bit-exact with the oracle)."""
    scene = SCENES[name]()
    it_o = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                              scene.tile_height, sort=True)
    off_o = oracle.tile_offsets(it_o.keys, scene.C, scene.tile_width, scene.tile_height)
    masks = (np.random.default_rng(len(name)).uniform(size=off_o.shape) < 0.6).astype(np.int32)
    ras_o = oracle.rasterize_fwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                                 scene.width, scene.height, scene.tile_size, off_o, it_o.flatten_ids, it_o.n_isects,
                                 scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold, masks=masks)
    fr = gpu_frame(scene)
    ren = binding.gs_rasterize_fwd(dev(scene.means2d), dev(scene.conics), dev(scene.colors), dev(scene.opacities),
                                   None if scene.backgrounds is None else dev(scene.backgrounds), scene.width,
                                   scene.height, scene.tile_size, fr.isect_offsets, fr.isect.flatten_ids,
                                   fr.isect.n_isects, scene.alpha_cutoff, scene.alpha_clamp,
                                   scene.transmittance_threshold, masks=dev(masks))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ren.render_colors), ras_o.render_colors)
    np.testing.assert_array_equal(host(ren.render_T), ras_o.render_T)
    np.testing.assert_array_equal(host(ren.last_ids) >= 0, ras_o.last_ids >= 0)

"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding and the oracle on the same
seeded inputs, and compare."""
import numpy as np
import torch

import oracle
from tile_binned_gaussian_amd import binding, frame


def require_gpu():
    assert torch.cuda.is_available(), "these tests need a ROCm GPU"
    binding.load_library()  # fails loudly if the HIP library is not built


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def gpu_isect(scene, sort):
    it = binding.gs_isect_tiles(dev(scene.means2d), dev(scene.radii), dev(scene.depths), scene.tile_size,
                                scene.tile_width, scene.tile_height, sort=sort)
    torch.cuda.synchronize()
    return it


def keys_u64(t):
    return host(t).view(np.uint64)


def assert_isect_equal(scene, it_gpu, it_orc, sorted_):
    np.testing.assert_array_equal(host(it_gpu.tiles_per_gauss), it_orc.tiles_per_gauss)
    np.testing.assert_array_equal(host(it_gpu.gauss_offsets).astype(np.int64), it_orc.gauss_offsets)
    assert it_gpu.n_isects == it_orc.n_isects
    np.testing.assert_array_equal(keys_u64(it_gpu.isect_ids), it_orc.keys)
    np.testing.assert_array_equal(host(it_gpu.flatten_ids), it_orc.flatten_ids)


def oracle_lists(scene, openmp=False):
    """The oracle's sorted intersections and tile offsets of a scene: the only lists any oracle call in the GPU tests
    is given (never the GPU's). openmp: the oracle's OpenMP build (the same result)."""
    it = oracle.isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                            scene.tile_height, sort=True, openmp=openmp)
    off = oracle.tile_offsets(it.keys, scene.C, scene.tile_width, scene.tile_height)
    return it, off


def oracle_frame(scene, masks=None, openmp=False):
    """The oracle's whole frame: sorted intersections, tile offsets and the composite over them (openmp: the
    OpenMP build, the same bits)."""
    it, off = oracle_lists(scene, openmp=openmp)
    ras = oracle.rasterize_fwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                               scene.width, scene.height, scene.tile_size, off, it.flatten_ids, it.n_isects,
                               scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold, masks=masks,
                               openmp=openmp)
    return it, off, ras


def gpu_frame(scene):
    ds = frame.to_device(scene)
    fr = frame.render_frame(ds)
    torch.cuda.synchronize()
    return fr


def last_splat(last, ids):
    """Splat named by each last-composited index (-1 where nothing was composited)."""
    last = np.asarray(last, np.int64)
    if ids.size == 0:
        assert (last == -1).all()
        return last
    return np.where(last >= 0, ids[np.maximum(last, 0)], -1)


def assert_raster_equal(scene, fr_gpu, ras_orc, orc_ids):
    """Bit-exact colours, alphas and T; last ids compared as the splat they name."""
    np.testing.assert_array_equal(host(fr_gpu.render.render_colors), ras_orc.render_colors)
    np.testing.assert_array_equal(host(fr_gpu.render.render_T), ras_orc.render_T)
    np.testing.assert_array_equal(host(fr_gpu.render.render_alphas), ras_orc.render_alphas)
    g_last = host(fr_gpu.render.last_ids).astype(np.int64)
    o_last = ras_orc.last_ids.astype(np.int64)
    g_ids = host(fr_gpu.isect.flatten_ids)
    np.testing.assert_array_equal(last_splat(g_last, g_ids), last_splat(o_last, orc_ids))
    # within tolerance too (the bar stated for colour and transmittance)
    np.testing.assert_allclose(host(fr_gpu.render.render_colors), ras_orc.render_colors, atol=1e-4, rtol=0)

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


def sampled_tiles(offsets, n_isects, count, seed):
    """The heaviest tiles plus a seeded random sample (global tile indices)."""
    flat = offsets.reshape(-1).astype(np.int64)
    lengths = np.diff(np.append(flat, n_isects))
    heavy = np.argsort(-lengths, kind="stable")[: count // 4]
    rng = np.random.default_rng(seed)
    rand = rng.choice(flat.size, size=min(flat.size, count - heavy.size), replace=False)
    return np.unique(np.concatenate([heavy, rand]))


def check_tiles_against_oracle(scene, fr_gpu, tiles):
    """Composite the sampled tiles in the oracle from its own per-tile lists and compare to the GPU frame."""
    off_g = host(fr_gpu.isect_offsets).reshape(-1).astype(np.int64)
    ids_g = host(fr_gpu.isect.flatten_ids)
    n = fr_gpu.isect.n_isects
    lists = oracle.tile_lists(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                              scene.tile_height, tiles)
    col_g = host(fr_gpu.render.render_colors)
    T_g = host(fr_gpu.render.render_T)
    last_g = host(fr_gpu.render.last_ids)
    ts, tw, th = scene.tile_size, scene.tile_width, scene.tile_height
    for t, lst in zip(tiles, lists):
        s = off_g[t]
        e = off_g[t + 1] if t + 1 < off_g.size else n
        np.testing.assert_array_equal(ids_g[s:e], lst, err_msg=f"tile {t} list")
        oc, oT, ol, _ = oracle.rasterize_tile(scene.means2d, scene.conics, scene.colors, scene.opacities,
                                              scene.backgrounds, scene.width, scene.height, ts, tw, th, t, lst,
                                              scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold)
        cam, local = divmod(int(t), tw * th)
        ty, tx = divmod(local, tw)
        y0, x0 = ty * ts, tx * ts
        y1, x1 = min(y0 + ts, scene.height), min(x0 + ts, scene.width)
        np.testing.assert_array_equal(col_g[cam, y0:y1, x0:x1], oc[: y1 - y0, : x1 - x0], err_msg=f"tile {t}")
        np.testing.assert_array_equal(T_g[cam, y0:y1, x0:x1], oT[: y1 - y0, : x1 - x0], err_msg=f"tile {t}")
        gl = last_g[cam, y0:y1, x0:x1].astype(np.int64)
        olp = ol[: y1 - y0, : x1 - x0]
        np.testing.assert_array_equal(last_splat(gl, ids_g), last_splat(olp, lst), err_msg=f"tile {t} last ids")
        assert ((gl == -1) | ((gl >= s) & (gl < e))).all()

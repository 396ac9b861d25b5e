"""CPU oracle for the tile-binned splat rasterizer (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may import this package. The
product path (``tile_binned_gaussian_amd``) never imports, links or runs it, and this package never imports the
product path: the two share only the seeded inputs from ``tile_binned_gaussian_amd.synth``.

The arithmetic lives in ``gs_oracle.c`` (plain C, float32 where the pages compute in float, no contraction);
this module marshals numpy arrays into it. Definitions are cited in the C file.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")  # the same source built with OpenMP (the composite's tile loop)
_lib = None
_lib_omp = None

OK, ERR_INVALID_ARG, ERR_OUT_OF_GRID, ERR_NOMEM = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math: float32 results are reproducible), once as is and
    once with OpenMP; the tests use the first."""
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall", "-fPIC", "-shared"]
    for out, extra in ((_LIB, ["-Wno-unknown-pragmas"]), (_LIB_OMP, ["-fopenmp"])):
        if force or not os.path.exists(out):
            tmp = out + ".tmp"
            subprocess.check_call(["gcc", *flags, *extra, _SRC, "-o", tmp, "-lm"])
            os.replace(tmp, out)
    return _LIB


def _load(openmp: bool = False):
    global _lib, _lib_omp
    if (_lib_omp if openmp else _lib) is None:
        path = _LIB_OMP if openmp else _LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
        lib = _declare(ctypes.CDLL(path))
        if openmp:
            _lib_omp = lib
        else:
            _lib = lib
    return _lib_omp if openmp else _lib


@contextlib.contextmanager
def variant(path):
    """Runs the wrappers of this module against another build of the oracle's source (the tests' mutated copies,
    each with one planted mistake) instead of liboracle.so, for the duration of the block."""
    global _lib
    saved = _load()
    _lib = _declare(ctypes.CDLL(path))
    try:
        yield _lib
    finally:
        _lib = saved


def _declare(lib):
    """Declares every exported signature on a loaded build of gs_oracle.c."""
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.orc_bits_for.argtypes, lib.orc_bits_for.restype = [I64], I32
    lib.orc_threads.argtypes, lib.orc_threads.restype = [], I32
    lib.orc_bounds.argtypes = [F, F, F, F, I32, I32, I32, P]
    lib.orc_bounds.restype = None
    lib.orc_isect_count.argtypes = [P, P, I32, I64, I64, I32, I32, I32, P, P]
    lib.orc_isect_count.restype = I64
    lib.orc_isect_emit.argtypes = [P, P, I32, P, I64, I64, I32, I32, I32, P, P]
    lib.orc_isect_emit.restype = I32
    lib.orc_sort_pairs.argtypes, lib.orc_sort_pairs.restype = [P, P, I64], I32
    lib.orc_tile_offsets.argtypes, lib.orc_tile_offsets.restype = [P, I64, I64, I32, I32, P], I32
    lib.orc_exp_neg.argtypes, lib.orc_exp_neg.restype = [F], F
    lib.orc_exp_neg_array.argtypes, lib.orc_exp_neg_array.restype = [P, P, I64], None
    lib.orc_composite_pixel.argtypes = [P, P, P, P, I32, P, I64, I64, I32, I32, F, F, F, P, P, P, P]
    lib.orc_composite_pixel.restype = None
    lib.orc_rasterize_fwd.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I32, I32, I32, P, P, I64, P, F, F, F,
                                      P, I64, P, P, P, P]
    lib.orc_rasterize_fwd.restype = I64
    lib.orc_rasterize_fwd_traced.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I32, I32, I32, P, P, I64, P, F,
                                             F, F, P, I64, I64, I64, P, P, P, P, P, P]
    lib.orc_rasterize_fwd_traced.restype = I64
    lib.orc_composite_pixel_traced.argtypes = [P, P, P, P, I32, P, I64, I64, I32, I32, F, F, F, I64, P, P, P,
                                               P, P, P]
    lib.orc_composite_pixel_traced.restype = None
    lib.orc_tile_lists.argtypes = [P, P, I32, P, I64, I64, I32, I32, I32, P, I64, P, P]
    lib.orc_tile_lists.restype = I64
    lib.orc_rasterize_tile.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, I64, P, I64, F, F, F, P, P,
                                       P]
    lib.orc_rasterize_tile.restype = I64
    lib.orc_rects.argtypes, lib.orc_rects.restype = [P, P, I32, I64, I32, I32, I32, P], None
    lib.orc_rasterize_bwd.argtypes = [P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, I32, P, P, I64, P, F,
                                      F, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.orc_rasterize_bwd.restype = I32
    lib.orc_project.argtypes = [P, P, P, P, I64, I64, I32, I32, F, F, F, F, I32, P, P, P, P, P]
    lib.orc_project.restype = None
    lib.orc_bin_tiles.argtypes = [P, P, I32, P, I64, I64, I32, I32, I32, I64, P, P]
    lib.orc_bin_tiles.restype = I64
    lib.orc_rasterize_bins.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I32, I32, I32, P, I64, F, F, F, P, P,
                                       P, P]
    lib.orc_rasterize_bins.restype = I64
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def threads(openmp: bool = False) -> int:
    """Threads the compositing loop uses in the plain (1) or the OpenMP build."""
    return int(_load(openmp).orc_threads())


def bits_for(count: int) -> int:
    """Smallest b >= 0 with 2^b >= count (tile_bits for count = w*h, camera bits for count = C)."""
    return int(_load().orc_bits_for(int(count)))


def bounds(mean_x, mean_y, radius_x, radius_y, tile_size, tile_width, tile_height):
    out = np.zeros(4, np.int32)
    _load().orc_bounds(float(mean_x), float(mean_y), float(radius_x), float(radius_y), int(tile_size),
                       int(tile_width), int(tile_height), _p(out))
    return tuple(int(v) for v in out)


@dataclass
class Isect:
    tiles_per_gauss: np.ndarray  # [C, N] int32
    gauss_offsets: np.ndarray  # [C*N] int64, exclusive prefix of the counts
    keys: np.ndarray  # [n] uint64
    flatten_ids: np.ndarray  # [n] int32
    n_isects: int


def isect_tiles(means2d, radii, depths, tile_size, tile_width, tile_height, sort=True, openmp=False,
                timings=None) -> Isect:
    """Intersections of every (camera, splat) with the tile grid, as the pages' isect_tiles returns them.
    openmp: the OpenMP build (emission and the sort's merges on the host's threads; the same result).
    timings: a dict that receives the wall time of each step in seconds (count_scan_s, emit_s, sort_s)."""
    import time
    lib = _load(openmp)
    means2d = _c(means2d, np.float32)
    radii = _c(radii, np.float32)
    depths = _c(depths, np.float32)
    C, N = means2d.shape[0], means2d.shape[1]
    rpg = 2 if radii.ndim == 3 else 1
    tiles_per = np.zeros((C, N), np.int32)
    goff = np.zeros(C * N, np.int64)
    t0 = time.perf_counter()
    n = int(lib.orc_isect_count(_p(means2d), _p(radii), rpg, C, N, tile_size, tile_width, tile_height,
                                _p(tiles_per), _p(goff)))
    t1 = time.perf_counter()
    keys = np.zeros(n, np.uint64)
    ids = np.zeros(n, np.int32)
    if lib.orc_isect_emit(_p(means2d), _p(radii), rpg, _p(depths), C, N, tile_size, tile_width, tile_height,
                          _p(keys), _p(ids)) != OK:
        raise MemoryError("oracle emission allocation failed")
    t2 = time.perf_counter()
    if sort and n > 1:
        rc = lib.orc_sort_pairs(_p(keys), _p(ids), n)
        if rc != OK:
            raise MemoryError("oracle sort allocation failed")
    t3 = time.perf_counter()
    if timings is not None:
        timings.update(count_scan_s=t1 - t0, emit_s=t2 - t1, sort_s=t3 - t2)
    return Isect(tiles_per, goff, keys, ids, n)


def sort_pairs(keys, ids):
    """Stable ascending sort by the unsigned key; returns new arrays."""
    k = np.array(keys, dtype=np.uint64, copy=True)
    i = np.array(ids, dtype=np.int32, copy=True)
    if _load().orc_sort_pairs(_p(k), _p(i), k.size) != OK:
        raise MemoryError("oracle sort allocation failed")
    return k, i


def tile_offsets(keys, C, tile_width, tile_height):
    """Per-tile exclusive offsets [C, th, tw] int32; raises ValueError for a key outside the tile grid."""
    k = _c(keys, np.uint64)
    out = np.zeros((C, tile_height, tile_width), np.int32)
    rc = _load().orc_tile_offsets(_p(k), k.size, C, tile_width, tile_height, _p(out))
    if rc == ERR_OUT_OF_GRID:
        raise ValueError("intersection key is outside the tile grid")
    if rc != OK:
        raise MemoryError("oracle offsets allocation failed")
    return out


def exp_neg(sigma) -> np.ndarray:
    """The oracle's float32 e^-sigma, elementwise."""
    s = np.ascontiguousarray(sigma, dtype=np.float32)
    out = np.empty(s.shape, np.float32)
    _load().orc_exp_neg_array(_p(s), _p(out), s.size)
    return out


def composite_pixel(means2d, conics, colors, opacities, list_ids, x, y, alpha_cutoff, alpha_clamp,
                    transmittance_threshold):
    """Composite one pixel over an explicit front-to-back list of flat splat ids.

    Returns (acc[K], T, last_position, n_eval); last_position indexes ``list_ids`` (-1 if none composited)."""
    lib = _load()
    means2d = _c(means2d, np.float32).reshape(-1, 2)
    conics = _c(conics, np.float32).reshape(-1, 3)
    K = colors.shape[-1]
    colors = _c(colors, np.float32).reshape(-1, K)
    opacities = _c(opacities, np.float32).reshape(-1)
    lst = _c(list_ids, np.int32)
    acc = np.zeros(K, np.float32)
    T = np.zeros(1, np.float32)
    last = np.zeros(1, np.int64)
    ne = np.zeros(1, np.int64)
    lib.orc_composite_pixel(_p(means2d), _p(conics), _p(colors), _p(opacities), K, _p(lst), 0, lst.size, int(x),
                            int(y), float(alpha_cutoff), float(alpha_clamp), float(transmittance_threshold),
                            _p(acc), _p(T), _p(last), _p(ne))
    return acc, float(T[0]), int(last[0]), int(ne[0])


@dataclass
class Raster:
    render_colors: np.ndarray  # [C, H, W, K]
    render_alphas: np.ndarray  # [C, H, W] = 1 - T
    render_T: np.ndarray  # [C, H, W]
    last_ids: np.ndarray  # [C, H, W] int32
    n_eval: int


def rasterize_fwd(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, isect_offsets,
                  flatten_ids, n_isects, alpha_cutoff, alpha_clamp, transmittance_threshold, tiles=None,
                  masks=None, openmp=False) -> Raster:
    """Front-to-back compositing over every tile (or only the listed global tiles; other pixels stay NaN).
    openmp: use the OpenMP build (tiles over the host's threads; the same results)."""
    lib = _load(openmp)
    means2d = _c(means2d, np.float32)
    C = means2d.shape[0]
    K = colors.shape[-1]
    off = _c(isect_offsets, np.int32)
    th, tw = off.shape[1], off.shape[2]
    colors = _c(colors, np.float32)
    bg = None if backgrounds is None else _c(backgrounds, np.float32)
    out_c = np.full((C, height, width, K), np.nan, np.float32)
    out_a = np.full((C, height, width), np.nan, np.float32)
    out_t = np.full((C, height, width), np.nan, np.float32)
    out_l = np.full((C, height, width), -2, np.int32)
    tl = None if tiles is None else _c(tiles, np.int64)
    n_eval = lib.orc_rasterize_fwd(_p(means2d), _p(_c(conics, np.float32)), _p(colors),
                                   _p(_c(opacities, np.float32)), _p(bg), C, K, width, height, tile_size, tw, th,
                                   _p(off), _p(_c(flatten_ids, np.int32)), int(n_isects),
                                   _p(None if masks is None else _c(masks, np.int32)), float(alpha_cutoff),
                                   float(alpha_clamp), float(transmittance_threshold), _p(tl),
                                   0 if tl is None else tl.size, _p(out_c), _p(out_a), _p(out_t), _p(out_l))
    if n_eval < 0:
        raise ValueError("invalid rasterize arguments")
    return Raster(out_c, out_a, out_t, out_l, int(n_eval))


@dataclass
class TracedRaster(Raster):
    trace_ids: np.ndarray  # [C, H, W, max_splat_steps] int32 flat splat ids; entries past the count hold -2
    trace_counts: np.ndarray  # [C, H, W] int32


def rasterize_fwd_traced(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, isect_offsets,
                         flatten_ids, n_isects, alpha_cutoff, alpha_clamp, transmittance_threshold, max_splat_steps,
                         max_list_entries=-1, masks=None, trace=True, tiles=None, openmp=False) -> TracedRaster:
    """The traced forward: every tile's list cut to its first ``max_list_entries`` entries (negative: whole
    lists), every pixel capped at ``max_splat_steps`` composited splats (negative: uncapped, only without a
    trace), and each pixel's composited flat splat ids recorded in order. tiles: only these global tiles (other
    pixels keep the fill values). openmp: the OpenMP build (tiles on the host's threads; the same results)."""
    lib = _load(openmp)
    means2d = _c(means2d, np.float32)
    C = means2d.shape[0]
    K = colors.shape[-1]
    off = _c(isect_offsets, np.int32)
    th, tw = off.shape[1], off.shape[2]
    colors = _c(colors, np.float32)
    bg = None if backgrounds is None else _c(backgrounds, np.float32)
    S = int(max_splat_steps)
    out_c = np.full((C, height, width, K), np.nan, np.float32)
    out_a = np.full((C, height, width), np.nan, np.float32)
    out_t = np.full((C, height, width), np.nan, np.float32)
    out_l = np.full((C, height, width), -2, np.int32)
    tr = np.full((C, height, width, max(S, 0)), -2, np.int32) if trace else None
    cnt = np.full((C, height, width), -2, np.int32) if trace else None
    tl = None if tiles is None else _c(tiles, np.int64)
    n_eval = lib.orc_rasterize_fwd_traced(_p(means2d), _p(_c(conics, np.float32)), _p(colors),
                                          _p(_c(opacities, np.float32)), _p(bg), C, K, width, height, tile_size, tw,
                                          th, _p(off), _p(_c(flatten_ids, np.int32)), int(n_isects),
                                          _p(None if masks is None else _c(masks, np.int32)), float(alpha_cutoff),
                                          float(alpha_clamp), float(transmittance_threshold), _p(tl),
                                          0 if tl is None else tl.size, int(max_list_entries), S, _p(out_c),
                                          _p(out_a), _p(out_t), _p(out_l), _p(tr), _p(cnt))
    if n_eval < 0:
        raise ValueError("invalid rasterize arguments")
    return TracedRaster(out_c, out_a, out_t, out_l, int(n_eval), tr, cnt)


def composite_pixel_traced(means2d, conics, colors, opacities, list_ids, x, y, alpha_cutoff, alpha_clamp,
                           transmittance_threshold, max_steps):
    """orc_composite_pixel_traced over an explicit list: (acc[K], T, last_position, n_eval, trace of flat ids)."""
    lib = _load()
    means2d = _c(means2d, np.float32).reshape(-1, 2)
    conics = _c(conics, np.float32).reshape(-1, 3)
    K = colors.shape[-1]
    colors = _c(colors, np.float32).reshape(-1, K)
    opacities = _c(opacities, np.float32).reshape(-1)
    lst = _c(list_ids, np.int32)
    acc = np.zeros(K, np.float32)
    T = np.zeros(1, np.float32)
    last = np.zeros(1, np.int64)
    ne = np.zeros(1, np.int64)
    steps = np.zeros(1, np.int64)
    tr = np.full(max(lst.size, 1), -2, np.int32)
    lib.orc_composite_pixel_traced(_p(means2d), _p(conics), _p(colors), _p(opacities), K, _p(lst), 0, lst.size,
                                   int(x), int(y), float(alpha_cutoff), float(alpha_clamp),
                                   float(transmittance_threshold), int(max_steps), _p(acc), _p(T), _p(last), _p(ne),
                                   _p(tr), _p(steps))
    return acc, float(T[0]), int(last[0]), int(ne[0]), tr[:int(steps[0])].copy()


def tile_lists(means2d, radii, depths, tile_size, tile_width, tile_height, tiles):
    """For each listed global tile: flat ids of the splats whose rectangle contains it, by (depth bits, id)."""
    lib = _load()
    means2d = _c(means2d, np.float32)
    radii = _c(radii, np.float32)
    depths = _c(depths, np.float32)
    C, N = means2d.shape[0], means2d.shape[1]
    rpg = 2 if radii.ndim == 3 else 1
    tl = _c(tiles, np.int64)
    counts = np.zeros(tl.size, np.int64)
    total = lib.orc_tile_lists(_p(means2d), _p(radii), rpg, _p(depths), C, N, tile_size, tile_width, tile_height,
                               _p(tl), tl.size, _p(counts), None)
    ids = np.zeros(max(total, 0), np.int32)
    lib.orc_tile_lists(_p(means2d), _p(radii), rpg, _p(depths), C, N, tile_size, tile_width, tile_height,
                       _p(tl), tl.size, _p(counts), _p(ids))
    out, pos = [], 0
    for c in counts:
        out.append(ids[pos:pos + int(c)])
        pos += int(c)
    return out


@dataclass
class Bins:
    bin_ids: np.ndarray  # [C, th, tw, capacity] int32 flat ids by (depth bits, id), -1 in empty slots
    bin_counts: np.ndarray  # [C, th, tw] int32 full count (> capacity when the bin overflowed)
    largest: int


def bin_tiles(means2d, radii, depths, tile_size, tile_width, tile_height, capacity) -> Bins:
    """Fixed-capacity per-tile bins (orc_bin_tiles)."""
    lib = _load()
    means2d = _c(means2d, np.float32)
    radii = _c(radii, np.float32)
    C, N = means2d.shape[0], means2d.shape[1]
    rpg = 2 if radii.ndim == 3 else 1
    ids = np.full((C, tile_height, tile_width, int(capacity)), -2, np.int32)
    counts = np.full((C, tile_height, tile_width), -2, np.int32)
    largest = lib.orc_bin_tiles(_p(means2d), _p(radii), rpg, _p(_c(depths, np.float32)), C, N, tile_size, tile_width,
                                tile_height, int(capacity), _p(ids), _p(counts))
    if largest < 0:
        raise ValueError("invalid bin arguments")
    return Bins(ids, counts, int(largest))


def rasterize_bins(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, bin_ids,
                   alpha_cutoff, alpha_clamp, transmittance_threshold) -> Raster:
    """Compositing over fixed-capacity bins [C, th, tw, capacity] (orc_rasterize_bins); last ids are bin
    positions."""
    lib = _load()
    means2d = _c(means2d, np.float32)
    C = means2d.shape[0]
    K = colors.shape[-1]
    bins = _c(bin_ids, np.int32)
    th, tw, cap = bins.shape[1], bins.shape[2], bins.shape[3]
    bg = None if backgrounds is None else _c(backgrounds, np.float32)
    out_c = np.full((C, height, width, K), np.nan, np.float32)
    out_a = np.full((C, height, width), np.nan, np.float32)
    out_t = np.full((C, height, width), np.nan, np.float32)
    out_l = np.full((C, height, width), -2, np.int32)
    n_eval = lib.orc_rasterize_bins(_p(means2d), _p(_c(conics, np.float32)), _p(_c(colors, np.float32)),
                                    _p(_c(opacities, np.float32)), _p(bg), C, K, width, height, tile_size, tw, th,
                                    _p(bins), cap, float(alpha_cutoff), float(alpha_clamp),
                                    float(transmittance_threshold), _p(out_c), _p(out_a), _p(out_t), _p(out_l))
    if n_eval < 0:
        raise ValueError("invalid rasterize arguments")
    return Raster(out_c, out_a, out_t, out_l, int(n_eval))


def rasterize_tile(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, tile_width,
                   tile_height, tile, list_ids, alpha_cutoff, alpha_clamp, transmittance_threshold):
    """Composite one global tile over an explicit front-to-back list of flat ids.

    Returns (colors [ts, ts, K], T [ts, ts], last_pos [ts, ts] indexing list_ids, n_eval); pixels outside the image
    hold NaN / -2."""
    lib = _load()
    K = colors.shape[-1]
    lst = _c(list_ids, np.int32)
    oc = np.full((tile_size, tile_size, K), np.nan, np.float32)
    ot = np.full((tile_size, tile_size), np.nan, np.float32)
    ol = np.full((tile_size, tile_size), -2, np.int64)
    bg = None if backgrounds is None else _c(backgrounds, np.float32)
    ne = lib.orc_rasterize_tile(_p(_c(means2d, np.float32)), _p(_c(conics, np.float32)), _p(_c(colors, np.float32)),
                                _p(_c(opacities, np.float32)), _p(bg), K, width, height, tile_size, tile_width,
                                tile_height, int(tile), _p(lst), lst.size, float(alpha_cutoff), float(alpha_clamp),
                                float(transmittance_threshold), _p(oc), _p(ot), _p(ol))
    return oc, ot, ol, int(ne)


def rects(means2d, radii, tile_size, tile_width, tile_height):
    """[C*N, 4] int32 tile rectangles (x0, y0, x1, y1)."""
    means2d = _c(means2d, np.float32)
    radii = _c(radii, np.float32)
    M = means2d.shape[0] * means2d.shape[1]
    out = np.zeros((M, 4), np.int32)
    _load().orc_rects(_p(means2d), _p(radii), 2 if radii.ndim == 3 else 1, M, tile_size, tile_width, tile_height,
                      _p(out))
    return out


@dataclass
class RasterGrad:
    """Exact gradients (float64) of L = sum(grad_colors * render_colors) + sum(grad_alphas * render_alphas); per entry
    the sum of the terms' magnitudes (abs_*) and the derived bound on how far a float32 evaluation of each term by
    the pages' recurrence may lie from it (err_*, summed over the entry's terms). A float32 result summed in any order
    with at most D additions on a path lies within err + D * 2^-24 * abs of the exact gradient (to first order)."""
    means2d: np.ndarray  # [C, N, 2]
    conics: np.ndarray  # [C, N, 3]
    colors: np.ndarray  # [C, N, K]
    opacities: np.ndarray  # [C, N]
    backgrounds: np.ndarray | None  # [C, K]
    means2d_abs: np.ndarray  # [C, N, 2]
    abs_means2d: np.ndarray
    abs_conics: np.ndarray
    abs_colors: np.ndarray
    abs_opacities: np.ndarray
    abs_backgrounds: np.ndarray | None
    err_means2d: np.ndarray
    err_conics: np.ndarray
    err_colors: np.ndarray
    err_opacities: np.ndarray
    err_backgrounds: np.ndarray | None

    def bound(self, field, adds):
        """|float result - exact| bound of one output: err + (adds + 2) * 2^-24 * abs, widened by 2% for the
        first-order analysis (adds: the summation depth, an array broadcast against the field)."""
        u = 2.0 ** -24
        return 1.02 * (getattr(self, "err_" + field) + (np.asarray(adds, np.float64) + 2.0) * u *
                       getattr(self, "abs_" + field)) + 1e-30


def rasterize_bwd(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, isect_offsets,
                  flatten_ids, n_isects, alpha_cutoff, alpha_clamp, render_alphas, last_ids, grad_colors,
                  grad_alphas, masks=None) -> RasterGrad:
    """Exact backward of the composite over every tile (orc_rasterize_bwd), with magnitudes and error bounds."""
    lib = _load()
    means2d = _c(means2d, np.float32)
    C, N = means2d.shape[0], means2d.shape[1]
    K = colors.shape[-1]
    off = _c(isect_offsets, np.int32)
    th, tw = off.shape[1], off.shape[2]
    bg = None if backgrounds is None else _c(backgrounds, np.float32)
    z = lambda *shape: np.zeros(shape, np.float64)  # noqa: E731
    g = [z(C, N, 2), z(C, N, 3), z(C, N, K), z(C, N), None if bg is None else z(C, K), z(C, N, 2)]
    a = [z(C, N, 2), z(C, N, 3), z(C, N, K), z(C, N), None if bg is None else z(C, K)]
    e = [z(C, N, 2), z(C, N, 3), z(C, N, K), z(C, N), None if bg is None else z(C, K)]
    rc = lib.orc_rasterize_bwd(_p(means2d), _p(_c(conics, np.float32)), _p(_c(colors, np.float32)),
                               _p(_c(opacities, np.float32)), _p(bg), C, N, K, width, height, tile_size, tw, th,
                               _p(off), _p(_c(flatten_ids, np.int32)), int(n_isects),
                               _p(None if masks is None else _c(masks, np.int32)), float(alpha_cutoff),
                               float(alpha_clamp), _p(_c(render_alphas, np.float32)), _p(_c(last_ids, np.int32)),
                               _p(_c(grad_colors, np.float32)), _p(_c(grad_alphas, np.float32)),
                               *[_p(x) for x in g], *[_p(x) for x in a], *[_p(x) for x in e])
    if rc == -2:
        raise MemoryError("oracle backward allocation failed")
    if rc != 0:
        raise ValueError("invalid rasterize backward arguments")
    return RasterGrad(*g, *a, *e)


@dataclass
class Projection:
    radii: np.ndarray  # [C, N, 2] int32
    means2d: np.ndarray  # [C, N, 2]
    depths: np.ndarray  # [C, N]
    conics: np.ndarray  # [C, N, 3]
    compensations: np.ndarray | None  # [C, N]


def project(means, covars, viewmats, Ks, width, height, eps2d=0.3, near_plane=0.01, far_plane=1e10,
            radius_clip=0.0, compensation=False, orthographic=False) -> Projection:
    """EWA projection of [N, 3] means and [N, 3, 3] covariances into C cameras ([C, 4, 4] views, [C, 3, 3] K)."""
    lib = _load()
    means = _c(means, np.float32)
    N = means.shape[0]
    views = _c(viewmats, np.float32)
    C = views.shape[0]
    radii = np.zeros((C, N, 2), np.int32)
    m2 = np.zeros((C, N, 2), np.float32)
    dep = np.zeros((C, N), np.float32)
    con = np.zeros((C, N, 3), np.float32)
    comp = np.zeros((C, N), np.float32) if compensation else None
    lib.orc_project(_p(means), _p(_c(covars, np.float32)), _p(views), _p(_c(Ks, np.float32)), C, N, int(width),
                    int(height), float(eps2d), float(near_plane), float(far_plane), float(radius_clip),
                    int(bool(orthographic)), _p(radii), _p(m2), _p(dep), _p(con), _p(comp))
    return Projection(radii, m2, dep, con, comp)


def scene_pipeline(scene, sort=True):
    """Whole path on the CPU for a synth.Scene: intersections, offsets and the composite."""
    it = isect_tiles(scene.means2d, scene.radii, scene.depths, scene.tile_size, scene.tile_width,
                     scene.tile_height, sort=sort)
    off = tile_offsets(it.keys, scene.C, scene.tile_width, scene.tile_height)
    ras = rasterize_fwd(scene.means2d, scene.conics, scene.colors, scene.opacities, scene.backgrounds,
                        scene.width, scene.height, scene.tile_size, off, it.flatten_ids, it.n_isects,
                        scene.alpha_cutoff, scene.alpha_clamp, scene.transmittance_threshold)
    return it, off, ras

"""Thin ctypes binding of libgs_raster (C ABI in include/gs_raster.h), one Python function per entry point.

Argument marshalling only: every step runs in the HIP library. PyTorch supplies device memory (tensors on a ROCm
device) and the stream (torch's current stream unless one is passed). The library must be built
(``python -m tile_binned_gaussian_amd.build``); loading fails loudly otherwise, and there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
from dataclasses import dataclass

import torch  # loads the HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgs_raster.so")

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_OUT_OF_GRID, GS_ERR_WORKSPACE, GS_ERR_DEVICE = range(5)
_STATUS = {1: "GS_ERR_INVALID_ARG", 2: "GS_ERR_OUT_OF_GRID", 3: "GS_ERR_WORKSPACE", 4: "GS_ERR_DEVICE"}

EXPORTS = ("gs_last_error", "gs_isect_workspace_bytes", "gs_isect_tiles", "gs_sort_workspace_bytes",
           "gs_sort_keys", "gs_tile_ranges_workspace_bytes", "gs_tile_ranges", "gs_rasterize_workspace_bytes",
           "gs_rasterize_fwd", "gs_rasterize_fwd_hwexp", "gs_rasterize_fwd_traced", "gs_rasterize_bwd",
           "gs_project_fwd", "gs_bin_tiles", "gs_rasterize_fwd_bins", "gs_set_spin_limit", "gs_device_check",
           "gs_sort_keys_static")


class GsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libgs_raster.so and declares every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m tile_binned_gaussian_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I64, I32, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gs_last_error.argtypes, lib.gs_last_error.restype = [], ctypes.c_char_p
    lib.gs_isect_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, I32]
    lib.gs_isect_workspace_bytes.restype = SZ
    lib.gs_isect_tiles.argtypes = [P, P, I32, P, I64, I64, I32, I32, I32, I32, P, P, P, P, P, I64, P, SZ, P]
    lib.gs_isect_tiles.restype = I32
    lib.gs_sort_workspace_bytes.argtypes, lib.gs_sort_workspace_bytes.restype = [I64, I32], SZ
    lib.gs_sort_keys.argtypes, lib.gs_sort_keys.restype = [P, P, I64, I32, P, SZ, P], I32
    lib.gs_tile_ranges_workspace_bytes.argtypes, lib.gs_tile_ranges_workspace_bytes.restype = [], SZ
    lib.gs_tile_ranges.argtypes = [P, I64, I64, I32, I32, P, I32, P, SZ, P]
    lib.gs_tile_ranges.restype = I32
    lib.gs_rasterize_workspace_bytes.argtypes = [I64, I32, I32]
    lib.gs_rasterize_workspace_bytes.restype = SZ
    lib.gs_rasterize_fwd.argtypes = [P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, I32, P, P, I64, P, F, F, F,
                                     P, P, P, P, P, P, SZ, P]
    lib.gs_rasterize_fwd.restype = I32
    lib.gs_rasterize_fwd_hwexp.argtypes = [P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, I32, P, P, I64, P, F, F,
                                           F, P, P, P, P, P, P]
    lib.gs_rasterize_fwd_hwexp.restype = I32
    lib.gs_rasterize_fwd_traced.argtypes = [P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, I32, P, P, I64, P, F,
                                            F, F, I32, I32, P, P, P, P, P, P, P, P, SZ, P]
    lib.gs_rasterize_fwd_traced.restype = I32
    lib.gs_bin_tiles.argtypes = [P, P, I32, P, I64, I64, I32, I32, I32, I32, P, P, P]
    lib.gs_bin_tiles.restype = I32
    lib.gs_rasterize_fwd_bins.argtypes = [P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, I32, P, P, I32, F, F, F,
                                          P, P, P, P, P, P]
    lib.gs_rasterize_fwd_bins.restype = I32
    lib.gs_rasterize_bwd.argtypes = [P, P, P, P, P, I64, I64, I32, I32, I32, I32, I32, I32, P, P, I64, P, F, F,
                                     P, P, P, P, P, P, P, P, P, P, P]
    lib.gs_rasterize_bwd.restype = I32
    lib.gs_project_fwd.argtypes = [P, P, P, P, I64, I64, I32, I32, F, F, F, F, I32, P, P, P, P, P, P]
    lib.gs_project_fwd.restype = I32
    lib.gs_sort_keys_static.argtypes, lib.gs_sort_keys_static.restype = [P, P, I64, I32, P], I32
    lib.gs_set_spin_limit.argtypes, lib.gs_set_spin_limit.restype = [ctypes.c_uint32], ctypes.c_uint32
    lib.gs_device_check.argtypes, lib.gs_device_check.restype = [P], I32
    _lib = lib
    return lib


def _check(status: int):
    if status != GS_OK:
        raise GsError(status, _lib.gs_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_scoped(fn):
    """Runs fn with its `stream` argument (when one is given) as torch's current stream, so that every buffer the
    call allocates - workspaces, outputs, a grown workspace and the copy into it - belongs to the stream its
    kernels run on: torch's caching allocator then never hands such a buffer to another stream while work queued
    on this one may still use it, and the copy is ordered after the work that produced its source."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrapper


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _req_layout(t, name, dtype, shape=None):
    """Type, dtype, shape and contiguity of one argument (no device check)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _req(t, name, dtype, device=None, shape=None):
    _req_layout(t, name, dtype, shape)
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


@dataclass
class Intersections:
    tiles_per_gauss: torch.Tensor  # [C, N] int32
    gauss_offsets: torch.Tensor  # [C*N] int32
    isect_ids: torch.Tensor  # [n] int64 (the u64 key bits)
    flatten_ids: torch.Tensor  # [n] int32
    n_isects: int


@_stream_scoped
def gs_isect_tiles(means2d, radii, depths, tile_size, tile_width, tile_height, sort=True, stream=None,
                   workspace=None) -> Intersections:
    """Both phases of gs_isect_tiles: count (synchronises once for the size), then emit (and sort)."""
    lib = load_library()
    dev = means2d.device
    _req(means2d, "means2d", torch.float32, dev)
    if means2d.dim() != 3 or means2d.shape[2] != 2:
        raise ValueError("means2d must be [C, N, 2]")
    C, N = means2d.shape[0], means2d.shape[1]
    _req(radii, "radii", torch.float32, dev)
    if tuple(radii.shape) == (C, N):
        rpg = 1
    elif tuple(radii.shape) == (C, N, 2):
        rpg = 2
    else:
        raise ValueError(f"radii must be [C, N] or [C, N, 2] (got {tuple(radii.shape)})")
    _req(depths, "depths", torch.float32, dev, (C, N))
    s = _stream(stream)
    tiles_per = torch.empty((C, N), dtype=torch.int32, device=dev)
    goff = torch.empty(C * N, dtype=torch.int32, device=dev)
    n_out = ctypes.c_int64(0)
    ws = workspace if workspace is not None else _workspace(
        lib.gs_isect_workspace_bytes(C, N, 0, tile_width, tile_height, int(bool(sort))), dev)
    _check(lib.gs_isect_tiles(_ptr(means2d), _ptr(radii), rpg, _ptr(depths), C, N, tile_size, tile_width,
                              tile_height, int(bool(sort)), _ptr(tiles_per), _ptr(goff), ctypes.byref(n_out), None,
                              None, 0, _ptr(ws), ws.numel(), s))
    n = int(n_out.value)
    keys = torch.empty(n, dtype=torch.int64, device=dev)
    ids = torch.empty(n, dtype=torch.int32, device=dev)
    if n == 0:
        return Intersections(tiles_per, goff, keys, ids, n)
    need = lib.gs_isect_workspace_bytes(C, N, n, tile_width, tile_height, int(bool(sort)))
    if ws.numel() < need:
        # phase 1 left the depth order at the start of the workspace; phase 2 reads it there
        prefix = lib.gs_isect_workspace_bytes(C, N, 0, tile_width, tile_height, int(bool(sort)))
        grown = _workspace(need, dev)
        grown[:prefix].copy_(ws[:prefix])
        ws = grown
    _check(lib.gs_isect_tiles(_ptr(means2d), _ptr(radii), rpg, _ptr(depths), C, N, tile_size, tile_width,
                              tile_height, int(bool(sort)), None, _ptr(goff), None, _ptr(keys), _ptr(ids), n,
                              _ptr(ws), ws.numel(), s))
    return Intersections(tiles_per, goff, keys, ids, n)


@_stream_scoped
def gs_sort_keys(keys, flatten_ids, end_bit=64, stream=None, workspace=None):
    """Stable in-place sort of (keys, flatten_ids) by bits [0, end_bit) of the keys."""
    lib = load_library()
    _req(keys, "keys", torch.int64)
    _req(flatten_ids, "flatten_ids", torch.int32, keys.device, (keys.numel(),))
    n = keys.numel()
    ws = workspace if workspace is not None else _workspace(lib.gs_sort_workspace_bytes(n, end_bit), keys.device)
    _check(lib.gs_sort_keys(_ptr(keys), _ptr(flatten_ids), n, end_bit, _ptr(ws), ws.numel(), _stream(stream)))
    return keys, flatten_ids


def gs_sort_keys_static(keys, flatten_ids, end_bit=64, stream=None):
    """gs_sort_keys without a workspace (the library's static scratch; at most 2^22 pairs; allocates nothing).
    Calls that overlap on one GPU race."""
    lib = load_library()
    _req(keys, "keys", torch.int64)
    _req(flatten_ids, "flatten_ids", torch.int32, keys.device, (keys.numel(),))
    _check(lib.gs_sort_keys_static(_ptr(keys), _ptr(flatten_ids), keys.numel(), end_bit, _stream(stream)))
    return keys, flatten_ids


def gs_set_spin_limit(limit: int) -> int:
    """Look-back rounds a sort partition may wait before it gives up (passes launched afterwards); returns the
    previous limit."""
    return int(load_library().gs_set_spin_limit(int(limit)))


def gs_device_check(stream=None):
    """Synchronises the stream, then raises GsError (GS_ERR_DEVICE) if a sort's bounded wait gave up on this GPU
    since the last check (the device error word is cleared either way)."""
    _check(load_library().gs_device_check(_stream(stream)))


@_stream_scoped
def gs_tile_ranges(sorted_keys, C, tile_width, tile_height, validate=False, out=None, stream=None,
                   workspace=None):
    """Per-tile offsets [C, th, tw] int32 of sorted keys (boundary detection)."""
    lib = load_library()
    _req(sorted_keys, "sorted_keys", torch.int64)
    dev = sorted_keys.device
    if out is None:
        out = torch.empty((C, tile_height, tile_width), dtype=torch.int32, device=dev)
    _req(out, "isect_offsets", torch.int32, dev, (C, tile_height, tile_width))
    ws = workspace if workspace is not None else _workspace(lib.gs_tile_ranges_workspace_bytes(), dev)
    _check(lib.gs_tile_ranges(_ptr(sorted_keys), sorted_keys.numel(), C, tile_width, tile_height, _ptr(out),
                              int(bool(validate)), _ptr(ws), ws.numel(), _stream(stream)))
    return out


@dataclass
class Render:
    render_colors: torch.Tensor  # [C, H, W, K]
    render_alphas: torch.Tensor  # [C, H, W]
    render_T: torch.Tensor  # [C, H, W]
    last_ids: torch.Tensor  # [C, H, W] int32


def _raster_inputs(means2d, conics, colors, opacities, backgrounds, isect_offsets, flatten_ids, masks):
    dev = means2d.device
    _req(means2d, "means2d", torch.float32, dev)
    C, N = means2d.shape[0], means2d.shape[1]
    _req(conics, "conics", torch.float32, dev, (C, N, 3))
    _req(colors, "colors", torch.float32, dev)
    if colors.dim() != 3 or tuple(colors.shape[:2]) != (C, N):
        raise ValueError("colors must be [C, N, K]")
    _req(opacities, "opacities", torch.float32, dev, (C, N))
    if backgrounds is not None:
        _req(backgrounds, "backgrounds", torch.float32, dev, (C, colors.shape[2]))
    _req(isect_offsets, "isect_offsets", torch.int32, dev)
    if isect_offsets.dim() != 3 or isect_offsets.shape[0] != C:
        raise ValueError("isect_offsets must be [C, th, tw]")
    _req(flatten_ids, "flatten_ids", torch.int32, dev)
    if masks is not None:
        _req(masks, "masks", torch.int32, dev, tuple(isect_offsets.shape))
    return dev, C, N, colors.shape[2], isect_offsets.shape[1], isect_offsets.shape[2]


def _render_out(C, height, width, K, dev):
    return Render(torch.empty((C, height, width, K), dtype=torch.float32, device=dev),
                  torch.empty((C, height, width), dtype=torch.float32, device=dev),
                  torch.empty((C, height, width), dtype=torch.float32, device=dev),
                  torch.empty((C, height, width), dtype=torch.int32, device=dev))


def _check_render_out(out, C, height, width, K, dev):
    """A caller-supplied output set must match the image batch (the kernels write every pixel of it): every
    field's layout is checked first, then its device."""
    fields = [(out.render_colors, "render_colors", torch.float32, (C, height, width, K)),
              (out.render_alphas, "render_alphas", torch.float32, (C, height, width)),
              (out.render_T, "render_T", torch.float32, (C, height, width)),
              (out.last_ids, "last_ids", torch.int32, (C, height, width))]
    fields = [f for i, f in enumerate(fields) if i < 2 or f[0] is not None]
    for t, name, dtype, shape in fields:
        _req_layout(t, name, dtype, shape)
    for t, name, dtype, shape in fields:
        _req(t, name, dtype, dev, shape)


def _n_isects(flatten_ids, n_isects):
    """The intersection count the kernels may index: flatten_ids' length, or a given count that fits in it."""
    n = flatten_ids.numel() if n_isects is None else int(n_isects)
    if n < 0 or n > flatten_ids.numel():
        raise ValueError(f"n_isects = {n} outside [0, flatten_ids.numel() = {flatten_ids.numel()}]")
    return n


def _check_eval_counts(eval_counts, dev):
    if eval_counts is not None:
        _req(eval_counts, "eval_counts", torch.int64, dev, (5,))


@_stream_scoped
def gs_rasterize_fwd(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, isect_offsets,
                     flatten_ids, n_isects=None, alpha_cutoff=1.0 / 255.0, alpha_clamp=0.99,
                     transmittance_threshold=1e-4, out=None, stream=None, workspace=None, eval_counts=None,
                     masks=None) -> Render:
    """Front-to-back compositing of every tile; returns colours, 1 - T, T and the last composited index.

    eval_counts: optional int64 [5] device tensor that the launch adds to (evaluations by the definition, alpha >=
    cutoff, composited, evaluations executed, splats staged)."""
    lib = load_library()
    dev, C, N, K, th, tw = _raster_inputs(means2d, conics, colors, opacities, backgrounds, isect_offsets,
                                          flatten_ids, masks)
    n = _n_isects(flatten_ids, n_isects)
    _check_eval_counts(eval_counts, dev)
    if out is None:
        out = _render_out(C, height, width, K, dev)
    _check_render_out(out, C, height, width, K, dev)
    ws = workspace if workspace is not None else _workspace(lib.gs_rasterize_workspace_bytes(C, tw, th), dev)
    _check(lib.gs_rasterize_fwd(_ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(backgrounds), C, N,
                                K, width, height, tile_size, tw, th, _ptr(isect_offsets), _ptr(flatten_ids), n,
                                _ptr(masks), float(alpha_cutoff), float(alpha_clamp), float(transmittance_threshold),
                                _ptr(out.render_colors), _ptr(out.render_alphas), _ptr(out.render_T),
                                _ptr(out.last_ids), _ptr(eval_counts), _ptr(ws), ws.numel(), _stream(stream)))
    return out


@_stream_scoped
def gs_rasterize_fwd_hwexp(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, isect_offsets,
                           flatten_ids, n_isects=None, alpha_cutoff=1.0 / 255.0, alpha_clamp=0.99,
                           transmittance_threshold=1e-4, out=None, stream=None, eval_counts=None,
                           masks=None) -> Render:
    """gs_rasterize_fwd with the hardware exponential (faster; not bit-identical to the specified one)."""
    lib = load_library()
    dev, C, N, K, th, tw = _raster_inputs(means2d, conics, colors, opacities, backgrounds, isect_offsets,
                                          flatten_ids, masks)
    n = _n_isects(flatten_ids, n_isects)
    _check_eval_counts(eval_counts, dev)
    if out is None:
        out = _render_out(C, height, width, K, dev)
    _check_render_out(out, C, height, width, K, dev)
    _check(lib.gs_rasterize_fwd_hwexp(_ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(backgrounds),
                                      C, N, K, width, height, tile_size, tw, th, _ptr(isect_offsets),
                                      _ptr(flatten_ids), n, _ptr(masks), float(alpha_cutoff), float(alpha_clamp),
                                      float(transmittance_threshold), _ptr(out.render_colors),
                                      _ptr(out.render_alphas), _ptr(out.render_T), _ptr(out.last_ids),
                                      _ptr(eval_counts), _stream(stream)))
    return out


@dataclass
class TracedRender(Render):
    trace_ids: torch.Tensor | None  # [C, H, W, max_splat_steps] int32 flat splat ids (past the count: unwritten)
    trace_counts: torch.Tensor | None  # [C, H, W] int32


@_stream_scoped
def gs_rasterize_fwd_traced(means2d, conics, colors, opacities, backgrounds, width, height, tile_size,
                            isect_offsets, flatten_ids, max_splat_steps, max_list_entries=-1, n_isects=None,
                            alpha_cutoff=1.0 / 255.0, alpha_clamp=0.99, transmittance_threshold=1e-4, trace=True,
                            out=None, stream=None, workspace=None, eval_counts=None, masks=None) -> TracedRender:
    """The traced forward: each tile's list cut to its first max_list_entries entries (negative: whole lists),
    each pixel stopped after max_splat_steps composited splats, and (trace=True) each pixel's composited flat splat
    ids recorded in order with their count. Entries of a trace row past its count are left unwritten."""
    lib = load_library()
    dev, C, N, K, th, tw = _raster_inputs(means2d, conics, colors, opacities, backgrounds, isect_offsets,
                                          flatten_ids, masks)
    S = int(max_splat_steps)
    if S < 0:
        raise ValueError("max_splat_steps must be >= 0")
    n = _n_isects(flatten_ids, n_isects)
    _check_eval_counts(eval_counts, dev)
    if out is None:
        r = _render_out(C, height, width, K, dev)
        out = TracedRender(r.render_colors, r.render_alphas, r.render_T, r.last_ids,
                           torch.empty((C, height, width, S), dtype=torch.int32, device=dev) if trace else None,
                           torch.empty((C, height, width), dtype=torch.int32, device=dev) if trace else None)
    _check_render_out(out, C, height, width, K, dev)
    if out.trace_ids is not None:
        _req(out.trace_ids, "trace_ids", torch.int32, dev, (C, height, width, S))
    if out.trace_counts is not None:
        _req(out.trace_counts, "trace_counts", torch.int32, dev, (C, height, width))
    ws = workspace if workspace is not None else _workspace(lib.gs_rasterize_workspace_bytes(C, tw, th), dev)
    _check(lib.gs_rasterize_fwd_traced(_ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(backgrounds),
                                       C, N, K, width, height, tile_size, tw, th, _ptr(isect_offsets),
                                       _ptr(flatten_ids), n, _ptr(masks), float(alpha_cutoff), float(alpha_clamp),
                                       float(transmittance_threshold), int(max_list_entries), S,
                                       _ptr(out.render_colors), _ptr(out.render_alphas), _ptr(out.render_T),
                                       _ptr(out.last_ids), _ptr(out.trace_ids), _ptr(out.trace_counts),
                                       _ptr(eval_counts), _ptr(ws), ws.numel(), _stream(stream)))
    return out


@dataclass
class Bins:
    bin_ids: torch.Tensor  # [C, th, tw, capacity] int32, -1 in empty slots
    bin_counts: torch.Tensor  # [C, th, tw] int32 full counts (> capacity: the bin overflowed)


@_stream_scoped
def gs_bin_tiles(means2d, radii, depths, tile_size, tile_width, tile_height, capacity, out=None,
                 stream=None) -> Bins:
    """Fixed-capacity per-tile bins: each tile's splats in (depth, id) order, -1 after them, and full counts."""
    lib = load_library()
    dev = means2d.device
    _req(means2d, "means2d", torch.float32, dev)
    if means2d.dim() != 3 or means2d.shape[2] != 2:
        raise ValueError("means2d must be [C, N, 2]")
    C, N = means2d.shape[0], means2d.shape[1]
    _req(radii, "radii", torch.float32, dev)
    if tuple(radii.shape) == (C, N):
        rpg = 1
    elif tuple(radii.shape) == (C, N, 2):
        rpg = 2
    else:
        raise ValueError(f"radii must be [C, N] or [C, N, 2] (got {tuple(radii.shape)})")
    _req(depths, "depths", torch.float32, dev, (C, N))
    if out is None:
        out = Bins(torch.empty((C, tile_height, tile_width, int(capacity)), dtype=torch.int32, device=dev),
                   torch.empty((C, tile_height, tile_width), dtype=torch.int32, device=dev))
    _req(out.bin_ids, "bin_ids", torch.int32, dev, (C, tile_height, tile_width, int(capacity)))
    _req(out.bin_counts, "bin_counts", torch.int32, dev, (C, tile_height, tile_width))
    _check(lib.gs_bin_tiles(_ptr(means2d), _ptr(radii), rpg, _ptr(depths), C, N, tile_size, tile_width, tile_height,
                            int(capacity), _ptr(out.bin_ids), _ptr(out.bin_counts), _stream(stream)))
    return out


@_stream_scoped
def gs_rasterize_fwd_bins(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, bin_ids,
                          bin_counts, alpha_cutoff=1.0 / 255.0, alpha_clamp=0.99, transmittance_threshold=1e-4,
                          out=None, stream=None, eval_counts=None) -> Render:
    """Front-to-back compositing over fixed-capacity bins; last ids are bin positions t * capacity + m."""
    lib = load_library()
    dev = means2d.device
    _req(bin_ids, "bin_ids", torch.int32, dev)
    if bin_ids.dim() != 4:
        raise ValueError("bin_ids must be [C, th, tw, capacity]")
    _, C, N, K, th, tw = _raster_inputs(means2d, conics, colors, opacities, backgrounds, bin_counts,
                                        bin_ids, None)
    if tuple(bin_ids.shape[:3]) != (C, th, tw):
        raise ValueError("bin_ids and bin_counts disagree on [C, th, tw]")
    _check_eval_counts(eval_counts, dev)
    if out is None:
        out = _render_out(C, height, width, K, dev)
    _check_render_out(out, C, height, width, K, dev)
    _check(lib.gs_rasterize_fwd_bins(_ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(backgrounds),
                                     C, N, K, width, height, tile_size, tw, th, _ptr(bin_ids), _ptr(bin_counts),
                                     bin_ids.shape[3], float(alpha_cutoff), float(alpha_clamp),
                                     float(transmittance_threshold), _ptr(out.render_colors), _ptr(out.render_alphas),
                                     _ptr(out.render_T), _ptr(out.last_ids), _ptr(eval_counts), _stream(stream)))
    return out


@dataclass
class RasterGrad:
    means2d: torch.Tensor  # [C, N, 2]
    conics: torch.Tensor  # [C, N, 3]
    colors: torch.Tensor  # [C, N, K]
    opacities: torch.Tensor  # [C, N]
    backgrounds: torch.Tensor | None  # [C, K]
    means2d_abs: torch.Tensor | None  # [C, N, 2]


@_stream_scoped
def gs_rasterize_bwd(means2d, conics, colors, opacities, backgrounds, width, height, tile_size, isect_offsets,
                     flatten_ids, render_alphas, last_ids, grad_render_colors, grad_render_alphas, n_isects=None,
                     alpha_cutoff=1.0 / 255.0, alpha_clamp=0.99, grad_backgrounds=None, absgrad=False, out=None,
                     stream=None, masks=None) -> RasterGrad:
    """Gradients of sum(grad_render_colors * colours) + sum(grad_render_alphas * alphas) of gs_rasterize_fwd.

    grad_backgrounds: None -> computed when backgrounds is given; False -> not computed."""
    lib = load_library()
    dev = means2d.device
    _req(means2d, "means2d", torch.float32, dev)
    C, N = means2d.shape[0], means2d.shape[1]
    _req(conics, "conics", torch.float32, dev, (C, N, 3))
    _req(colors, "colors", torch.float32, dev)
    if colors.dim() != 3 or tuple(colors.shape[:2]) != (C, N):
        raise ValueError("colors must be [C, N, K]")
    K = colors.shape[2]
    _req(opacities, "opacities", torch.float32, dev, (C, N))
    if backgrounds is not None:
        _req(backgrounds, "backgrounds", torch.float32, dev, (C, K))
    _req(isect_offsets, "isect_offsets", torch.int32, dev)
    th, tw = isect_offsets.shape[1], isect_offsets.shape[2]
    _req(flatten_ids, "flatten_ids", torch.int32, dev)
    _req(render_alphas, "render_alphas", torch.float32, dev, (C, height, width))
    _req(last_ids, "last_ids", torch.int32, dev, (C, height, width))
    _req(grad_render_colors, "grad_render_colors", torch.float32, dev, (C, height, width, K))
    _req(grad_render_alphas, "grad_render_alphas", torch.float32, dev, (C, height, width))
    n = _n_isects(flatten_ids, n_isects)
    if isect_offsets.dim() != 3 or isect_offsets.shape[0] != C:
        raise ValueError("isect_offsets must be [C, th, tw]")
    want_bg = backgrounds is not None if grad_backgrounds is None else bool(grad_backgrounds)
    if out is None:
        e = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)  # noqa: E731
        out = RasterGrad(e(C, N, 2), e(C, N, 3), e(C, N, K), e(C, N), e(C, K) if want_bg else None,
                         e(C, N, 2) if absgrad else None)
    _req(out.means2d, "grad_means2d", torch.float32, dev, (C, N, 2))
    _req(out.conics, "grad_conics", torch.float32, dev, (C, N, 3))
    _req(out.colors, "grad_colors", torch.float32, dev, (C, N, K))
    _req(out.opacities, "grad_opacities", torch.float32, dev, (C, N))
    if out.backgrounds is not None:
        _req(out.backgrounds, "grad_backgrounds", torch.float32, dev, (C, K))
    if out.means2d_abs is not None:
        _req(out.means2d_abs, "grad_means2d_abs", torch.float32, dev, (C, N, 2))
    if masks is not None:
        _req(masks, "masks", torch.int32, dev, (C, th, tw))
    _check(lib.gs_rasterize_bwd(_ptr(means2d), _ptr(conics), _ptr(colors), _ptr(opacities), _ptr(backgrounds), C, N,
                                K, width, height, tile_size, tw, th, _ptr(isect_offsets), _ptr(flatten_ids), n,
                                _ptr(masks), float(alpha_cutoff), float(alpha_clamp), _ptr(render_alphas),
                                _ptr(last_ids), _ptr(grad_render_colors), _ptr(grad_render_alphas), _ptr(out.means2d),
                                _ptr(out.conics), _ptr(out.colors), _ptr(out.opacities), _ptr(out.backgrounds),
                                _ptr(out.means2d_abs), _stream(stream)))
    return out


@dataclass
class Projection:
    radii: torch.Tensor  # [C, N, 2] int32
    means2d: torch.Tensor  # [C, N, 2]
    depths: torch.Tensor  # [C, N]
    conics: torch.Tensor  # [C, N, 3]
    compensations: torch.Tensor | None  # [C, N]


@_stream_scoped
def gs_project_fwd(means, covars, viewmats, Ks, width, height, eps2d=0.3, near_plane=0.01, far_plane=1e10,
                   radius_clip=0.0, compensation=False, orthographic=False, out=None, stream=None) -> Projection:
    """EWA projection of [N, 3] means and [N, 3, 3] covariances into C cameras."""
    lib = load_library()
    dev = means.device
    _req(means, "means", torch.float32, dev)
    if means.dim() != 2 or means.shape[1] != 3:
        raise ValueError("means must be [N, 3]")
    N = means.shape[0]
    _req(covars, "covars", torch.float32, dev, (N, 3, 3))
    _req(viewmats, "viewmats", torch.float32, dev)
    if viewmats.dim() != 3 or tuple(viewmats.shape[1:]) != (4, 4):
        raise ValueError("viewmats must be [C, 4, 4]")
    C = viewmats.shape[0]
    _req(Ks, "Ks", torch.float32, dev, (C, 3, 3))
    if out is None:
        out = Projection(torch.empty((C, N, 2), dtype=torch.int32, device=dev),
                         torch.empty((C, N, 2), dtype=torch.float32, device=dev),
                         torch.empty((C, N), dtype=torch.float32, device=dev),
                         torch.empty((C, N, 3), dtype=torch.float32, device=dev),
                         torch.empty((C, N), dtype=torch.float32, device=dev) if compensation else None)
    _check(lib.gs_project_fwd(_ptr(means), _ptr(covars), _ptr(viewmats), _ptr(Ks), C, N, int(width), int(height),
                              float(eps2d), float(near_plane), float(far_plane), float(radius_clip),
                              int(bool(orthographic)), _ptr(out.radii), _ptr(out.means2d), _ptr(out.depths),
                              _ptr(out.conics), _ptr(out.compensations), _stream(stream)))
    return out

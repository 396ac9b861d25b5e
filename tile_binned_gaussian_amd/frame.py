"""One frame through the four entry points of libgs_raster, with device buffers from PyTorch.

Marshalling only: intersections (count, emit and sort), tile ranges, then compositing, all on one stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding


@dataclass
class DeviceScene:
    """A synth.Scene moved to the GPU (contiguous float32 tensors)."""

    C: int
    N: int
    width: int
    height: int
    tile_size: int
    tile_width: int
    tile_height: int
    means2d: torch.Tensor
    radii: torch.Tensor
    depths: torch.Tensor
    conics: torch.Tensor
    colors: torch.Tensor
    opacities: torch.Tensor
    backgrounds: torch.Tensor | None
    alpha_cutoff: float
    alpha_clamp: float
    transmittance_threshold: float


def to_device(scene, device="cuda") -> DeviceScene:
    t = lambda a: torch.from_numpy(a).to(device).contiguous()  # noqa: E731
    return DeviceScene(scene.C, scene.N, scene.width, scene.height, scene.tile_size, scene.tile_width,
                       scene.tile_height, t(scene.means2d), t(scene.radii), t(scene.depths), t(scene.conics),
                       t(scene.colors), t(scene.opacities),
                       None if scene.backgrounds is None else t(scene.backgrounds), scene.alpha_cutoff,
                       scene.alpha_clamp, scene.transmittance_threshold)


@dataclass
class FrameResult:
    isect: binding.Intersections
    isect_offsets: torch.Tensor
    render: binding.Render


def render_frame(ds: DeviceScene, stream=None) -> FrameResult:
    it = binding.gs_isect_tiles(ds.means2d, ds.radii, ds.depths, ds.tile_size, ds.tile_width, ds.tile_height,
                                sort=True, stream=stream)
    off = binding.gs_tile_ranges(it.isect_ids, ds.C, ds.tile_width, ds.tile_height, stream=stream)
    ren = binding.gs_rasterize_fwd(ds.means2d, ds.conics, ds.colors, ds.opacities, ds.backgrounds, ds.width,
                                   ds.height, ds.tile_size, off, it.flatten_ids, it.n_isects, ds.alpha_cutoff,
                                   ds.alpha_clamp, ds.transmittance_threshold, stream=stream)
    return FrameResult(it, off, ren)

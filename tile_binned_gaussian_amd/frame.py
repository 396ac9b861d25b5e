"""One frame through the four entry points of libgs_raster, with device buffers from PyTorch.

Marshalling only: intersections (count, emit and sort), tile ranges, then compositing, all on one stream.
"""
from __future__ import annotations

import ctypes
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


class FramePlan:
    """Preallocated buffers for repeated frames of one scene, so that a timed loop allocates nothing.

    run() issues: count (one synchronisation for the intersection count), emit with the sort folded in
    (gs_isect_tiles with sort=1), tile ranges and the composite, with optional torch events recorded between the
    steps on the same stream. run_generic_sort() times gs_sort_keys alone on the frame's unsorted keys."""

    def __init__(self, ds: DeviceScene, stream=None):
        self.ds = ds
        self.lib = binding.load_library()
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        # every buffer belongs to the plan's stream (torch's caching allocator then reuses a freed one only in
        # that stream's order), and the workspace growth below copies on that stream too
        with torch.cuda.stream(self.stream):
            self._allocate(ds)
        self.capacity = -1
        self.n_isects = 0

    def _allocate(self, ds):
        dev = ds.means2d.device
        C, N = ds.C, ds.N
        self.rpg = 2 if ds.radii.dim() == 3 else 1
        self.tile_bits = _bits_for(ds.tile_width * ds.tile_height)
        self.end_bit = 32 + self.tile_bits + _bits_for(C)
        self.tiles_per = torch.empty((C, N), dtype=torch.int32, device=dev)
        self.goff = torch.empty(C * N, dtype=torch.int32, device=dev)
        self.offsets = torch.empty((C, ds.tile_height, ds.tile_width), dtype=torch.int32, device=dev)
        K = ds.colors.shape[2]
        self.render = binding.Render(torch.empty((C, ds.height, ds.width, K), dtype=torch.float32, device=dev),
                                     torch.empty((C, ds.height, ds.width), dtype=torch.float32, device=dev),
                                     torch.empty((C, ds.height, ds.width), dtype=torch.float32, device=dev),
                                     torch.empty((C, ds.height, ds.width), dtype=torch.int32, device=dev))
        # one intersection workspace for both phases: phase 1 leaves the depth order at its start for phase 2
        self.ws_isect = torch.empty(max(self.lib.gs_isect_workspace_bytes(C, N, 0, ds.tile_width, ds.tile_height, 1),
                                        1), dtype=torch.uint8, device=dev)
        self.ws_ranges = torch.empty(self.lib.gs_tile_ranges_workspace_bytes(), dtype=torch.uint8, device=dev)
        self.ws_raster = torch.empty(max(self.lib.gs_rasterize_workspace_bytes(C, ds.tile_width, ds.tile_height), 1),
                                     dtype=torch.uint8, device=dev)
        # page-locked host word for the intersection count (the device writes it without blocking the host)
        self.n_host = torch.zeros(1, dtype=torch.int64, pin_memory=True)

    def _ensure(self, n):
        if n <= self.capacity:
            return
        with torch.cuda.stream(self.stream):
            self._grow(n)

    def _grow(self, n):
        dev = self.ds.means2d.device
        self.keys = torch.empty(max(n, 1), dtype=torch.int64, device=dev)
        self.ids = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        need = self.lib.gs_isect_workspace_bytes(self.ds.C, self.ds.N, n, self.ds.tile_width, self.ds.tile_height, 1)
        if need > self.ws_isect.numel():
            grown = torch.empty(need, dtype=torch.uint8, device=dev)
            grown[:self.ws_isect.numel()].copy_(self.ws_isect)
            self.ws_isect = grown
        self.capacity = n

    def _count(self, s):
        ds, lib, P = self.ds, self.lib, binding._ptr
        binding._check(lib.gs_isect_tiles(P(ds.means2d), P(ds.radii), self.rpg, P(ds.depths), ds.C, ds.N,
                                          ds.tile_size, ds.tile_width, ds.tile_height, 1, P(self.tiles_per),
                                          P(self.goff), P(self.n_host), None, None, 0, P(self.ws_isect),
                                          self.ws_isect.numel(), s))
        return int(self.n_host[0])

    def _emit(self, s, n, sort):
        ds, lib, P = self.ds, self.lib, binding._ptr
        if n > 0:
            binding._check(lib.gs_isect_tiles(P(ds.means2d), P(ds.radii), self.rpg, P(ds.depths), ds.C, ds.N,
                                              ds.tile_size, ds.tile_width, ds.tile_height, int(sort), None,
                                              P(self.goff), None, P(self.keys), P(self.ids), n, P(self.ws_isect),
                                              self.ws_isect.numel(), s))

    def run(self, events=None, eval_counts=None):
        """One frame. events: optional list of 5 torch.cuda.Event recorded before count, emit+sort, ranges and
        the composite, and after the composite."""
        ds, lib, P = self.ds, self.lib, binding._ptr
        s = binding._stream(self.stream)
        ev = events or [None] * 5
        rec = lambda i: ev[i] is not None and ev[i].record(self.stream)  # noqa: E731
        rec(0)
        n = self._count(s)
        self._ensure(n)
        self.n_isects = n
        rec(1)
        self._emit(s, n, sort=True)
        rec(2)
        binding._check(lib.gs_tile_ranges(P(self.keys), n, ds.C, ds.tile_width, ds.tile_height, P(self.offsets), 0,
                                          P(self.ws_ranges), self.ws_ranges.numel(), s))
        rec(3)
        r = self.render
        binding._check(lib.gs_rasterize_fwd(P(ds.means2d), P(ds.conics), P(ds.colors), P(ds.opacities),
                                            P(ds.backgrounds), ds.C, ds.N, ds.colors.shape[2], ds.width, ds.height,
                                            ds.tile_size, ds.tile_width, ds.tile_height, P(self.offsets),
                                            P(self.ids), n, None, ctypes.c_float(ds.alpha_cutoff),
                                            ctypes.c_float(ds.alpha_clamp),
                                            ctypes.c_float(ds.transmittance_threshold), P(r.render_colors),
                                            P(r.render_alphas), P(r.render_T), P(r.last_ids), P(eval_counts),
                                            P(self.ws_raster), self.ws_raster.numel(), s))
        rec(4)
        return n

    def run_generic_sort(self, repeats, warmup=2):
        """Median milliseconds of gs_sort_keys over bits [0, end_bit) on this frame's unsorted keys (each repeat
        re-emits the unsorted order first, outside the timed interval)."""
        s = binding._stream(self.stream)
        n = self._count(s)
        self._ensure(n)
        with torch.cuda.stream(self.stream):
            ws = torch.empty(max(self.lib.gs_sort_workspace_bytes(n, self.end_bit), 1), dtype=torch.uint8,
                             device=self.ds.means2d.device)
        times = []
        for r in range(warmup + repeats):
            self._emit(s, n, sort=False)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            binding._check(self.lib.gs_sort_keys(binding._ptr(self.keys), binding._ptr(self.ids), n, self.end_bit,
                                                 binding._ptr(ws), ws.numel(), s))
            b.record(self.stream)
            b.synchronize()
            if r >= warmup:
                times.append(a.elapsed_time(b))
        times.sort()
        return times[len(times) // 2], n


class BackwardPlan:
    """The composite's backward on a FramePlan's last frame, with preallocated gradients and fixed seeded output
    gradients (standard normal), for timing."""

    def __init__(self, plan: FramePlan, seed=0, absgrad=False):
        self.plan = plan
        ds = plan.ds
        with torch.cuda.stream(plan.stream):  # buffers belong to the stream the backward runs on
            g = torch.Generator(device=ds.means2d.device).manual_seed(seed)
            C, H, W, K = ds.C, ds.height, ds.width, ds.colors.shape[2]
            self.gc = torch.randn((C, H, W, K), generator=g, device=ds.means2d.device)
            self.ga = torch.randn((C, H, W), generator=g, device=ds.means2d.device)
            e = lambda *shape: torch.empty(shape, dtype=torch.float32, device=ds.means2d.device)  # noqa: E731
            self.out = binding.RasterGrad(e(C, ds.N, 2), e(C, ds.N, 3), e(C, ds.N, K), e(C, ds.N),
                                          None if ds.backgrounds is None else e(C, K),
                                          e(C, ds.N, 2) if absgrad else None)

    def run(self):
        plan, ds = self.plan, self.plan.ds
        return binding.gs_rasterize_bwd(ds.means2d, ds.conics, ds.colors, ds.opacities, ds.backgrounds, ds.width,
                                        ds.height, ds.tile_size, plan.offsets, plan.ids, plan.render.render_alphas,
                                        plan.render.last_ids, self.gc, self.ga, n_isects=plan.n_isects,
                                        alpha_cutoff=ds.alpha_cutoff, alpha_clamp=ds.alpha_clamp, out=self.out,
                                        stream=plan.stream)


def _bits_for(count: int) -> int:
    bits = 0
    while (1 << bits) < count:
        bits += 1
    return bits

"""MI355X-native (gfx950, HIP) tile-binned splat rasterizer.

The compute lives in ``libgs_raster.so`` (C ABI declared in ``include/gs_raster.h``): intersections and keys,
a stable onesweep radix sort, boundary-detect tile ranges and per-tile compositing. ``binding`` wraps each entry
point with the same name; ``frame`` chains them for one frame; ``synth`` draws seeded inputs.

Importing this package loads nothing; the binding loads the library on first use and fails loudly when it is
missing (there is no CPU fallback).
"""

__all__ = ["binding", "frame", "synth", "build"]

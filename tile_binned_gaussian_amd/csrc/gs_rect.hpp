// Tile rectangles of splats ([gsplat] gsplat 1.0.0 intersections.c: gs_clamp_tile, gs_bounds), shared by the
// intersection and the fixed-capacity binning kernels.
#pragma once

#include "gs_internal.hpp"

namespace gs {

// Tile index from a floor/ceil result, clamped to [0, maximum] (gs_clamp_tile). The clamp is applied to the
// float so NaN and values beyond int range are defined (NaN -> 0).
__device__ __forceinline__ int clamp_tile(float v, int maximum) {
    if (!(v > 0.0f)) return 0;
    if (v > static_cast<float>(maximum)) return maximum;
    return static_cast<int>(v);
}

struct Rect {
    int x0, y0, x1, y1;
};

// gs_bounds: empty for a non-positive radius; IEEE float32 division by the tile size.
__device__ __forceinline__ Rect tile_rect(float mx, float my, float rx, float ry, float ts, int tw, int th) {
    Rect r{0, 0, 0, 0};
    if (rx <= 0.0f || ry <= 0.0f) return r;
    r.x0 = clamp_tile(floorf((mx - rx) / ts), tw);
    r.y0 = clamp_tile(floorf((my - ry) / ts), th);
    r.x1 = clamp_tile(ceilf((mx + rx) / ts), tw);
    r.y1 = clamp_tile(ceilf((my + ry) / ts), th);
    return r;
}

template <int RPG>
__device__ __forceinline__ Rect rect_of(const float2 *__restrict__ means, const float *__restrict__ radii, int i,
                                        float ts, int tw, int th) {
    const float2 m = means[i];
    float rx, ry;
    if (RPG == 2) {
        const float2 r = reinterpret_cast<const float2 *>(radii)[i];
        rx = r.x;
        ry = r.y;
    } else {
        rx = radii[i];
        ry = rx;
    }
    return tile_rect(m.x, m.y, rx, ry, ts, tw, th);
}

}  // namespace gs

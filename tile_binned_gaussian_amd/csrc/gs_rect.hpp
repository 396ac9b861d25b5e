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

// A rectangle (x0, y0, width, height) in one 32-bit word, for tile grids whose four fields fit:
// x0 | width << cx | y0 << 2 cx | height << (2 cx + cy), with cx bits for values up to tile_width and cy bits for
// values up to tile_height (2 (cx + cy) <= 32). Used where rectangles are stored and gathered, so each costs 4
// bytes instead of 16.
struct RectPacking {
    int cx, cy;  // field widths; cx = 0 when the grid's rectangles do not fit one word
};
inline RectPacking rect_packing(int tile_width, int tile_height) {
    const int cx = bits_for(static_cast<int64_t>(tile_width) + 1), cy = bits_for(static_cast<int64_t>(tile_height) + 1);
    return 2 * (cx + cy) <= 32 ? RectPacking{cx, cy} : RectPacking{0, 0};
}
__device__ __forceinline__ uint32_t pack_rect(int x0, int y0, int w, int h, RectPacking p) {
    return static_cast<uint32_t>(x0) | static_cast<uint32_t>(w) << p.cx | static_cast<uint32_t>(y0) << (2 * p.cx) |
           static_cast<uint32_t>(h) << (2 * p.cx + p.cy);
}
__device__ __forceinline__ int4 unpack_rect(uint32_t v, RectPacking p) {
    const uint32_t mx = (1u << p.cx) - 1u, my = (1u << p.cy) - 1u;
    return make_int4(static_cast<int>(v & mx), static_cast<int>((v >> (2 * p.cx)) & my),
                     static_cast<int>((v >> p.cx) & mx), static_cast<int>((v >> (2 * p.cx + p.cy)) & my));
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

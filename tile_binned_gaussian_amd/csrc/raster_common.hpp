// Device helpers shared by the composite and its backward: the float32 exponential both sides of the oracle
// comparison implement, and the conservative per-region cull of a splat's alpha >= cutoff footprint.
#pragma once

#include "gs_internal.hpp"

#include <cmath>

namespace gs {
namespace {

// e^-sigma in float32: Cody and Waite's range reduction (k = rint(-sigma / ln 2), r = -sigma - k ln 2 with ln 2
// split into a 15-bit high part and a low correction, both by fma) and the degree-7 Taylor polynomial of e^r
// evaluated by fma, scaled by 2^k. sigma > 80 (or NaN) gives 0, which also keeps 2^k a normal scale.
__device__ __forceinline__ float exp_neg(float sigma) {
    if (!(sigma <= 80.0f)) return 0.0f;
    const float t = -sigma;
    const float k = __builtin_rintf(t * 0x1.715476p+0f);  // 1 / ln 2
    float r = __builtin_fmaf(-k, 0x1.62e4p-1f, t);         // ln 2, high 15 bits
    r = __builtin_fmaf(-k, 0x1.7f7d1cp-20f, r);             // ln 2 - high part
    float q = 0x1.a01a02p-13f;                              // 1/7!
    q = __builtin_fmaf(q, r, 0x1.6c16c2p-10f);              // 1/6!
    q = __builtin_fmaf(q, r, 0x1.111112p-7f);               // 1/5!
    q = __builtin_fmaf(q, r, 0x1.555556p-5f);               // 1/4!
    q = __builtin_fmaf(q, r, 0x1.555556p-3f);               // 1/3!
    q = __builtin_fmaf(q, r, 0.5f);
    q = __builtin_fmaf(q, r, 1.0f);
    q = __builtin_fmaf(q, r, 1.0f);
    return __builtin_ldexpf(q, static_cast<int>(k));
}

// Cody and Waite's reduction r = t - k ln 2 (ln 2 split as in exp_neg) and the degree-7 Taylor polynomial q = e^r,
// for t = -sigma and k = rint(t / ln 2) given.
__device__ __forceinline__ float exp_reduced_poly(float t, float k) {
    float r = __builtin_fmaf(-k, 0x1.62e4p-1f, t);
    r = __builtin_fmaf(-k, 0x1.7f7d1cp-20f, r);
    float q = 0x1.a01a02p-13f;
    q = __builtin_fmaf(q, r, 0x1.6c16c2p-10f);
    q = __builtin_fmaf(q, r, 0x1.111112p-7f);
    q = __builtin_fmaf(q, r, 0x1.555556p-5f);
    q = __builtin_fmaf(q, r, 0x1.555556p-3f);
    q = __builtin_fmaf(q, r, 0.5f);
    q = __builtin_fmaf(q, r, 1.0f);
    q = __builtin_fmaf(q, r, 1.0f);
    return q;
}

// The reduction and polynomial of exp_neg without its range test: q = e^r with -sigma = k ln 2 + r.
__device__ __forceinline__ float exp_neg_parts(float sigma, float &k) {
    const float t = -sigma;
    k = __builtin_rintf(t * 0x1.715476p+0f);  // 1 / ln 2
    return exp_reduced_poly(t, k);
}

// The same function without branches (a select replaces the early return), for lock-step loops where every lane
// evaluates it anyway. Identical bits: the polynomial path is the one above, and any sigma that is not <= 80
// (including NaN) selects 0.
__device__ __forceinline__ float exp_neg_select(float sigma) {
    float k;
    const float q = exp_neg_parts(sigma, k);
    const int ki = (sigma <= 80.0f) ? static_cast<int>(k) : 0;
    const float e = __builtin_ldexpf(q, ki);
    return (sigma <= 80.0f) ? e : 0.0f;
}

// exp_neg for 0 <= sigma <= 80 (the polynomial path), with k = rint(-sigma / ln 2) formed by adding and subtracting
// 1.5 * 2^23 (which rounds the already rounded product to the nearest integer, ties to even, as rintf does, since
// |k| <= 116) and 2^k applied by adding k to the exponent field of q (in [0.7, 1.42]): the result's exponent stays
// at 2^-117 or above, so the sum is the exact scaling, and the bits are exp_neg's. Both steps are plain adds, which
// issue in pairs where the rounding, conversion and ldexp instructions do not.
__device__ __forceinline__ float exp_neg_short(float sigma) {
    const float t = -sigma;
    const float shifted = t * 0x1.715476p+0f + 0x1.8p+23f;  // 1 / ln 2; k in the low bits
    const float q = exp_reduced_poly(t, shifted - 0x1.8p+23f);
    // (bits(shifted) << 23) is k << 23 modulo 2^32: the constant's own bits lie at positions 22 and up
    return __int_as_float(__float_as_int(q) + static_cast<int>(static_cast<uint32_t>(__float_as_int(shifted)) << 23));
}

// e^-sigma by the hardware base-2 exponential (v_exp_f32, about 1 ulp) of -sigma log2(e): a product and one
// transcendental instruction instead of the 14 operations above, not bit-identical to them; sigma > 80 or NaN
// gives 0 as above. The cull below stays exact with it: the product's rounding moves the exponent by at most
// 80 * 2^-24, a relative change of the result far inside the cull's 5% margin, and 2^t <= 1 for t <= 0.
__device__ __forceinline__ float exp_neg_hw(float sigma) {
    const float e = __builtin_amdgcn_exp2f(-sigma * 0x1.715476p+0f);
    return (sigma <= 80.0f) ? e : 0.0f;
}

// Conservative cull of one splat against a wave's pixel region (pixel-centre box [x0, x1] x [y0, y1]). The splat
// is dropped for the region only when alpha < cutoff at every pixel of the box, so skipping it there leaves every
// output bit unchanged:
//  - opacity < cutoff: alpha = opacity * E(sigma) <= opacity since E(sigma) <= 1 for sigma >= 0;
//  - otherwise alpha >= cutoff needs sigma_exact <= L = ln(opacity / cutoff) + 0.05. The set {sigma <= L} lies
//    inside |dx| <= sqrt(2 L S_xx), |dy| <= sqrt(2 L S_yy) with S = inverse of the conic (the marginal bound of a
//    quadratic form): a box test first; then the minimum of sigma over the region's continuous box (no smaller
//    than over its pixel centres) must not exceed thr = 1.004 L + 1e-3. The 5% alpha margin in L and the 0.4% in
//    thr cover float32 rounding: with trace^2 <= 1000 det a computed sigma is within 24 * 2^-24 * trace^2 / det
//    < 0.15% of the exact one, E is within one ulp of e^-sigma, the minimiser along an edge is found to within
//    rounding (the quadratic is flat there, so the value moves by a second-order amount the 1e-3 covers), and
//    0.9985 (ln(o / cutoff) + 0.05) > ln(o / cutoff) for every opacity up to 1e6; the box is padded for the
//    rounding of its own arithmetic;
//  - non-positive-definite, badly conditioned or non-finite conics, opacities above 1e6 or NaN, and means beyond
//    1e6 pixels are never culled.
struct CullBox {
    float x0, x1, y0, y1;  // bounding box of the alpha >= cutoff footprint, or +-inf when not culled
    float thr, ra, rc;     // sigma bound for the region test and 1/a, 1/c (finite only when culled)
    bool never;            // the splat can reach the cutoff nowhere
    bool exact;            // the region test applies
};

__device__ __forceinline__ CullBox cull_box(float2 m, float a, float b, float c, float o, float alpha_cutoff,
                                           float log_cutoff) {
    CullBox box{-INFINITY, INFINITY, -INFINITY, INFINITY, 0.0f, 0.0f, 0.0f, false, false};
    if (o < alpha_cutoff) {
        box.never = true;
        return box;
    }
    const float det = a * c - b * b;
    const float tr = a + c;
    if (!(o >= alpha_cutoff) || !(o <= 1.0e6f) || !(det > 0.0f) || !(a > 0.0f) || !(c > 0.0f) ||
        !(tr * tr <= 1.0e3f * det) || !(fabsf(m.x) < 1.0e6f) || !(fabsf(m.y) < 1.0e6f))
        return box;
    // The hardware logarithm, reciprocal and square root (within a few ulp) stand in for the correctly rounded
    // functions: their errors, below 1e-6 absolute in L and a few 2^-24 relative in rx, ry and 1/a, 1/c, are far
    // inside the margins (0.05 in L, 1e-4 relative in rx, ry); a reciprocal or logarithm flushed to 0 or infinity
    // leaves rx or ry infinite or NaN, and the splat is then never culled.
    const float L = __logf(o) - log_cutoff + 0.05f;
    const float rdet = __builtin_amdgcn_rcpf(det);
    float rx = __builtin_amdgcn_sqrtf(2.0f * L * (c * rdet)) * 1.0001f;
    float ry = __builtin_amdgcn_sqrtf(2.0f * L * (a * rdet)) * 1.0001f;
    if (!(rx < 1.0e6f) || !(ry < 1.0e6f)) return box;
    rx += 2.0e-3f + 1.0e-6f * (fabsf(m.x) + rx);
    ry += 2.0e-3f + 1.0e-6f * (fabsf(m.y) + ry);
    box.x0 = m.x - rx;
    box.x1 = m.x + rx;
    box.y0 = m.y - ry;
    box.y1 = m.y + ry;
    box.thr = 1.004f * L + 1.0e-3f;
    box.ra = __builtin_amdgcn_rcpf(a);
    box.rc = __builtin_amdgcn_rcpf(c);
    box.exact = true;
    return box;
}

// sigma = 0.5 (a dx^2 + c dy^2) + b dx dy at an offset from the mean
__device__ __forceinline__ float quad_form(float a, float b, float c, float dx, float dy) {
    return 0.5f * (a * dx * dx + c * dy * dy) + b * dx * dy;
}

// Whether sigma can be <= thr somewhere in the box [x0, x1] x [y0, y1]: yes if the mean is inside; otherwise the
// minimum of the convex quadratic lies on the boundary, on an edge that faces the mean (at a minimiser inside the
// top edge the gradient is (0, -t), t >= 0, which for a positive-definite form means the mean lies on or above the
// top edge's line, and likewise for the other edges), so only the edge nearest the mean in x and the one nearest
// in y are searched, each a one-dimensional quadratic minimised at the clamped stationary point. A nearest edge
// with the mean within its range is merely one more point of the box, which leaves the minimum found unchanged.
__device__ __forceinline__ bool region_reach(float2 m, float a, float b, float c, float ra, float rc, float thr,
                                             float x0, float x1, float y0, float y1) {
    if (m.x >= x0 && m.x <= x1 && m.y >= y0 && m.y <= y1) return true;
    const float lx = x0 - m.x, hx = x1 - m.x, ly = y0 - m.y, hy = y1 - m.y;
    const float ex = m.x < x0 ? lx : hx, ey = m.y < y0 ? ly : hy;
    const float best = fminf(quad_form(a, b, c, ex, fminf(fmaxf(-b * ex * rc, ly), hy)),
                             quad_form(a, b, c, fminf(fmaxf(-b * ey * ra, lx), hx), ey));
    return best <= thr;
}

// region_reach for the four 8 x 8 quadrants of a 16 x 16 tile at once: quadrant w covers the pixel-centre box
// [ox + 8 (w & 1) + 0.5, ox + 8 (w & 1) + 7.5] x [oy + 8 (w >> 1) + 0.5, oy + 8 (w >> 1) + 7.5] (ox, oy: the tile's
// first pixel). Bit w is set when the splat's box overlaps quadrant w and the region test passes for it, with the
// values region_reach computes (so the same decisions): the quadrants share two x ranges and two y ranges, so each
// range's edge offsets, nearest edge, stationary-point product and a ex^2 (c ey^2) term are computed once.
__device__ __forceinline__ uint32_t quadrant_reach(float2 m, float a, float b, float c, const CullBox &box, float ox,
                                                   float oy) {
    float lx[2], hx[2], ex[2], sx[2], ax[2], ly[2], hy[2], ey[2], sy[2], cy[2];
    bool xo[2], xin[2], yo[2], yin[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float x0 = ox + (i ? 8.5f : 0.5f), x1 = ox + (i ? 15.5f : 7.5f);
        xo[i] = box.x1 >= x0 && box.x0 <= x1;
        xin[i] = m.x >= x0 && m.x <= x1;
        lx[i] = x0 - m.x;
        hx[i] = x1 - m.x;
        ex[i] = m.x < x0 ? lx[i] : hx[i];
        sx[i] = -b * ex[i] * box.rc;
        ax[i] = a * ex[i] * ex[i];
        const float y0 = oy + (i ? 8.5f : 0.5f), y1 = oy + (i ? 15.5f : 7.5f);
        yo[i] = box.y1 >= y0 && box.y0 <= y1;
        yin[i] = m.y >= y0 && m.y <= y1;
        ly[i] = y0 - m.y;
        hy[i] = y1 - m.y;
        ey[i] = m.y < y0 ? ly[i] : hy[i];
        sy[i] = -b * ey[i] * box.ra;
        cy[i] = c * ey[i] * ey[i];
    }
    uint32_t bits = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int i = w & 1, j = w >> 1;
        // the nearest x edge at its clamped stationary y, and the nearest y edge at its clamped stationary x, as
        // quad_form evaluates them
        const float dyx = fminf(fmaxf(sx[i], ly[j]), hy[j]);
        const float dxy = fminf(fmaxf(sy[j], lx[i]), hx[i]);
        const float qx = 0.5f * (ax[i] + c * dyx * dyx) + b * ex[i] * dyx;
        const float qy = 0.5f * (a * dxy * dxy + cy[j]) + b * dxy * ey[j];
        const bool reach = (xin[i] && yin[j]) || fminf(qx, qy) <= box.thr;
        bits |= (xo[i] && yo[j] && reach ? 1u : 0u) << w;
    }
    return bits;
}

}  // namespace
}  // namespace gs

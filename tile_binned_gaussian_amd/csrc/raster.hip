// Per-tile front-to-back alpha compositing on gfx950. One workgroup per tile, one pixel per thread (tiles up to
// 16x16; 4 pixels per thread up to 32x32). The tile's splats are staged in batches through LDS (mean, conic,
// opacity, colour), every lane reads the same LDS word (a broadcast), and a pixel stops at the transmittance
// early-out; a workgroup vote ends the tile once every pixel has stopped. No matrix cores: nothing here is a
// dense contraction.
//
// Definitions: the front-to-back inverse of gsplat 1.0.0 raster_backward.c (gs_raster_backward_pixel: pixel
// centre, delta, quadratic form, alpha clamp, skip test, render alpha = 1 - T; gs_raster_backward_without_gvl:
// tile walk and range end), with alpha_cutoff and transmittance_threshold from rlx-metal 0.2.9
// splat_training.rs (training_forward_metal_traced).
#include "raster_common.hpp"

#include <cmath>

namespace gs {
namespace {

constexpr int kMaxThreads = 256;
// records evaluated per iteration of the composite's loop outside the traced build (independent exponential
// chains; with 3 colour channels, 3 measured 6% faster than 1 and 2% faster than 2 on the 1M-splat 1080p frame, and
// 4 spills past the 64 registers of 8 waves per SIMD; 4 channels take 2, which fits)
template <int K>
constexpr int kUnroll = K > 3 ? 2 : 3;
// cull word bit of a staged splat that may not take the composite's short step (bits 0-3: the waves it reaches)
constexpr uint32_t kNotShort = 0x80000000u;
// Index-word bit of a staged record that holds the conic's a and c themselves. The other records hold a / 2 and
// c / 2, which is exact, and so is every product of the quadratic form then: a, c >= 2^-60 (and, within the cull's
// exact case, a, c < 6e20 with |dx|, |dy| < 2.1e6 for any pixel of a region the splat is listed for), so with
// |dx| >= 2^-26 whenever it is not 0 each product stays normal and finite, and halving commutes with rounding. The
// sum a/2 dx^2 + c/2 dy^2 is then bit for bit 0.5 (a dx^2 + c dy^2), the specified form, one multiplication
// shorter.
constexpr int32_t kWholeConic = INT32_MIN;

// The quadratic form of a staged record at (dx, dy), in the specified operation order; `whole`: the record holds a
// and c themselves, else their halves.
__device__ __forceinline__ float record_sigma(float a, float b, float c, bool whole, float dx, float dy) {
    const float s = a * dx * dx + c * dy * dy;
    return (whole ? 0.5f * s : s) + b * dx * dy;
}

struct RasterArgs {
    const float2 *means;
    const float *conics;
    const float *colors;
    const float *opacities;
    const float *backgrounds;
    const int32_t *offsets;
    const int32_t *ids;
    const int32_t *masks;  // nullable [C, th, tw]: 0 = composite nothing in this tile
    int64_t n_isects;
    int n_splats;  // C * N: ids outside [0, n_splats) (the -1 of an empty bin slot) are skipped, never gathered
    int total_tiles, width, height, tile_size, tile_width, tile_height;
    float alpha_cutoff, alpha_clamp, transmittance_threshold;
    float *out_colors, *out_alphas, *out_T;
    int32_t *out_last;
    unsigned long long *eval_counts;  // nullable: the five work counts of the ABI
    float log_cutoff;                 // ln(alpha_cutoff), for the conservative cull
    int max_list;                     // >= 0: composite only the first max_list entries of each tile's range
    int max_steps;                    // traced kernels: a pixel stops after this many composited splats
    int32_t *trace_ids;               // traced kernels, nullable: [C, H, W, max_steps] flat splat ids
    int32_t *trace_counts;            // traced kernels, nullable: [C, H, W] composited splats per pixel
    int trace_vec;                    // trace_ids is 16-byte aligned and max_steps a multiple of 4
    const int32_t *bin_counts;        // nullable: ranges from fixed-capacity bins instead of offsets
    int capacity;                     // bin capacity (bin t occupies ids[t * capacity, (t + 1) * capacity))
    int short_step;                   // alpha_cutoff >= 1e-20: batches of well-conditioned splats take the short step
};

// Traced kernels stage each pixel's trace in LDS, kTraceChunk ids per thread, and store a full chunk as four
// contiguous 16-byte non-temporal pieces (one whole 64-byte segment that bypasses the caches the composite's
// gathers use), so rows reach memory in whole segments rather than as scattered 4-byte writes. The per-thread
// slots are kTraceChunk + 1 words apart (no LDS bank conflicts when the threads of a wave write different slots).
// The staging area (17 KB) lowers the traced build's occupancy from 8 to 4 workgroups per CU; the untraced
// build does not allocate it.
constexpr int kTraceChunk = 16;
constexpr int kTraceStride = kTraceChunk + 1;
typedef int v4i __attribute__((ext_vector_type(4)));

// Store the n staged ids `buf` as trace entries [j, j + n) of the row `row`.
__device__ __forceinline__ void flush_trace(int32_t *row, int j, const int32_t *buf, int n, bool vec) {
    if (vec && n == kTraceChunk) {
#pragma unroll
        for (int k = 0; k < kTraceChunk; k += 4)
            __builtin_nontemporal_store(v4i{buf[k], buf[k + 1], buf[k + 2], buf[k + 3]},
                                        reinterpret_cast<v4i *>(row + j + k));
    } else {
        for (int k = 0; k < n; ++k) row[j + k] = buf[k];
    }
}

// The range [start, end) of global tile `tile` in `ids`: [offsets[tile], next offset or n_isects), or with
// bins the first min(count, capacity) slots of the tile's bin; empty when the tile's mask is 0, cut to its first
// max_list entries when max_list >= 0. Caller-supplied offsets are clamped to 0 <= start <= end <= n_isects, so
// offsets that disagree with n_isects never address outside the ids.
__device__ __forceinline__ void tile_range(const RasterArgs &a, int tile, int &start, int &end) {
    if (a.bin_counts) {
        start = tile * a.capacity;
        int c = a.bin_counts[tile];
        c = c < 0 ? 0 : (c < a.capacity ? c : a.capacity);
        end = start + c;
    } else {
        const int n = static_cast<int>(a.n_isects);
        start = min(max(a.offsets[tile], 0), n);
        end = tile + 1 < a.total_tiles ? a.offsets[tile + 1] : n;
        end = min(max(end, start), n);
    }
    if (a.masks && a.masks[tile] == 0) end = start;
    if (a.max_list >= 0 && end - start > a.max_list) end = start + a.max_list;
}

// The tile of workgroup b. Workgroups are dealt to the 8 XCDs round-robin (b on XCD b mod 8), each XCD with its own
// L2; tiles side by side stage mostly the same splats. So the grid is cut into stripes of two tile rows, stripe s
// going to XCD s mod 8: the i-th workgroup an XCD receives takes the i-th tile of its stripes, in order, and the
// tiles past the last whole round of 8 stripes go round-robin. A bijection of [0, tiles). Measured against the
// plain order on the composite alone: 1M-splat 1080p frame unchanged (0.327 vs 0.329 ms) with 31% fewer bytes
// fetched (469 vs 684 MB per launch), 6M-splat frame 6% faster, 4-camera frame 3% faster; one contiguous band per
// XCD fetched less (412 MB) but was 3% slower on the 1M-splat frame, where the splats cluster.
__device__ __forceinline__ int tile_of_block(int b, int tiles, int tile_width) {
    const int xcd = b & 7, i = b >> 3;
    const int stripe = 2 * tile_width;
    const int full = tiles / (8 * stripe);
    return i < full * stripe ? (i / stripe) * (8 * stripe) + xcd * stripe + (i % stripe) : b;
}

template <int K, int PPT, bool COUNT, bool TRACE, bool HWEXP>
__global__ __launch_bounds__(kMaxThreads) void raster_fwd_kernel(RasterArgs a) {
    __shared__ float2 s_xy[kMaxThreads];
    __shared__ float4 s_abco[kMaxThreads];
    __shared__ float s_rgb[kMaxThreads * K];
    __shared__ int32_t s_g[kMaxThreads];  // the staged ids (-1: outside [0, n_splats), e.g. an empty bin slot)

    const int tile = tile_of_block(static_cast<int>(blockIdx.x), a.total_tiles, a.tile_width);
    const int per_camera = a.tile_width * a.tile_height;
    const int camera = tile / per_camera;
    const int local = tile - camera * per_camera;
    const int ty = local / a.tile_width;
    const int tx = local - ty * a.tile_width;
    int start, end;
    tile_range(a, tile, start, end);
    const int ts = a.tile_size;
    const int nthreads = blockDim.x;

    float px[PPT], py[PPT], T[PPT], acc[PPT][K];
    int last[PPT], xs[PPT], ys[PPT], stop[PPT], steps[PPT];
    bool done[PPT];
    unsigned long long n_pass = 0, n_comp = 0, n_exec = 0, n_staged = 0;
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
        const int pix = threadIdx.x + q * nthreads;
        const int lx = pix % ts, ly = pix / ts;
        xs[q] = tx * ts + lx;
        ys[q] = ty * ts + ly;
        done[q] = !(pix < ts * ts && xs[q] < a.width && ys[q] < a.height) || (TRACE && a.max_steps == 0);
        steps[q] = 0;
        px[q] = static_cast<float>(xs[q]) + 0.5f;
        py[q] = static_cast<float>(ys[q]) + 0.5f;
        T[q] = 1.0f;
        last[q] = -1;
        stop[q] = end;
#pragma unroll
        for (int k = 0; k < K; ++k) acc[q][k] = 0.0f;
    }

    for (int base = start; base < end; base += nthreads) {
        bool mine_done = true;
#pragma unroll
        for (int q = 0; q < PPT; ++q) mine_done = mine_done && done[q];
        if (__syncthreads_and(mine_done)) break;  // also orders the previous batch's LDS reads before refilling
        const int idx = base + static_cast<int>(threadIdx.x);
        if (idx < end) {
            if (COUNT) ++n_staged;
            const int g0 = a.ids[idx];
            const int g = static_cast<unsigned>(g0) < static_cast<unsigned>(a.n_splats) ? g0 : -1;
            s_g[threadIdx.x] = g;
            if (g >= 0) {
                s_xy[threadIdx.x] = a.means[g];
                const float *cg = a.conics + 3 * static_cast<int64_t>(g);
                s_abco[threadIdx.x] = make_float4(cg[0], cg[1], cg[2], a.opacities[g]);
#pragma unroll
                for (int k = 0; k < K; ++k) s_rgb[threadIdx.x * K + k] = a.colors[static_cast<int64_t>(g) * K + k];
            }
        }
        __syncthreads();
        const int count = end - base < nthreads ? end - base : nthreads;
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            if (done[q]) continue;
            for (int j = 0; j < count; ++j) {
                if (s_g[j] < 0) continue;
                if (COUNT) ++n_exec;
                const float2 m = s_xy[j];
                const float4 c = s_abco[j];
                const float dx = m.x - px[q];
                const float dy = m.y - py[q];
                const float sigma = 0.5f * (c.x * dx * dx + c.z * dy * dy) + c.y * dx * dy;
                if (sigma < 0.0f) continue;
                float alpha = c.w * (HWEXP ? exp_neg_hw(sigma) : exp_neg(sigma));
                if (alpha > a.alpha_clamp) alpha = a.alpha_clamp;
                if (alpha < a.alpha_cutoff) continue;
                if (COUNT) ++n_pass;
                const float t_next = T[q] * (1.0f - alpha);
                if (t_next <= a.transmittance_threshold) {
                    done[q] = true;
                    if (COUNT) stop[q] = base + j + 1;
                    break;
                }
                if (COUNT) ++n_comp;
                const float v = alpha * T[q];
#pragma unroll
                for (int k = 0; k < K; ++k) acc[q][k] = acc[q][k] + s_rgb[j * K + k] * v;
                T[q] = t_next;
                last[q] = base + j;
                if (TRACE) {
                    if (a.trace_ids) {
                        const int64_t p = (static_cast<int64_t>(camera) * a.height + ys[q]) * a.width + xs[q];
                        a.trace_ids[p * a.max_steps + steps[q]] = s_g[j];
                    }
                    if (++steps[q] == a.max_steps) {
                        done[q] = true;
                        if (COUNT) stop[q] = base + j + 1;
                        break;
                    }
                }
            }
        }
    }

#pragma unroll
    for (int q = 0; q < PPT; ++q) {
        const int pix = threadIdx.x + q * nthreads;
        if (!(pix < ts * ts && xs[q] < a.width && ys[q] < a.height)) continue;
        const int64_t p = (static_cast<int64_t>(camera) * a.height + ys[q]) * a.width + xs[q];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float bg = a.backgrounds ? a.backgrounds[camera * K + k] : 0.0f;
            a.out_colors[p * K + k] = acc[q][k] + T[q] * bg;
        }
        a.out_alphas[p] = 1.0f - T[q];
        if (a.out_T) a.out_T[p] = T[q];
        if (a.out_last) a.out_last[p] = last[q];
        if (TRACE && a.trace_counts) a.trace_counts[p] = steps[q];
    }
    if (COUNT) {
        // evaluations under the definition: every splat of the range up to and including the one that stops
        // the pixel (the whole range otherwise), for each pixel inside the image
        unsigned long long n_eval = 0;
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const int pix = threadIdx.x + q * nthreads;
            if (pix < ts * ts && xs[q] < a.width && ys[q] < a.height) n_eval += static_cast<unsigned>(stop[q] - start);
        }
        atomicAdd(&a.eval_counts[0], n_eval);
        atomicAdd(&a.eval_counts[1], n_pass);
        atomicAdd(&a.eval_counts[2], n_comp);
        atomicAdd(&a.eval_counts[3], n_exec);
        atomicAdd(&a.eval_counts[4], n_staged);
    }
}

// Tiles up to 16x16, one pixel per thread. With 16x16 tiles each wave owns an 8x8 quadrant; otherwise pixels are
// row-major and a wave's region is the rows it covers. Each staged splat is one 48-byte LDS record (mean, conic,
// opacity, intersection index, colour) plus a bit per wave telling whether its alpha >= cutoff footprint can touch
// that wave's region (cull_box); a wave compacts the batch to the byte offsets of the records with its bit set, in
// order, and evaluates only those. Skipped splats would have been skipped by the cutoff test at every pixel of the
// region, so the result is the same to the bit. The evaluation loop runs in lock step without per-lane exits: a
// pixel that stops only sets `done`, and the wave leaves the loop once every lane is done. Outside the traced build
// a step has no branch either: every lane reads the colour and computes the update, and selects keep it only where
// the splat composites (the same float operations, so the same bits; 5% faster than branching on the cutoff).
template <int K, bool COUNT, bool TRACE, bool HWEXP>
__global__ __launch_bounds__(kMaxThreads, (TRACE || COUNT) ? 1 : 8) void raster_cull_kernel(RasterArgs a) {
    constexpr int kRec = 12;  // floats per record: mx my a b | c o index id | colour[4]
    __shared__ float4 s_rec[kMaxThreads * kRec / 4];
    __shared__ uint32_t s_mask[kMaxThreads];
    __shared__ uint16_t s_list[kMaxThreads / kWave][kMaxThreads];
    __shared__ int32_t s_trace[TRACE ? kMaxThreads * kTraceStride : 1];

    const int tile = tile_of_block(static_cast<int>(blockIdx.x), a.total_tiles, a.tile_width);
    const int per_camera = a.tile_width * a.tile_height;
    const int camera = tile / per_camera;
    const int local = tile - camera * per_camera;
    const int ty = local / a.tile_width;
    const int tx = local - ty * a.tile_width;
    int start, end;
    tile_range(a, tile, start, end);
    const int ts = a.tile_size;
    const int nthreads = blockDim.x;
    const int wave = threadIdx.x / kWave;
    const int lane = __lane_id();
    const bool quadrants = (ts == 16);

    // this thread's pixel
    int lx, ly;
    if (quadrants) {
        lx = (wave & 1) * 8 + (lane & 7);
        ly = (wave >> 1) * 8 + (lane >> 3);
    } else {
        lx = static_cast<int>(threadIdx.x) % ts;
        ly = static_cast<int>(threadIdx.x) / ts;
    }
    const int x = tx * ts + lx, y = ty * ts + ly;
    const bool inside = static_cast<int>(threadIdx.x) < ts * ts && x < a.width && y < a.height;
    const float px = static_cast<float>(x) + 0.5f, py = static_cast<float>(y) + 0.5f;
    const int64_t p = (static_cast<int64_t>(camera) * a.height + y) * a.width + x;

    // The pixel-centre box of wave w's region (for the cull bits), in pixel coordinates. It is rebuilt from the tile's
    // origin where it is used rather than kept for all four waves: the 16 floats held across the loop cost the step
    // its registers (the kernel then spilled).
    const int tile_x0 = tx * ts, tile_y0 = ty * ts;
    auto region = [ts, quadrants, tile_x0, tile_y0](int w, float &x0, float &x1, float &y0, float &y1) {
        int qx0, qx1, qy0, qy1;
        if (quadrants) {
            qx0 = (w & 1) * 8;
            qx1 = qx0 + 7;
            qy0 = (w >> 1) * 8;
            qy1 = qy0 + 7;
        } else {
            qx0 = 0;
            qx1 = ts - 1;
            qy0 = (w * kWave) / ts;
            qy1 = (w * kWave + kWave - 1) / ts;
        }
        x0 = static_cast<float>(tile_x0 + qx0) + 0.5f;
        x1 = static_cast<float>(tile_x0 + qx1) + 0.5f;
        y0 = static_cast<float>(tile_y0 + qy0) + 0.5f;
        y1 = static_cast<float>(tile_y0 + qy1) + 0.5f;
    };

    float T = 1.0f, acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = 0.0f;
    int last = -1, stop = end, steps = 0;
    int32_t *const my_trace = s_trace + (TRACE ? threadIdx.x * kTraceStride : 0);
    bool done = !inside || (TRACE && a.max_steps == 0);
    unsigned long long n_pass = 0, n_comp = 0, n_exec = 0, n_staged = 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const char *rec_base = reinterpret_cast<const char *>(s_rec);
    // the transmittance threshold as a bit pattern ordered against non-negative finite floats as the threshold is
    // (0 for +-0, below every such pattern when negative, above every one when NaN)
    const float thr = a.transmittance_threshold;
    const int thr_bits = thr > 0.0f ? __float_as_int(thr) : (thr == 0.0f ? 0 : (thr < 0.0f ? -1 : INT_MAX));

    for (int base = start; base < end; base += nthreads) {
        if (__syncthreads_and(done)) break;  // also orders the previous batch's LDS reads before refilling
        const int idx = base + static_cast<int>(threadIdx.x);
        const int g0 = idx < end ? a.ids[idx] : -1;
        // outside [0, n_splats) (an empty bin slot): never listed
        const int g = static_cast<unsigned>(g0) < static_cast<unsigned>(a.n_splats) ? g0 : -1;
        if (g >= 0) {
            if (COUNT) ++n_staged;
            const float2 m = a.means[g];
            const float *cg = a.conics + 3 * static_cast<int64_t>(g);
            const float ca = cg[0], cb = cg[1], cc = cg[2], o = a.opacities[g];
            float4 col = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            const float *cs = a.colors + static_cast<int64_t>(g) * K;
            col.x = cs[0];
            if (K > 1) col.y = cs[1];
            if (K > 2) col.z = cs[2];
            if (K > 3) col.w = cs[3];
            const CullBox box = cull_box(m, ca, cb, cc, o, a.alpha_cutoff, a.log_cutoff);
            // bit 31: the splat may not take the short step (its conic is not a well-conditioned positive-definite
            // one within the cull's bounds with a, c >= 2^-60, or a colour is not finite); the others hold a / 2 and
            // c / 2 (kWholeConic)
            const bool well = box.exact && ca >= 0x1p-60f && cc >= 0x1p-60f && __builtin_isfinite(col.x) &&
                              __builtin_isfinite(col.y) && __builtin_isfinite(col.z) && __builtin_isfinite(col.w);
            s_rec[threadIdx.x * 3 + 0] = make_float4(m.x, m.y, well ? 0.5f * ca : ca, cb);
            s_rec[threadIdx.x * 3 + 1] =
                make_float4(well ? 0.5f * cc : cc, o, __int_as_float(well ? idx : (idx | kWholeConic)), __int_as_float(g));
            s_rec[threadIdx.x * 3 + 2] = col;
            uint32_t bits = well ? 0u : kNotShort;
            if (!box.never && quadrants && box.exact) {
                bits |= quadrant_reach(m, ca, cb, cc, box, static_cast<float>(tile_x0), static_cast<float>(tile_y0));
            } else if (!box.never) {
#pragma unroll
                for (int w = 0; w < kMaxThreads / kWave; ++w) {
                    float qx0, qx1, qy0, qy1;
                    region(w, qx0, qx1, qy0, qy1);
                    bool touch = box.x1 >= qx0 && box.x0 <= qx1 && box.y1 >= qy0 && box.y0 <= qy1;
                    if (touch && box.exact)
                        touch = region_reach(m, ca, cb, cc, box.ra, box.rc, box.thr, qx0, qx1, qy0, qy1);
                    bits |= (touch ? 1u : 0u) << w;
                }
            }
            s_mask[threadIdx.x] = bits;
        } else if (idx < end) {
            s_mask[threadIdx.x] = 0u;
        }
        __syncthreads();
        const int count = end - base < nthreads ? end - base : nthreads;
        // this wave's splats of the batch, in order, as byte offsets of their records; whether all of them may take
        // the short step
        int listed = 0;
        bool long_step = !a.short_step;
        for (int c0 = 0; c0 < count; c0 += kWave) {
            const int j = c0 + lane;
            const uint32_t mj = j < count ? s_mask[j] : 0u;
            const bool keep = (mj >> wave) & 1u;
            long_step = long_step || __ballot(keep && (mj & kNotShort)) != 0;
            const uint64_t ballot = __ballot(keep);
            if (keep) s_list[wave][listed + __popcll(ballot & lt_mask)] = static_cast<uint16_t>(j * kRec * 4);
            listed += __popcll(ballot);
        }
        int jj = 0;
        if constexpr (!TRACE) {
            // kUnroll records per iteration: their quadratic forms and exponentials are independent chains, and the
            // steps then apply in list order (written out here and below rather than shared through a lambda, whose
            // by-reference captures cost registers)
            // The short step, for a batch whose listed splats all have well-conditioned positive-definite conics
            // (the cull's exact case: a > 0, c > 0, det > 0, trace^2 <= 1000 det, opacity in [cutoff, 1e6], mean
            // within 1e6 px; and a, c >= 2^-60, so the records hold their halves) and finite colours, with
            // alpha_cutoff >= 1e-20. It gives the bits of the step below:
            //  - such a conic's computed sigma is within 0.15% of the exact quadratic form at the same dx, dy (the
            //    cull's bound), so it is never negative and the sign test can go; an overflow gives +inf or NaN,
            //    never -inf (the cross term is at most half the diagonal terms);
            //  - sigma <= 80 takes the same polynomial (exp_neg_short, exact there); above 80, or NaN, it is taken at
            //    min(sigma, 80), which gives e^-80 < 2e-35, so alpha (at most 1e6 times that) fails the cutoff exactly
            //    as the specified alpha of 0 does, and alpha is used nowhere else;
            //  - E <= 1 keeps alpha finite, so min(alpha, clamp) is the clamp's select;
            //  - a splat that does not composite adds colour * 0 = +-0 to every accumulator, which changes none:
            //    they start at +0, and a round-to-nearest sum is -0 only when both terms are, so none is ever -0;
            //  - t_next is finite and not negative, so its order against the threshold is that of the bit patterns,
            //    and one comparison (as a wave mask and its complement) decides both halting and compositing.
            if (!long_step) {
                for (; jj + kUnroll<K> <= listed; jj += kUnroll<K>) {
                    if (__ballot(!done) == 0) break;
                    float4 q0[kUnroll<K>], col[kUnroll<K>];
                    float2 q1[kUnroll<K>];
                    int at[kUnroll<K>];
                    float al[kUnroll<K>];
#pragma unroll
                    for (int h = 0; h < kUnroll<K>; ++h) {
                        const char *r = rec_base + s_list[wave][jj + h];
                        q0[h] = *reinterpret_cast<const float4 *>(r);
                        q1[h] = *reinterpret_cast<const float2 *>(r + 16);
                        col[h] = *reinterpret_cast<const float4 *>(r + 32);
                        at[h] = __float_as_int(*reinterpret_cast<const float *>(r + 24));
                    }
#pragma unroll
                    for (int h = 0; h < kUnroll<K>; ++h) {
                        const float dx = q0[h].x - px;
                        const float dy = q0[h].y - py;
                        const float sigma = record_sigma(q0[h].z, q0[h].w, q1[h].x, false, dx, dy);
                        const float e = q1[h].y * (HWEXP ? exp_neg_hw(sigma) : exp_neg_short(fminf(sigma, 80.0f)));
                        al[h] = fminf(e, a.alpha_clamp);
                    }
#pragma unroll
                    for (int h = 0; h < kUnroll<K>; ++h) {
                        const float alpha = al[h];
                        if (COUNT && !done) ++n_exec;
                        const bool pass = !done && !(alpha < a.alpha_cutoff);
                        // t_next is finite and not negative here (alpha in [0, clamp], T in [0, 1]), so its order against
                        // the threshold is that of the bit patterns, and one comparison decides both outcomes
                        const float t_next = T * (1.0f - alpha);
                        const uint64_t above_m = __ballot(__float_as_int(t_next) > thr_bits);
                        const bool above = __builtin_amdgcn_inverse_ballot_w64(above_m);
                        const bool below = __builtin_amdgcn_inverse_ballot_w64(~above_m);
                        const bool halt = pass && below;
                        const bool comp = pass && above;
                        const float v = comp ? alpha * T : 0.0f;
                        acc[0] = acc[0] + col[h].x * v;
                        if (K > 1) acc[1] = acc[1] + col[h].y * v;
                        if (K > 2) acc[2] = acc[2] + col[h].z * v;
                        if (K > 3) acc[3] = acc[3] + col[h].w * v;
                        T = comp ? t_next : T;
                        last = comp ? at[h] : last;
                        done = done || halt;
                        if (COUNT) {
                            n_pass += pass ? 1u : 0u;
                            n_comp += comp ? 1u : 0u;
                            if (halt) stop = at[h] + 1;
                        }
                    }
                }
            }
            for (; jj + kUnroll<K> <= listed; jj += kUnroll<K>) {
                if (__ballot(!done) == 0) break;
                float4 q0[kUnroll<K>], col[kUnroll<K>];
                float2 q1[kUnroll<K>];
                int at[kUnroll<K>];
                float sg[kUnroll<K>], al[kUnroll<K>];
#pragma unroll
                for (int h = 0; h < kUnroll<K>; ++h) {
                    const char *r = rec_base + s_list[wave][jj + h];
                    q0[h] = *reinterpret_cast<const float4 *>(r);
                    q1[h] = *reinterpret_cast<const float2 *>(r + 16);
                    col[h] = *reinterpret_cast<const float4 *>(r + 32);
                    at[h] = __float_as_int(*reinterpret_cast<const float *>(r + 24));
                }
#pragma unroll
                for (int h = 0; h < kUnroll<K>; ++h) {
                    const float dx = q0[h].x - px;
                    const float dy = q0[h].y - py;
                    sg[h] = record_sigma(q0[h].z, q0[h].w, q1[h].x, at[h] < 0, dx, dy);
                    at[h] &= INT32_MAX;
                    const float e = q1[h].y * (HWEXP ? exp_neg_hw(sg[h]) : exp_neg_select(sg[h]));
                    al[h] = e > a.alpha_clamp ? a.alpha_clamp : e;
                }
#pragma unroll
                for (int h = 0; h < kUnroll<K>; ++h) {
                    const float sigma = sg[h], alpha = al[h];
                    if (COUNT && !done) ++n_exec;
                    const bool pass = !done && !(sigma < 0.0f) && !(alpha < a.alpha_cutoff);
                    const float t_next = T * (1.0f - alpha);
                    const bool halt = pass && t_next <= a.transmittance_threshold;
                    const bool comp = pass && !halt;
                    const float v = alpha * T;
                    acc[0] = comp ? acc[0] + col[h].x * v : acc[0];
                    if (K > 1) acc[1] = comp ? acc[1] + col[h].y * v : acc[1];
                    if (K > 2) acc[2] = comp ? acc[2] + col[h].z * v : acc[2];
                    if (K > 3) acc[3] = comp ? acc[3] + col[h].w * v : acc[3];
                    T = comp ? t_next : T;
                    last = comp ? at[h] : last;
                    done = done || halt;
                    if (COUNT) {
                        n_pass += pass ? 1u : 0u;
                        n_comp += comp ? 1u : 0u;
                        if (halt) stop = at[h] + 1;
                    }
                }
            }
        }
        for (; jj < listed; ++jj) {
            if (__ballot(!done) == 0) break;
            const char *rec = rec_base + s_list[wave][jj];
            const float4 r0 = *reinterpret_cast<const float4 *>(rec);
            const float2 r1 = *reinterpret_cast<const float2 *>(rec + 16);
            const int word = __float_as_int(*reinterpret_cast<const float *>(rec + 24));
            const float dx = r0.x - px;
            const float dy = r0.y - py;
            const float sigma = record_sigma(r0.z, r0.w, r1.x, word < 0, dx, dy);
            const int at = word & INT32_MAX;
            float alpha = r1.y * (HWEXP ? exp_neg_hw(sigma) : exp_neg_select(sigma));
            alpha = alpha > a.alpha_clamp ? a.alpha_clamp : alpha;
            if constexpr (!TRACE) {
                if (COUNT && !done) ++n_exec;
                const bool pass = !done && !(sigma < 0.0f) && !(alpha < a.alpha_cutoff);
                const float t_next = T * (1.0f - alpha);
                const bool halt = pass && t_next <= a.transmittance_threshold;
                const bool comp = pass && !halt;
                const float4 col = *reinterpret_cast<const float4 *>(rec + 32);
                const float v = alpha * T;
                acc[0] = comp ? acc[0] + col.x * v : acc[0];
                if (K > 1) acc[1] = comp ? acc[1] + col.y * v : acc[1];
                if (K > 2) acc[2] = comp ? acc[2] + col.z * v : acc[2];
                if (K > 3) acc[3] = comp ? acc[3] + col.w * v : acc[3];
                T = comp ? t_next : T;
                last = comp ? at : last;
                done = done || halt;
                if (COUNT) {
                    n_pass += pass ? 1u : 0u;
                    n_comp += comp ? 1u : 0u;
                    if (halt) stop = at + 1;
                }
            } else {
                if (COUNT && !done) ++n_exec;
                if (!done && !(sigma < 0.0f) && !(alpha < a.alpha_cutoff)) {
                    if (COUNT) ++n_pass;
                    const float t_next = T * (1.0f - alpha);
                    if (t_next <= a.transmittance_threshold) {
                        done = true;
                        if (COUNT) stop = at + 1;
                    } else {
                        if (COUNT) ++n_comp;
                        const float4 col = *reinterpret_cast<const float4 *>(rec + 32);
                        const float v = alpha * T;
                        acc[0] = acc[0] + col.x * v;
                        if (K > 1) acc[1] = acc[1] + col.y * v;
                        if (K > 2) acc[2] = acc[2] + col.z * v;
                        if (K > 3) acc[3] = acc[3] + col.w * v;
                        T = t_next;
                        last = at;
                        my_trace[steps & (kTraceChunk - 1)] =
                            __float_as_int(*reinterpret_cast<const float *>(rec + 28));
                        ++steps;
                        if (a.trace_ids && (steps & (kTraceChunk - 1)) == 0)
                            flush_trace(a.trace_ids + p * a.max_steps, steps - kTraceChunk, my_trace, kTraceChunk,
                                        a.trace_vec);
                        if (steps == a.max_steps) {
                            done = true;
                            if (COUNT) stop = last + 1;
                        }
                    }
                }
            }
        }
    }

    if (inside) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float bg = a.backgrounds ? a.backgrounds[camera * K + k] : 0.0f;
            a.out_colors[p * K + k] = acc[k] + T * bg;
        }
        a.out_alphas[p] = 1.0f - T;
        if (a.out_T) a.out_T[p] = T;
        if (a.out_last) a.out_last[p] = last;
        if (TRACE && a.trace_counts) a.trace_counts[p] = steps;
        if (TRACE && a.trace_ids) {
            // the steps after the last full chunk
            const int r = steps & (kTraceChunk - 1);
            flush_trace(a.trace_ids + p * a.max_steps, steps - r, my_trace, r, false);
        }
    }
    if (COUNT) {
        const unsigned long long n_eval = inside ? static_cast<unsigned>(stop - start) : 0u;
        atomicAdd(&a.eval_counts[0], n_eval);
        atomicAdd(&a.eval_counts[1], n_pass);
        atomicAdd(&a.eval_counts[2], n_comp);
        atomicAdd(&a.eval_counts[3], n_exec);
        atomicAdd(&a.eval_counts[4], n_staged);
    }
}

template <int K, bool COUNT, bool TRACE, bool HWEXP>
gs_status launch_kct(const RasterArgs &args, int threads, int ppt, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.total_tiles)), block(static_cast<unsigned>(threads));
    if (ppt == 1) hipLaunchKernelGGL((raster_cull_kernel<K, COUNT, TRACE, HWEXP>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((raster_fwd_kernel<K, 4, COUNT, TRACE, HWEXP>), grid, block, 0, stream, args);
    GS_LAUNCH_TRY("raster_fwd_kernel");
    return ok();
}

// builds: the specified exponential with or without a trace, and the hardware exponential without one
template <int K>
gs_status launch_k(const RasterArgs &args, int threads, int ppt, bool trace, bool hw_exp, hipStream_t stream) {
    const bool count = args.eval_counts != nullptr;
    if (hw_exp)
        return count ? launch_kct<K, true, false, true>(args, threads, ppt, stream)
                     : launch_kct<K, false, false, true>(args, threads, ppt, stream);
    if (trace)
        return count ? launch_kct<K, true, true, false>(args, threads, ppt, stream)
                     : launch_kct<K, false, true, false>(args, threads, ppt, stream);
    return count ? launch_kct<K, true, false, false>(args, threads, ppt, stream)
                 : launch_kct<K, false, false, false>(args, threads, ppt, stream);
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_rasterize_workspace_bytes(int64_t C, int tile_width, int tile_height) {
    if (C < 1 || tile_width < 1 || tile_height < 1) return 0;
    return align_up(static_cast<size_t>(C) * tile_width * tile_height * sizeof(int32_t), 256);
}

namespace {

gs_status rasterize(const char *fn, const float *means2d, const float *conics, const float *colors,
                    const float *opacities, const float *backgrounds, int64_t C, int64_t N, int K, int width,
                    int height, int tile_size, int tile_width, int tile_height, const int32_t *isect_offsets,
                    const int32_t *flatten_ids, int64_t n_isects, const int32_t *bin_counts, int capacity,
                    const int32_t *masks, float alpha_cutoff,
                    float alpha_clamp, float transmittance_threshold, int max_list_entries, int max_splat_steps,
                    float *render_colors, float *render_alphas, float *render_T, int32_t *last_ids,
                    int32_t *trace_ids, int32_t *trace_counts, int exp_mode, uint64_t *eval_counts,
                    void *workspace, size_t workspace_bytes, void *stream_handle) {
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    if (C < 1 || N < 0 || C * N >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "%s: need C >= 1, N >= 0 and C*N < 2^31", fn);
    if (K < 1 || K > 4) return fail(GS_ERR_INVALID_ARG, "%s: K = %d channels outside [1, 4]", fn, K);
    if (width < 1 || height < 1 || tile_size < 1 || tile_size > 32)
        return fail(GS_ERR_INVALID_ARG, "%s: need width, height >= 1 and 1 <= tile_size <= 32", fn);
    if (tile_width != (width + tile_size - 1) / tile_size || tile_height != (height + tile_size - 1) / tile_size)
        return fail(GS_ERR_INVALID_ARG,
                    "%s: tile grid %dx%d does not match ceil(%d/%d) x ceil(%d/%d)", fn, tile_width,
                    tile_height, width, tile_size, height, tile_size);
    const int64_t total_tiles = C * tile_width * tile_height;
    if (total_tiles >= (int64_t(1) << 31) || C * height * width * K >= (int64_t(1) << 40))
        return fail(GS_ERR_INVALID_ARG, "%s: image batch too large", fn);
    if (bin_counts) {
        // fixed-capacity bins: the ids array is [C, th, tw, capacity]
        if (capacity < 1 || total_tiles * capacity >= (int64_t(1) << 31))
            return fail(GS_ERR_INVALID_ARG, "%s: need capacity >= 1 and C*th*tw*capacity < 2^31", fn);
        n_isects = total_tiles * capacity;
    } else if (!isect_offsets) {
        return fail(GS_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    }
    if (n_isects < 0 || n_isects >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "%s: n_isects = %lld outside [0, 2^31)", fn, (long long)n_isects);
    if (!render_colors || !render_alphas || (n_isects > 0 && !flatten_ids) ||
        (N > 0 && (!means2d || !conics || !colors || !opacities)))
        return fail(GS_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (!(alpha_cutoff >= 0.0f) || !(alpha_clamp > 0.0f) || !(transmittance_threshold >= 0.0f))
        return fail(GS_ERR_INVALID_ARG, "%s: alpha_cutoff >= 0, alpha_clamp > 0 and "
                                        "transmittance_threshold >= 0 are required", fn);
    const size_t need = gs_rasterize_workspace_bytes(C, tile_width, tile_height);
    if (workspace_bytes > 0 && workspace_bytes < need)
        return fail(GS_ERR_WORKSPACE, "%s: needs %zu workspace bytes (got %zu)", fn, need, workspace_bytes);

    RasterArgs args{};
    args.means = reinterpret_cast<const float2 *>(means2d);
    args.conics = conics;
    args.colors = colors;
    args.opacities = opacities;
    args.backgrounds = backgrounds;
    args.offsets = isect_offsets;
    args.ids = flatten_ids;
    args.n_isects = n_isects;
    args.n_splats = static_cast<int>(C * N);
    args.masks = masks;
    args.total_tiles = static_cast<int>(total_tiles);
    args.width = width;
    args.height = height;
    args.tile_size = tile_size;
    args.tile_width = tile_width;
    args.tile_height = tile_height;
    args.alpha_cutoff = alpha_cutoff;
    args.alpha_clamp = alpha_clamp;
    args.transmittance_threshold = transmittance_threshold;
    args.out_colors = render_colors;
    args.out_alphas = render_alphas;
    args.out_T = render_T;
    args.out_last = last_ids;
    args.eval_counts = reinterpret_cast<unsigned long long *>(eval_counts);
    args.log_cutoff = alpha_cutoff > 0.0f ? static_cast<float>(std::log(static_cast<double>(alpha_cutoff))) : -INFINITY;
    args.max_list = max_list_entries < 0 ? -1 : max_list_entries;
    args.max_steps = max_splat_steps;
    args.trace_ids = trace_ids;
    args.trace_counts = trace_counts;
    args.trace_vec = (max_splat_steps % 4 == 0 && (reinterpret_cast<uintptr_t>(trace_ids) & 15) == 0) ? 1 : 0;
    args.bin_counts = bin_counts;
    args.capacity = capacity;
    args.short_step = alpha_cutoff >= 1.0e-20f ? 1 : 0;
    const bool trace = max_splat_steps >= 0;
    if (exp_mode != 0 && exp_mode != 1) return fail(GS_ERR_INVALID_ARG, "%s: exp_mode %d is not 0 or 1", fn, exp_mode);
    if (exp_mode == 1 && trace) return fail(GS_ERR_INVALID_ARG, "%s: the hardware exponential has no traced build", fn);

    const int pixels = tile_size * tile_size;
    int threads, ppt;
    if (pixels <= kMaxThreads) {
        threads = (pixels + kWave - 1) / kWave * kWave;
        ppt = 1;
    } else {
        threads = kMaxThreads;
        ppt = 4;
    }
    switch (K) {
        case 1: return launch_k<1>(args, threads, ppt, trace, exp_mode == 1, stream);
        case 2: return launch_k<2>(args, threads, ppt, trace, exp_mode == 1, stream);
        case 3: return launch_k<3>(args, threads, ppt, trace, exp_mode == 1, stream);
        default: return launch_k<4>(args, threads, ppt, trace, exp_mode == 1, stream);
    }
}

}  // namespace

extern "C" gs_status gs_rasterize_fwd(const float *means2d, const float *conics, const float *colors,
                                      const float *opacities, const float *backgrounds, int64_t C, int64_t N, int K,
                                      int width, int height, int tile_size, int tile_width, int tile_height,
                                      const int32_t *isect_offsets, const int32_t *flatten_ids, int64_t n_isects,
                                      const int32_t *masks, float alpha_cutoff, float alpha_clamp,
                                      float transmittance_threshold,
                                      float *render_colors, float *render_alphas, float *render_T, int32_t *last_ids,
                                      uint64_t *eval_counts, void *workspace, size_t workspace_bytes,
                                      void *stream_handle) {
    return rasterize("gs_rasterize_fwd", means2d, conics, colors, opacities, backgrounds, C, N, K, width, height,
                     tile_size, tile_width, tile_height, isect_offsets, flatten_ids, n_isects, nullptr, 0, masks,
                     alpha_cutoff, alpha_clamp, transmittance_threshold, -1, -1, render_colors, render_alphas,
                     render_T, last_ids, nullptr, nullptr, 0, eval_counts, workspace, workspace_bytes, stream_handle);
}

extern "C" gs_status gs_rasterize_fwd_traced(const float *means2d, const float *conics, const float *colors,
                                             const float *opacities, const float *backgrounds, int64_t C, int64_t N,
                                             int K, int width, int height, int tile_size, int tile_width,
                                             int tile_height, const int32_t *isect_offsets,
                                             const int32_t *flatten_ids, int64_t n_isects, const int32_t *masks,
                                             float alpha_cutoff, float alpha_clamp, float transmittance_threshold,
                                             int max_list_entries, int max_splat_steps, float *render_colors,
                                             float *render_alphas, float *render_T, int32_t *last_ids,
                                             int32_t *trace_ids, int32_t *trace_counts, uint64_t *eval_counts,
                                             void *workspace, size_t workspace_bytes, void *stream_handle) {
    if (max_splat_steps < 0)
        return fail(GS_ERR_INVALID_ARG, "gs_rasterize_fwd_traced: max_splat_steps = %d must be >= 0", max_splat_steps);
    return rasterize("gs_rasterize_fwd_traced", means2d, conics, colors, opacities, backgrounds, C, N, K, width,
                     height, tile_size, tile_width, tile_height, isect_offsets, flatten_ids, n_isects, nullptr, 0,
                     masks, alpha_cutoff, alpha_clamp, transmittance_threshold, max_list_entries, max_splat_steps,
                     render_colors, render_alphas, render_T, last_ids, trace_ids, trace_counts, 0, eval_counts,
                     workspace, workspace_bytes, stream_handle);
}

extern "C" gs_status gs_rasterize_fwd_bins(const float *means2d, const float *conics, const float *colors,
                                           const float *opacities, const float *backgrounds, int64_t C, int64_t N,
                                           int K, int width, int height, int tile_size, int tile_width,
                                           int tile_height, const int32_t *bin_ids, const int32_t *bin_counts,
                                           int capacity, float alpha_cutoff, float alpha_clamp,
                                           float transmittance_threshold, float *render_colors, float *render_alphas,
                                           float *render_T, int32_t *last_ids, uint64_t *eval_counts,
                                           void *stream_handle) {
    if (!bin_counts) return fail(GS_ERR_INVALID_ARG, "gs_rasterize_fwd_bins: bin_counts is NULL");
    return rasterize("gs_rasterize_fwd_bins", means2d, conics, colors, opacities, backgrounds, C, N, K, width,
                     height, tile_size, tile_width, tile_height, nullptr, bin_ids, 0, bin_counts, capacity, nullptr,
                     alpha_cutoff, alpha_clamp, transmittance_threshold, -1, -1, render_colors, render_alphas,
                     render_T, last_ids, nullptr, nullptr, 0, eval_counts, nullptr, 0, stream_handle);
}

extern "C" gs_status gs_rasterize_fwd_hwexp(const float *means2d, const float *conics, const float *colors,
                                            const float *opacities, const float *backgrounds, int64_t C, int64_t N,
                                            int K, int width, int height, int tile_size, int tile_width,
                                            int tile_height, const int32_t *isect_offsets,
                                            const int32_t *flatten_ids, int64_t n_isects, const int32_t *masks,
                                            float alpha_cutoff, float alpha_clamp, float transmittance_threshold,
                                            float *render_colors, float *render_alphas, float *render_T,
                                            int32_t *last_ids, uint64_t *eval_counts, void *stream_handle) {
    return rasterize("gs_rasterize_fwd_hwexp", means2d, conics, colors, opacities, backgrounds, C, N, K, width,
                     height, tile_size, tile_width, tile_height, isect_offsets, flatten_ids, n_isects, nullptr, 0,
                     masks, alpha_cutoff, alpha_clamp, transmittance_threshold, -1, -1, render_colors,
                     render_alphas, render_T, last_ids, nullptr, nullptr, 1, eval_counts, nullptr, 0, stream_handle);
}

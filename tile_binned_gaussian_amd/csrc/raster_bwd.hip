// Backward of the per-tile composite on gfx950: for L = <grad_colors, render_colors> + <grad_alphas,
// render_alphas>, the gradients of the splats' means, conics, colours and opacities (and of the background).
//
// One workgroup per tile, one pixel per thread (tiles up to 32x32). Each pixel rebuilds its state from the
// forward's outputs (final transmittance 1 - render_alpha, last composited index) and walks the tile's range back
// to front; batches of splats are staged through LDS from the back, with the same exact per-wave cull as the
// forward (a splat whose alpha stays below the cutoff over a wave's pixels contributes nothing there). For every
// staged splat that at least one lane of a wave uses, each gradient term is summed over each 16-lane row by DPP
// adds and the row sums are added into the splat's LDS accumulators; after the batch, one thread per splat adds
// them to the splat's gradient with float atomics (one set per splat and tile).
//
// Definition: gsplat 1.0.0 raster_backward.c, gs_raster_backward_pixel (the per-pixel back-to-front recurrence
// and its gradient terms) and gs_raster_backward_without_gvl (the tile walk), with the forward's exponential.
#include "raster_common.hpp"

namespace gs {
namespace {


struct BwdArgs {
    const float2 *means;
    const float *conics;
    const float *colors;
    const float *opacities;
    const float *backgrounds;
    const int32_t *offsets;
    const int32_t *ids;
    const int32_t *masks;  // nullable [C, th, tw]: 0 = no splat gradients from this tile
    int64_t n_isects;
    int n_splats;  // C * N: ids outside [0, n_splats) are skipped (never gathered, never given gradients)
    int total_tiles, width, height, tile_size, tile_width, tile_height;
    float alpha_cutoff, alpha_clamp, log_cutoff;
    const float *render_alphas;
    const int32_t *last_ids;
    const float *grad_colors_px;
    const float *grad_alphas_px;
    float *g_means, *g_conics, *g_colors, *g_opacities, *g_backgrounds, *g_means_abs;
};

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_read(float v) {
    // lanes the pattern does not reach (or rows outside kRowMask) read 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask,
                                                                 0xf, true));
}

// Sum of v over each row of 16 lanes, valid in lanes 15, 31, 47 and 63. Every lane must be active. Steps: swap
// neighbours and pairs within quads (every lane holds its quad's sum), then shift rows right by 4 and by 8.
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_read<0xb1, 0xf>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_read<0x4e, 0xf>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_read<0x114, 0xf>(v);  // row_shr:4
    v += dpp_read<0x118, 0xf>(v);  // row_shr:8
    return v;
}

// Sum of v over the 64 lanes, valid in lane 63: the row sums, then lane 15 broadcast into the next row (lane 31
// holds rows 0-1, lane 63 rows 2-3) and lane 31 into rows 2-3.
__device__ __forceinline__ float wave_sum_last(float v) {
    v = row_sum(v);
    v += dpp_read<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_read<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Adds the wave's sum of v to *dst in device memory (one lane, one hardware float atomic), skipping exact zeros.
__device__ __forceinline__ void wave_add(float v, float *dst, int lane) {
    const float s = wave_sum_last(v);
    if (lane == kWave - 1 && s != 0.0f) unsafeAtomicAdd(dst, s);
}

// Adds the four row sums of each of the N values to acc[0..N) in LDS (LDS float atomics, exact zeros skipped).
// For N >= 8 the first 8 values are reduced scatter-wise: in the two quad steps each lane keeps one half of every
// pair of values and adds its partner's copy of that half (value 2i + bit 0 of the lane after the first step, and
// q or q + 4, q = lane & 3, after the second), so each lane carries 2 of the 8 values through the row shifts by 4
// and by 8, and lanes 12-15 of a row end with the row sums of values q and q + 4. Values 8.. and all values when
// N < 8 take the plain steps (every lane of a quad keeps every sum; lane 15 of the row ends with the row sum).
// Every sum still has 4 levels of additions. The DPP steps of independent sums are interleaved.
template <int N>
__device__ __forceinline__ void rows_add_lds(float (&v)[N], float *acc, int lane) {
    if constexpr (N >= 8) {
        const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
        float w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float send = b0 ? v[2 * i] : v[2 * i + 1];
            const float keep = b0 ? v[2 * i + 1] : v[2 * i];
            w[i] = keep + dpp_read<0xb1, 0xf>(send);  // quad_perm [1, 0, 3, 2]
        }
#pragma unroll
        for (int i = 8; i < N; ++i) v[i] += dpp_read<0xb1, 0xf>(v[i]);
        float u[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float send = b1 ? w[2 * i] : w[2 * i + 1];
            const float keep = b1 ? w[2 * i + 1] : w[2 * i];
            u[i] = keep + dpp_read<0x4e, 0xf>(send);  // quad_perm [2, 3, 0, 1]
        }
#pragma unroll
        for (int i = 8; i < N; ++i) v[i] += dpp_read<0x4e, 0xf>(v[i]);
#pragma unroll
        for (int i = 0; i < 2; ++i) u[i] += dpp_read<0x114, 0xf>(u[i]);  // row_shr:4
#pragma unroll
        for (int i = 8; i < N; ++i) v[i] += dpp_read<0x114, 0xf>(v[i]);
#pragma unroll
        for (int i = 0; i < 2; ++i) u[i] += dpp_read<0x118, 0xf>(u[i]);  // row_shr:8
#pragma unroll
        for (int i = 8; i < N; ++i) v[i] += dpp_read<0x118, 0xf>(v[i]);
        if ((lane & 15) >= 12) {
            const int q = lane & 3;
            if (u[0] != 0.0f) atomicAdd(&acc[q], u[0]);
            if (u[1] != 0.0f) atomicAdd(&acc[q + 4], u[1]);
        }
        if ((lane & 15) == 15) {
#pragma unroll
            for (int i = 8; i < N; ++i)
                if (v[i] != 0.0f) atomicAdd(&acc[i], v[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += dpp_read<0xb1, 0xf>(v[i]);   // quad_perm [1, 0, 3, 2]
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += dpp_read<0x4e, 0xf>(v[i]);   // quad_perm [2, 3, 0, 1]
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += dpp_read<0x114, 0xf>(v[i]);  // row_shr:4
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += dpp_read<0x118, 0xf>(v[i]);  // row_shr:8
        if ((lane & 15) == 15) {
#pragma unroll
            for (int i = 0; i < N; ++i)
                if (v[i] != 0.0f) atomicAdd(&acc[i], v[i]);
        }
    }
}

template <int K, int kThreads>
__global__ __launch_bounds__(kThreads) void raster_bwd_kernel(BwdArgs a) {
    constexpr int kRec = 12;  // floats per record: mx my a b | c o index splat | colour[4]
    constexpr int kWaves = kThreads / kWave;
    // splats staged per round: 128 for 256-thread tiles keeps the workgroup at 13 KB of LDS, so 7 workgroups fit a CU
    // (the 71 registers allow 7 waves per SIMD; 256 splats, 27 KB, allowed 6): 1.7% faster on the 1M-splat frame
    constexpr int kBatch = kThreads > 256 ? 256 : 128;
    __shared__ float4 s_rec[kBatch * kRec / 4];
    __shared__ uint32_t s_mask[kBatch];
    __shared__ uint16_t s_list[kWaves][kBatch];
    __shared__ int s_top[kWaves];
    constexpr int kAcc = K + 6 + 2;  // colour[K], opacity, mean x y, conic a b c, |mean| x y
    __shared__ float s_acc[kBatch][kAcc];

    const int tile = static_cast<int>(blockIdx.x);
    const int per_camera = a.tile_width * a.tile_height;
    const int camera = tile / per_camera;
    const int local = tile - camera * per_camera;
    const int ty = local / a.tile_width;
    const int tx = local - ty * a.tile_width;
    // caller-supplied offsets clamped to 0 <= start <= end <= n_isects (never an access outside the ids); a tile
    // whose mask is 0 composites nothing (its range is taken as empty)
    const int n_all = static_cast<int>(a.n_isects);
    const int start = min(max(a.offsets[tile], 0), n_all);
    const int end_raw = tile + 1 < a.total_tiles ? a.offsets[tile + 1] : n_all;
    const int end = (a.masks && a.masks[tile] == 0) ? start : min(max(end_raw, start), n_all);
    const int ts = a.tile_size;
    const int nwaves = static_cast<int>(blockDim.x) / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = __lane_id();
    const bool quadrants = (ts == 16);

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

    // pixel state from the forward's outputs
    float gc[K], rest[K];
    float ga = 0.0f, ra = 0.0f;
    int last = -1;
#pragma unroll
    for (int k = 0; k < K; ++k) gc[k] = 0.0f;
    if (inside) {
        ra = a.render_alphas[p];
        last = a.last_ids[p];
        ga = a.grad_alphas_px[p];
#pragma unroll
        for (int k = 0; k < K; ++k) gc[k] = a.grad_colors_px[p * K + k];
    }
    float T = 1.0f - ra;
    float after = 1.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) rest[k] = a.backgrounds ? a.backgrounds[camera * K + k] : 0.0f;
    if (a.g_backgrounds) {
#pragma unroll
        for (int k = 0; k < K; ++k) wave_add(inside ? gc[k] * T : 0.0f, &a.g_backgrounds[camera * K + k], lane);
    }
    // a pixel takes part only with render_alpha > 0; it never uses an index past its last composited one
    const bool live = inside && ra > 0.0f;
    if (!live) last = -1;
    int wave_top = last;
    for (int d = 1; d < kWave; d <<= 1) wave_top = max(wave_top, __shfl_xor(wave_top, d, kWave));
    if (lane == 0) s_top[wave] = wave_top;

    // pixel-centre boxes of every wave's region, for the cull bits
    float rx0[kWaves], rx1[kWaves], ry0[kWaves], ry1[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
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
        rx0[w] = static_cast<float>(tx * ts + qx0) + 0.5f;
        rx1[w] = static_cast<float>(tx * ts + qx1) + 0.5f;
        ry0[w] = static_cast<float>(ty * ts + qy0) + 0.5f;
        ry1[w] = static_cast<float>(ty * ts + qy1) + 0.5f;
    }
    __syncthreads();
    int block_top = -1;
    for (int w = 0; w < nwaves; ++w) block_top = max(block_top, s_top[w]);
    const int top = min(end, block_top + 1);  // no pixel of the tile uses an index at or past this
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const char *rec_base = reinterpret_cast<const char *>(s_rec);

    for (int hi = top; hi > start; hi -= kBatch) {
        const int lo = hi - kBatch > start ? hi - kBatch : start;
        const int count = hi - lo;
        __syncthreads();  // the previous batch's LDS reads are complete
        for (int slot = static_cast<int>(threadIdx.x); slot < count; slot += static_cast<int>(blockDim.x)) {
            const int idx = lo + slot;
            const int g = a.ids[idx];
#pragma unroll
            for (int v = 0; v < kAcc; ++v) s_acc[slot][v] = 0.0f;
            if (static_cast<unsigned>(g) >= static_cast<unsigned>(a.n_splats)) {
                s_mask[slot] = 0u;  // never listed, so its accumulators stay zero and nothing is added for it
                continue;
            }
            const float2 m = a.means[g];
            const float *cg = a.conics + 3 * static_cast<int64_t>(g);
            const float ca = cg[0], cb = cg[1], cc = cg[2], o = a.opacities[g];
            float4 col = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            const float *cs = a.colors + static_cast<int64_t>(g) * K;
            col.x = cs[0];
            if (K > 1) col.y = cs[1];
            if (K > 2) col.z = cs[2];
            if (K > 3) col.w = cs[3];
            s_rec[slot * 3 + 0] = make_float4(m.x, m.y, ca, cb);
            s_rec[slot * 3 + 1] = make_float4(cc, o, __int_as_float(idx), __int_as_float(g));
            s_rec[slot * 3 + 2] = col;
            const CullBox box = cull_box(m, ca, cb, cc, o, a.alpha_cutoff, a.log_cutoff);
            uint32_t bits = 0;
            if (!box.never) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    bool touch = w < nwaves && box.x1 >= rx0[w] && box.x0 <= rx1[w] && box.y1 >= ry0[w] &&
                                 box.y0 <= ry1[w];
                    if (touch && box.exact)
                        touch = region_reach(m, ca, cb, cc, box.ra, box.rc, box.thr, rx0[w], rx1[w], ry0[w], ry1[w]);
                    bits |= (touch ? 1u : 0u) << w;
                }
            }
            s_mask[slot] = bits;
        }
        __syncthreads();
        // this wave's splats of the batch from the back, as byte offsets of their records
        int listed = 0;
        for (int c0 = count - 1; c0 >= 0; c0 -= kWave) {
            const int j = c0 - lane;
            const bool keep = j >= 0 && lo + j <= wave_top && ((s_mask[j] >> wave) & 1u);
            const uint64_t ballot = __ballot(keep);
            if (keep) s_list[wave][listed + __popcll(ballot & lt_mask)] = static_cast<uint16_t>(j * kRec * 4);
            listed += __popcll(ballot);
        }
        for (int jj = 0; jj < listed; ++jj) {
            const char *rec = rec_base + s_list[wave][jj];
            const float4 r0 = *reinterpret_cast<const float4 *>(rec);
            const float4 r1 = *reinterpret_cast<const float4 *>(rec + 16);
            const int idx = __float_as_int(r1.z);
            const float dx = r0.x - px;
            const float dy = r0.y - py;
            const float sigma = 0.5f * (r0.z * dx * dx + r1.x * dy * dy) + r0.w * dx * dy;
            const float response = exp_neg_select(sigma);
            const float raw = r1.y * response;
            const float alpha = raw > a.alpha_clamp ? a.alpha_clamp : raw;
            const bool valid = idx <= last && sigma >= 0.0f && alpha >= a.alpha_cutoff && T < 1.0f && alpha < 1.0f;
            if (__ballot(valid) == 0) continue;
            const float4 col = *reinterpret_cast<const float4 *>(rec + 32);
            const float cv[4] = {col.x, col.y, col.z, col.w};
            const float before = T / (1.0f - alpha);
            const float vis = before * alpha;
            float dot = 0.0f;
            float t_col[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                t_col[k] = gc[k] * vis;
                dot += gc[k] * (cv[k] - rest[k]);
            }
            const float g_alpha = before * (dot + ga * after);
            const float g_raw = raw < a.alpha_clamp ? g_alpha : 0.0f;
            const float t_op = g_raw * response;
            const float g_sigma = -g_raw * raw;
            const float t_mx = g_sigma * (r0.z * dx + r0.w * dy);
            const float t_my = g_sigma * (r1.x * dy + r0.w * dx);
            const float t_ca = g_sigma * 0.5f * dx * dx;
            const float t_cb = g_sigma * dx * dy;
            const float t_cc = g_sigma * 0.5f * dy * dy;
            float *acc = s_acc[s_list[wave][jj] / (kRec * 4)];
            float terms[K + 6];
#pragma unroll
            for (int k = 0; k < K; ++k) terms[k] = valid ? t_col[k] : 0.0f;
            terms[K] = valid ? t_op : 0.0f;
            terms[K + 1] = valid ? t_mx : 0.0f;
            terms[K + 2] = valid ? t_my : 0.0f;
            terms[K + 3] = valid ? t_ca : 0.0f;
            terms[K + 4] = valid ? t_cb : 0.0f;
            terms[K + 5] = valid ? t_cc : 0.0f;
            rows_add_lds(terms, acc, lane);
            if (a.g_means_abs) {
                float mag[2] = {valid ? fabsf(t_mx) : 0.0f, valid ? fabsf(t_my) : 0.0f};
                rows_add_lds(mag, acc + K + 6, lane);
            }
            if (valid) {
#pragma unroll
                for (int k = 0; k < K; ++k) rest[k] = alpha * cv[k] + (1.0f - alpha) * rest[k];
                after *= 1.0f - alpha;
                T = before;
            }
        }
        // the batch's sums per splat (over this tile's pixels) into the splats' gradients
        __syncthreads();
        for (int slot = static_cast<int>(threadIdx.x); slot < count; slot += static_cast<int>(blockDim.x)) {
            const float *acc = s_acc[slot];
            const int64_t g = __float_as_int(s_rec[slot * 3 + 1].w);
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (acc[k] != 0.0f) unsafeAtomicAdd(&a.g_colors[g * K + k], acc[k]);
            if (acc[K] != 0.0f) unsafeAtomicAdd(&a.g_opacities[g], acc[K]);
            if (acc[K + 1] != 0.0f) unsafeAtomicAdd(&a.g_means[g * 2], acc[K + 1]);
            if (acc[K + 2] != 0.0f) unsafeAtomicAdd(&a.g_means[g * 2 + 1], acc[K + 2]);
            if (acc[K + 3] != 0.0f) unsafeAtomicAdd(&a.g_conics[g * 3], acc[K + 3]);
            if (acc[K + 4] != 0.0f) unsafeAtomicAdd(&a.g_conics[g * 3 + 1], acc[K + 4]);
            if (acc[K + 5] != 0.0f) unsafeAtomicAdd(&a.g_conics[g * 3 + 2], acc[K + 5]);
            if (a.g_means_abs) {
                if (acc[K + 6] != 0.0f) unsafeAtomicAdd(&a.g_means_abs[g * 2], acc[K + 6]);
                if (acc[K + 7] != 0.0f) unsafeAtomicAdd(&a.g_means_abs[g * 2 + 1], acc[K + 7]);
            }
        }
    }
}

template <int K>
gs_status launch_bwd(const BwdArgs &args, int threads, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.total_tiles)), block(static_cast<unsigned>(threads));
    if (threads <= 256) hipLaunchKernelGGL((raster_bwd_kernel<K, 256>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((raster_bwd_kernel<K, 1024>), grid, block, 0, stream, args);
    GS_LAUNCH_TRY("raster_bwd_kernel");
    return ok();
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" gs_status gs_rasterize_bwd(const float *means2d, const float *conics, const float *colors,
                                      const float *opacities, const float *backgrounds, int64_t C, int64_t N, int K,
                                      int width, int height, int tile_size, int tile_width, int tile_height,
                                      const int32_t *isect_offsets, const int32_t *flatten_ids, int64_t n_isects,
                                      const int32_t *masks, float alpha_cutoff, float alpha_clamp,
                                      const float *render_alphas,
                                      const int32_t *last_ids, const float *grad_render_colors,
                                      const float *grad_render_alphas, float *grad_means2d, float *grad_conics,
                                      float *grad_colors, float *grad_opacities, float *grad_backgrounds,
                                      float *grad_means2d_abs, void *stream_handle) {
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    if (C < 1 || N < 0 || C * N >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_rasterize_bwd: need C >= 1, N >= 0 and C*N < 2^31");
    if (K < 1 || K > 4) return fail(GS_ERR_INVALID_ARG, "gs_rasterize_bwd: K = %d channels outside [1, 4]", K);
    if (width < 1 || height < 1 || tile_size < 1 || tile_size > 32)
        return fail(GS_ERR_INVALID_ARG, "gs_rasterize_bwd: need width, height >= 1 and 1 <= tile_size <= 32");
    if (tile_width != (width + tile_size - 1) / tile_size || tile_height != (height + tile_size - 1) / tile_size)
        return fail(GS_ERR_INVALID_ARG,
                    "gs_rasterize_bwd: tile grid %dx%d does not match ceil(%d/%d) x ceil(%d/%d)", tile_width,
                    tile_height, width, tile_size, height, tile_size);
    const int64_t total_tiles = C * tile_width * tile_height;
    if (total_tiles >= (int64_t(1) << 31) || C * height * width * K >= (int64_t(1) << 40))
        return fail(GS_ERR_INVALID_ARG, "gs_rasterize_bwd: image batch too large");
    if (n_isects < 0 || n_isects >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_rasterize_bwd: n_isects = %lld outside [0, 2^31)", (long long)n_isects);
    if (!isect_offsets || !render_alphas || !last_ids || !grad_render_colors || !grad_render_alphas ||
        (n_isects > 0 && !flatten_ids) ||
        (N > 0 && (!means2d || !conics || !colors || !opacities || !grad_means2d || !grad_conics || !grad_colors ||
                   !grad_opacities)))
        return fail(GS_ERR_INVALID_ARG, "gs_rasterize_bwd: a required pointer is NULL");
    if (!(alpha_cutoff >= 0.0f) || !(alpha_clamp > 0.0f))
        return fail(GS_ERR_INVALID_ARG, "gs_rasterize_bwd: alpha_cutoff >= 0 and alpha_clamp > 0 are required");

    // the gradients are sums: clear them first (fill kernels, so the work can sit in a graph)
    const size_t M = static_cast<size_t>(C * N);
    if (M > 0) {
        GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(grad_means2d), 0, M * 2, stream));
        GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(grad_conics), 0, M * 3, stream));
        GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(grad_colors), 0, M * K, stream));
        GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(grad_opacities), 0, M, stream));
        if (grad_means2d_abs) GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(grad_means2d_abs), 0, M * 2, stream));
    }
    if (grad_backgrounds)
        GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(grad_backgrounds), 0, static_cast<size_t>(C) * K, stream));

    BwdArgs args{};
    args.means = reinterpret_cast<const float2 *>(means2d);
    args.conics = conics;
    args.colors = colors;
    args.opacities = opacities;
    args.backgrounds = backgrounds;
    args.offsets = isect_offsets;
    args.n_splats = static_cast<int>(C * N);
    args.ids = flatten_ids;
    args.n_isects = n_isects;
    args.masks = masks;
    args.total_tiles = static_cast<int>(total_tiles);
    args.width = width;
    args.height = height;
    args.tile_size = tile_size;
    args.tile_width = tile_width;
    args.tile_height = tile_height;
    args.alpha_cutoff = alpha_cutoff;
    args.alpha_clamp = alpha_clamp;
    args.log_cutoff = alpha_cutoff > 0.0f ? static_cast<float>(std::log(static_cast<double>(alpha_cutoff))) : -INFINITY;
    args.render_alphas = render_alphas;
    args.last_ids = last_ids;
    args.grad_colors_px = grad_render_colors;
    args.grad_alphas_px = grad_render_alphas;
    args.g_means = grad_means2d;
    args.g_conics = grad_conics;
    args.g_colors = grad_colors;
    args.g_opacities = grad_opacities;
    args.g_backgrounds = grad_backgrounds;
    args.g_means_abs = grad_means2d_abs;

    const int pixels = tile_size * tile_size;
    const int threads = (pixels + kWave - 1) / kWave * kWave;
    switch (K) {
        case 1: return launch_bwd<1>(args, threads, stream);
        case 2: return launch_bwd<2>(args, threads, stream);
        case 3: return launch_bwd<3>(args, threads, stream);
        default: return launch_bwd<4>(args, threads, stream);
    }
}

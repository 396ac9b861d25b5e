/*
 * Plain, slow CPU oracle for the tile-binned splat rasterizer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
 * this file (built plain, and once more with OpenMP for the multi-core baseline and the largest test frames, where
 * the emission's splats, the merge sort's merges and the composite's tiles run in parallel with the same
 * per-element arithmetic). It shares no code, header, table or constant with the HIP library; the two meet only at the
 * seeded synthetic inputs.
 *
 * Sources (the pages the method is defined on):
 *   [gsplat] gsplat 1.0.0 Ruby gem, native C extension, file intersections.c: gs_tile_bits, gs_clamp_tile,
 *            gs_bounds, gs_radix_sort_without_gvl, gs_isect_tiles, gs_offset_encode.
 *   [gsplat-bwd] same gem, raster_backward.c: gs_raster_backward_pixel and gs_raster_backward_without_gvl,
 *            whose per-splat quantities (pixel centre, delta, quadratic form, alpha, clamp, skip test, range
 *            end) fix what the forward computes; the forward itself is not on the pages and is read as the
 *            front-to-back inverse of that backward.
 *   [rlx-metal] rlx-metal 0.2.9 splat_training.rs, training_forward_metal_traced: names alpha_cutoff and
 *            transmittance_threshold as forward parameters, and a cutoff default of 1/255; names the traced
 *            forward's max_splat_steps (per-pixel trace of composited splats kept for the backward: counts and
 *            ids) and the tile-list cap max_list_entries (orc_rasterize_fwd_traced).
 *   The composite's backward (orc_rasterize_bwd) is the exact gradient of the forward, the quantity whose
 *            back-to-front recurrence [gsplat-bwd] gs_raster_backward_pixel evaluates, computed here from
 *            front-to-back transmittances and suffix sums in double, with a derived bound for float32 evaluations.
 *   [gsplat-proj] the same gem's projection.c (gs_mat3_product, gs_camera_covar, gs_clip, gs_project_one): the
 *            EWA projection of 3D Gaussians into cameras (orc_project).
 *   [pytorch3d-fine] PyTorch3D rasterize_meshes.cu, RasterizeMeshesFineCudaKernel: reads per-bin lists of fixed
 *            capacity with -1 in empty slots (orc_bin_tiles, orc_rasterize_bins: the fixed-capacity alternative to
 *            sort-based binning).
 *
 * Arithmetic: float32 wherever the pages compute in float (all of the above do), evaluated in the pages'
 * expression order with no contraction (build with -ffp-contract=off, never -ffast-math); fmaf appears only
 * where the exponential below names it. Integer work is exact.
 *
 * Parity pins: every exported function here is checked by the CPU test suite (tests/test_oracle_*.py) against
 * closed forms, brute-force enumerations, library routines, invariants or another pinned oracle function, and each
 * pin is shown to catch a planted mistake in a mutated copy of this file (tests/oracle_mutants.py); none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_INVALID_ARG 1
#define ORC_ERR_OUT_OF_GRID 2
#define ORC_ERR_NOMEM 3

/* Smallest b >= 0 with 2^b >= count: [gsplat] gs_tile_bits (ceil(log2(w*h)); 0 for one tile).
 * The same rule gives the camera field width from C. */
/* Threads the compositing loop may use: the OpenMP maximum in the OpenMP build, 1 otherwise (not part of the
 * method; reported beside the CPU timings). */
#ifdef _OPENMP
#include <omp.h>
int orc_threads(void) { return omp_get_max_threads(); }
#else
int orc_threads(void) { return 1; }
#endif

int orc_bits_for(int64_t count)
{
    int bits = 0;
    uint64_t capacity = 1;
    while (capacity < (uint64_t)count) {
        capacity <<= 1;
        bits += 1;
    }
    return bits;
}

/* floor/ceil result -> tile index clamped to [0, maximum] ([gsplat] gs_clamp_tile). The clamp is taken on the
 * float before the int conversion so that huge or non-finite values are defined (NaN maps to 0); for finite
 * in-range values this equals converting first and clamping after. */
static int orc_clamp_tile(float value, int maximum)
{
    if (!(value > 0.0f)) return 0;
    if (value > (float)maximum) return maximum;
    return (int)value;
}

/* Tile rectangle [x0,x1) x [y0,y1) of one splat ([gsplat] gs_bounds). A non-positive radius gives the empty
 * rectangle. The division is by the tile size converted to float, as in the pages. */
void orc_bounds(float mean_x, float mean_y, float radius_x, float radius_y, int tile_size, int tile_width,
                int tile_height, int32_t bounds[4])
{
    if (radius_x <= 0.0f || radius_y <= 0.0f) {
        bounds[0] = bounds[1] = bounds[2] = bounds[3] = 0;
        return;
    }
    float ts = (float)tile_size;
    bounds[0] = orc_clamp_tile(floorf((mean_x - radius_x) / ts), tile_width);
    bounds[1] = orc_clamp_tile(floorf((mean_y - radius_y) / ts), tile_height);
    bounds[2] = orc_clamp_tile(ceilf((mean_x + radius_x) / ts), tile_width);
    bounds[3] = orc_clamp_tile(ceilf((mean_y + radius_y) / ts), tile_height);
}

static void orc_bounds_of(const float *means2d, const float *radii, int radii_per_gauss, int64_t index,
                          int tile_size, int tile_width, int tile_height, int32_t bounds[4])
{
    float rx = radii[index * radii_per_gauss];
    float ry = radii_per_gauss == 2 ? radii[index * 2 + 1] : rx;
    orc_bounds(means2d[index * 2], means2d[index * 2 + 1], rx, ry, tile_size, tile_width, tile_height, bounds);
}

/* Step 1 of [gsplat] gs_isect_tiles: per (camera, splat) tile count = clamped rectangle area, in row-major
 * [C, N] order, and the running write index (exclusive prefix) at which each splat's keys start.
 * Returns the total number of intersections. */
int64_t orc_isect_count(const float *means2d, const float *radii, int radii_per_gauss, int64_t C, int64_t N,
                        int tile_size, int tile_width, int tile_height, int32_t *tiles_per_gauss,
                        int64_t *gauss_offsets)
{
    int64_t total = 0;
    for (int64_t index = 0; index < C * N; ++index) {
        int32_t b[4];
        orc_bounds_of(means2d, radii, radii_per_gauss, index, tile_size, tile_width, tile_height, b);
        int64_t count = (int64_t)(b[2] - b[0]) * (int64_t)(b[3] - b[1]);
        if (tiles_per_gauss) tiles_per_gauss[index] = (int32_t)count;
        if (gauss_offsets) gauss_offsets[index] = total;
        total += count;
    }
    return total;
}

/* The 64-bit intersection key of [gsplat] gs_isect_tiles: the camera index above the tile index in the upper 32 bits
 * (the tile taking the low tile_bits of them), the depth's IEEE bit pattern in the lower 32. */
static uint64_t orc_pack_key(uint64_t camera, int tile_bits, uint64_t tile, uint32_t depth_bits)
{
    uint64_t upper = (camera << tile_bits) | tile;
    return (upper << 32) | (uint64_t)depth_bits;
}

/* Step 2 of [gsplat] gs_isect_tiles, stated per output slot: splat i (flat index camera * N + splat) owns the
 * slots [start_i, start_i + count_i), start_i being the exclusive prefix of the counts in flat order; its k-th
 * slot holds the k-th tile of its rectangle in row-major order, i.e. row y0 + k / w and column x0 + k % w with
 * w = x1 - x0, as key orc_pack_key(camera, tile_bits, row * tile_width + column, depth bits) and id i.
 * Writes exactly n_isects entries; returns 0. */
int orc_isect_emit(const float *means2d, const float *radii, int radii_per_gauss, const float *depths,
                   int64_t C, int64_t N, int tile_size, int tile_width, int tile_height, uint64_t *keys,
                   int32_t *flatten_ids)
{
    const int tile_bits = orc_bits_for((int64_t)tile_width * tile_height);
    const int64_t M = C * N;
    int64_t *start = (int64_t *)malloc((size_t)(M > 0 ? M : 1) * sizeof(int64_t));
    if (!start) return ORC_ERR_NOMEM;
    int64_t running = 0;
    for (int64_t i = 0; i < M; ++i) {
        int32_t r[4];
        orc_bounds_of(means2d, radii, radii_per_gauss, i, tile_size, tile_width, tile_height, r);
        start[i] = running;
        running += (int64_t)(r[2] - r[0]) * (int64_t)(r[3] - r[1]);
    }
    /* every splat writes only its own slots; the OpenMP build hands splats to the host's threads */
#pragma omp parallel for schedule(dynamic, 4096)
    for (int64_t i = 0; i < M; ++i) {
        int32_t r[4];
        orc_bounds_of(means2d, radii, radii_per_gauss, i, tile_size, tile_width, tile_height, r);
        const int64_t w = r[2] - r[0], count = w * (int64_t)(r[3] - r[1]);
        uint32_t depth_bits;
        memcpy(&depth_bits, &depths[i], sizeof depth_bits);
        for (int64_t k = 0; k < count; ++k) {
            const int64_t row = r[1] + k / w, column = r[0] + k % w;
            keys[start[i] + k] = orc_pack_key((uint64_t)(i / N), tile_bits,
                                              (uint64_t)(row * tile_width + column), depth_bits);
            flatten_ids[start[i] + k] = (int32_t)i;
        }
    }
    free(start);
    return ORC_OK;
}

/* Stable ascending sort of (key, id) pairs by the unsigned key. [gsplat] gs_radix_sort_without_gvl is a
 * stable LSD radix sort over all 64 bits, so its result is the stable order by key; written here as a plain
 * bottom-up merge sort, which is stable by construction (ties take the left run first). */
int orc_sort_pairs(uint64_t *keys, int32_t *ids, int64_t n)
{
    if (n < 2) return ORC_OK;
    uint64_t *tk = (uint64_t *)malloc((size_t)n * sizeof(uint64_t));
    int32_t *ti = (int32_t *)malloc((size_t)n * sizeof(int32_t));
    if (!tk || !ti) {
        free(tk);
        free(ti);
        return ORC_ERR_NOMEM;
    }
    uint64_t *sk = keys, *dk = tk;
    int32_t *si = ids, *di = ti;
    for (int64_t width = 1; width < n; width *= 2) {
        /* the merges of one pass are independent (the OpenMP build runs them on the host's threads) */
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t lo = 0; lo < n; lo += 2 * width) {
            int64_t mid = lo + width < n ? lo + width : n;
            int64_t hi = lo + 2 * width < n ? lo + 2 * width : n;
            int64_t a = lo, b = mid, o = lo;
            while (a < mid && b < hi) {
                if (sk[b] < sk[a]) {
                    dk[o] = sk[b];
                    di[o++] = si[b++];
                } else {
                    dk[o] = sk[a];
                    di[o++] = si[a++];
                }
            }
            while (a < mid) {
                dk[o] = sk[a];
                di[o++] = si[a++];
            }
            while (b < hi) {
                dk[o] = sk[b];
                di[o++] = si[b++];
            }
        }
        uint64_t *xk = sk;
        sk = dk;
        dk = xk;
        int32_t *xi = si;
        si = di;
        di = xi;
    }
    if (sk != keys) {
        memcpy(keys, sk, (size_t)n * sizeof(uint64_t));
        memcpy(ids, si, (size_t)n * sizeof(int32_t));
    }
    free(tk);
    free(ti);
    return ORC_OK;
}

/* The global tile camera * (w * h) + tile of a key, whose upper 32 bits hold camera << tile_bits | tile; -1 when
 * the camera or the tile lies outside the grid ([gsplat] gs_offset_encode rejects such a key). */
static int64_t orc_key_tile(uint64_t key, int tile_bits, int64_t C, int64_t per_camera)
{
    const uint64_t upper = key >> 32;
    const uint64_t camera = upper >> tile_bits;
    const uint64_t tile = upper - (camera << tile_bits);
    if (camera >= (uint64_t)C || tile >= (uint64_t)per_camera) return -1;
    return (int64_t)camera * per_camera + (int64_t)tile;
}

/* [gsplat] gs_offset_encode's output: offsets[t] = the number of keys whose global tile is below t, for every global
 * tile t of the [C, h, w] grid, so that tile t's keys are [offsets[t], offsets[t + 1]) (the last ending at n) in a
 * sorted key array. Counted here as the number of keys per tile, each tile's offset the previous tile's plus the
 * previous tile's count. A key outside the grid is an error (the pages raise ArgError). */
int orc_tile_offsets(const uint64_t *keys, int64_t n, int64_t C, int tile_width, int tile_height,
                     int32_t *offsets)
{
    const int tile_bits = orc_bits_for((int64_t)tile_width * tile_height);
    const int64_t per_camera = (int64_t)tile_width * tile_height;
    const int64_t tiles = C * per_camera;
    int64_t *per_tile = (int64_t *)calloc((size_t)(tiles > 0 ? tiles : 1), sizeof(int64_t));
    if (!per_tile) return ORC_ERR_NOMEM;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t t = orc_key_tile(keys[i], tile_bits, C, per_camera);
        if (t < 0) {
            free(per_tile);
            return ORC_ERR_OUT_OF_GRID;
        }
        per_tile[t] += 1;
    }
    for (int64_t t = 0; t < tiles; ++t) offsets[t] = t == 0 ? 0 : (int32_t)(offsets[t - 1] + per_tile[t - 1]);
    free(per_tile);
    return ORC_OK;
}

/* e^(-sigma) in float32 by Cody-Waite range reduction and a Taylor polynomial (W. J. Cody and W. Waite,
 * "Software Manual for the Elementary Functions", 1980, exponential chapter):
 *   k = nearest integer to -sigma / ln 2,   r = -sigma - k ln 2 (ln 2 split in a high part with trailing zero
 *   bits and a low correction, both applied with fmaf),   e^(-sigma) = 2^k * sum_{j<=7} r^j / j!.
 * Any sigma above 80 (or NaN) returns 0: e^-80 is far below any usable alpha, and the cut keeps every returned
 * value a normal float (k >= -116). The pages call the C library expf; this reading fixes one exponential
 * so that alpha, and every decision made on it, is reproducible to the bit. */
static const float ORC_LOG2E = 1.44269502162933349609375f;         /* nearest float to 1/ln 2 */
static const float ORC_LN2_HI = 0.693145751953125f;                /* ln 2 to 15 significant bits */
static const float ORC_LN2_LO = 1.428606765330187045037746429443359375e-6f; /* ln 2 - ORC_LN2_HI, rounded */

float orc_exp_neg(float sigma)
{
    if (!(sigma <= 80.0f)) return 0.0f;
    float t = -sigma;
    float k = rintf(t * ORC_LOG2E);
    float r = fmaf(-k, ORC_LN2_HI, t);
    r = fmaf(-k, ORC_LN2_LO, r);
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)k);
}

/* Elementwise orc_exp_neg over an array (for sweeps in the tests). */
void orc_exp_neg_array(const float *sigma, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_neg(sigma[i]);
}

/* The forward's per-splat quantities at the pixel centre (px, py), float32 in the expression order of [gsplat-bwd]
 * gs_raster_backward_pixel: d = mean - centre; sigma = 0.5 (a dx dx + c dy dy) + b dx dy with the conic (a, b, c);
 * E = orc_exp_neg(sigma); raw = opacity E; alpha = min(clamp, raw) (a NaN raw stays NaN). */
typedef struct {
    float dx, dy, sigma, E, raw, alpha;
} orc_eval;

static orc_eval orc_evaluate(const float *means2d, const float *conics, const float *opacities, int64_t g, float px,
                             float py, float alpha_clamp)
{
    orc_eval e;
    float a = conics[g * 3], b = conics[g * 3 + 1], c = conics[g * 3 + 2];
    e.dx = means2d[g * 2] - px;
    e.dy = means2d[g * 2 + 1] - py;
    e.sigma = 0.5f * (a * e.dx * e.dx + c * e.dy * e.dy) + b * e.dx * e.dy;
    e.E = orc_exp_neg(e.sigma);
    e.raw = opacities[g] * e.E;
    e.alpha = e.raw > alpha_clamp ? alpha_clamp : e.raw;
    return e;
}

/* Front-to-back compositing of one pixel over list[start, end) (the forward read from [gsplat-bwd]):
 *   centre (x + 0.5, y + 0.5); d = mean - centre;
 *   sigma = 0.5 * (a dx dx + c dy dy) + b dx dy with the conic (a, b, c), each product and sum rounded to float;
 *   sigma < 0 -> skip; alpha = min(clamp, opacity * e^-sigma); alpha < cutoff -> skip;
 *   T' = T (1 - alpha); T' <= threshold -> stop before this splat ([rlx-metal] transmittance_threshold);
 *   otherwise colour += colour_g * (alpha T), T = T', last = position.
 * The traced variant ([rlx-metal] max_splat_steps): a composited splat is one step; with max_steps >= 0 the
 * pixel stops right after its max_steps-th step (at once when max_steps is 0), and trace (nullable) receives the
 * flat splat id of each step in order. *steps_out (nullable) receives the number of steps.
 * Writes acc[K], the final transmittance and the last composited position (-1 if none); counts every
 * evaluation of sigma (including the stopping one) into *n_eval. */
void orc_composite_pixel_traced(const float *means2d, const float *conics, const float *colors,
                                const float *opacities, int K, const int32_t *list, int64_t start, int64_t end,
                                int x, int y, float alpha_cutoff, float alpha_clamp, float transmittance_threshold,
                                int64_t max_steps, float *acc, float *T_out, int64_t *last_out, int64_t *n_eval,
                                int32_t *trace, int64_t *steps_out)
{
    float px = (float)x + 0.5f;
    float py = (float)y + 0.5f;
    float T = 1.0f;
    int64_t last = -1;
    int64_t steps = 0;
    for (int k = 0; k < K; ++k) acc[k] = 0.0f;
    for (int64_t i = start; i < end; ++i) {
        if (max_steps >= 0 && steps >= max_steps) break;
        int64_t g = list[i];
        orc_eval e = orc_evaluate(means2d, conics, opacities, g, px, py, alpha_clamp);
        if (n_eval) *n_eval += 1;
        if (e.sigma < 0.0f) continue;
        float alpha = e.alpha;
        if (alpha < alpha_cutoff) continue;
        float T_next = T * (1.0f - alpha);
        if (T_next <= transmittance_threshold) break;
        float v = alpha * T;
        for (int k = 0; k < K; ++k) acc[k] = acc[k] + colors[g * K + k] * v;
        T = T_next;
        last = i;
        if (trace) trace[steps] = (int32_t)g;
        steps += 1;
    }
    *T_out = T;
    *last_out = last;
    if (steps_out) *steps_out = steps;
}

/* The untraced composite of one pixel: orc_composite_pixel_traced with no step cap and no trace. */
void orc_composite_pixel(const float *means2d, const float *conics, const float *colors,
                         const float *opacities, int K, const int32_t *list, int64_t start, int64_t end,
                         int x, int y, float alpha_cutoff, float alpha_clamp, float transmittance_threshold,
                         float *acc, float *T_out, int64_t *last_out, int64_t *n_eval)
{
    orc_composite_pixel_traced(means2d, conics, colors, opacities, K, list, start, end, x, y, alpha_cutoff,
                               alpha_clamp, transmittance_threshold, -1, acc, T_out, last_out, n_eval, NULL, NULL);
}

/* Forward rasterization over tiles ([gsplat-bwd] gs_raster_backward_without_gvl for the tile walk): global
 * tile t = (camera * th + ty) * tw + tx, its range [offsets[t], t + 1 < T ? offsets[t + 1] : n), the tile's
 * pixels clipped to width x height. Outputs per pixel: colour = acc + T * background (0 without one),
 * alpha = 1 - T, T, and last id (global intersection index, -1 if nothing composited).
 * tiles == NULL processes every tile; otherwise only the n_tiles listed (other pixels are left untouched).
 * masks (nullable, [C, th, tw] int32): a tile whose mask is 0 composites nothing (its pixels show the background,
 * T = 1, last id -1); the backward page skips such tiles' splats, which fixes this reading of the forward.
 * Traced variant ([rlx-metal] training_forward_metal_traced):
 *   max_list_entries >= 0 keeps only the first max_list_entries entries of every tile's list (the nearest
 *   ones); a negative value keeps whole lists;
 *   max_splat_steps >= 0 caps every pixel at that many composited splats (orc_composite_pixel_traced); a
 *   negative value leaves pixels uncapped;
 *   trace_ids (nullable, [C, H, W, max_splat_steps] int32) receives each pixel's composited flat splat ids in
 *   front-to-back order, entries past the pixel's count untouched; trace_counts (nullable, [C, H, W] int32)
 *   receives the count. Tracing needs max_splat_steps >= 0 (the row length).
 * Returns the number of sigma evaluations, or -1 for a bad argument. */
int64_t orc_rasterize_fwd_traced(const float *means2d, const float *conics, const float *colors,
                                 const float *opacities, const float *backgrounds, int64_t C, int K, int width,
                                 int height, int tile_size, int tile_width, int tile_height, const int32_t *offsets,
                                 const int32_t *flatten_ids, int64_t n_isects, const int32_t *masks,
                                 float alpha_cutoff, float alpha_clamp, float transmittance_threshold,
                                 const int64_t *tiles, int64_t n_tiles, int64_t max_list_entries,
                                 int64_t max_splat_steps, float *render_colors, float *render_alphas,
                                 float *render_T, int32_t *last_ids, int32_t *trace_ids, int32_t *trace_counts)
{
    int64_t per_camera = (int64_t)tile_width * tile_height;
    int64_t total_tiles = C * per_camera;
    int64_t count = tiles ? n_tiles : total_tiles;
    int64_t n_eval = 0;
    if (K < 1 || K > 64) return -1;
    if ((trace_ids || trace_counts) && max_splat_steps < 0) return -1;
    for (int64_t j = 0; tiles && j < count; ++j)
        if (tiles[j] < 0 || tiles[j] >= total_tiles) return -1;
    /* Tiles are independent (each writes only its own pixels and trace rows). Built with OpenMP, the tiles are
     * handed out one at a time to the host's threads - the pages' CPU parallelisation of compositing - with the
     * same per-pixel arithmetic; without OpenMP the pragma is ignored and the loop runs in order. */
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : n_eval)
    for (int64_t j = 0; j < count; ++j) {
        float acc[64];
        int64_t t = tiles ? tiles[j] : j;
        int64_t camera = t / per_camera;
        int64_t local = t % per_camera;
        int ty = (int)(local / tile_width), tx = (int)(local % tile_width);
        int64_t start = offsets[t];
        int64_t end = t + 1 < total_tiles ? offsets[t + 1] : n_isects;
        if (masks && masks[t] == 0) end = start; /* a masked tile composites nothing: background, T = 1 */
        if (max_list_entries >= 0 && end - start > max_list_entries) end = start + max_list_entries;
        for (int y = ty * tile_size; y < (ty + 1) * tile_size && y < height; ++y) {
            for (int x = tx * tile_size; x < (tx + 1) * tile_size && x < width; ++x) {
                float T;
                int64_t last, steps;
                int64_t pixel = (camera * height + y) * (int64_t)width + x;
                int32_t *trace = trace_ids ? trace_ids + pixel * max_splat_steps : NULL;
                orc_composite_pixel_traced(means2d, conics, colors, opacities, K, flatten_ids, start, end, x, y,
                                           alpha_cutoff, alpha_clamp, transmittance_threshold, max_splat_steps,
                                           acc, &T, &last, &n_eval, trace, &steps);
                for (int k = 0; k < K; ++k) {
                    float bg = backgrounds ? backgrounds[camera * K + k] : 0.0f;
                    render_colors[pixel * K + k] = acc[k] + T * bg;
                }
                render_alphas[pixel] = 1.0f - T;
                if (render_T) render_T[pixel] = T;
                if (last_ids) last_ids[pixel] = (int32_t)last;
                if (trace_counts) trace_counts[pixel] = (int32_t)steps;
            }
        }
    }
    return n_eval;
}

/* The untraced forward: orc_rasterize_fwd_traced with whole lists and no step cap. */
int64_t orc_rasterize_fwd(const float *means2d, const float *conics, const float *colors,
                          const float *opacities, const float *backgrounds, int64_t C, int K, int width,
                          int height, int tile_size, int tile_width, int tile_height, const int32_t *offsets,
                          const int32_t *flatten_ids, int64_t n_isects, const int32_t *masks, float alpha_cutoff,
                          float alpha_clamp, float transmittance_threshold, const int64_t *tiles, int64_t n_tiles,
                          float *render_colors, float *render_alphas, float *render_T, int32_t *last_ids)
{
    return orc_rasterize_fwd_traced(means2d, conics, colors, opacities, backgrounds, C, K, width, height, tile_size,
                                    tile_width, tile_height, offsets, flatten_ids, n_isects, masks, alpha_cutoff,
                                    alpha_clamp, transmittance_threshold, tiles, n_tiles, -1, -1, render_colors,
                                    render_alphas, render_T, last_ids, NULL, NULL);
}

/* Composite the pixels of one global tile over an explicit front-to-back list of flat ids (the same per-pixel
 * rule as orc_rasterize_fwd). Outputs are [ts*ts] per-tile arrays in row-major pixel order; pixels outside the
 * image are left untouched. last_pos indexes `list` (-1 if nothing composited). Returns the evaluation count. */
int64_t orc_rasterize_tile(const float *means2d, const float *conics, const float *colors, const float *opacities,
                           const float *backgrounds, int K, int width, int height, int tile_size, int tile_width,
                           int tile_height, int64_t tile, const int32_t *list, int64_t count, float alpha_cutoff,
                           float alpha_clamp, float transmittance_threshold, float *out_colors, float *out_T,
                           int64_t *out_last_pos)
{
    int64_t per_camera = (int64_t)tile_width * tile_height;
    int64_t camera = tile / per_camera;
    int64_t local = tile % per_camera;
    int ty = (int)(local / tile_width), tx = (int)(local % tile_width);
    int64_t n_eval = 0;
    float acc[64];
    if (K < 1 || K > 64) return -1;
    for (int ly = 0; ly < tile_size; ++ly) {
        for (int lx = 0; lx < tile_size; ++lx) {
            int x = tx * tile_size + lx, y = ty * tile_size + ly;
            if (x >= width || y >= height) continue;
            float T;
            int64_t last;
            orc_composite_pixel(means2d, conics, colors, opacities, K, list, 0, count, x, y, alpha_cutoff,
                                alpha_clamp, transmittance_threshold, acc, &T, &last, &n_eval);
            int64_t q = (int64_t)ly * tile_size + lx;
            for (int k = 0; k < K; ++k) {
                float bg = backgrounds ? backgrounds[camera * K + k] : 0.0f;
                out_colors[q * K + k] = acc[k] + T * bg;
            }
            out_T[q] = T;
            out_last_pos[q] = last;
        }
    }
    return n_eval;
}

/* Backward of the composite: the gradient of L = sum over pixels of <grad_colors_px, colour> + grad_alphas_px * alpha
 * with respect to every splat's colour, opacity, mean and conic (and the background), for the forward above ([gsplat-bwd]
 * gs_raster_backward_pixel and gs_raster_backward_without_gvl state the same gradient as a back-to-front recurrence).
 *
 * Definition used here, per pixel. The composited splats j = 1..L are the positions i of the tile's range with
 * i <= last_id, sigma >= 0, alpha >= cutoff and alpha < 1 (none when render_alpha is 0 or the tile's mask is 0), each with
 * the forward's float32 alpha_j, raw_j = opacity E_j and E_j (orc_evaluate). In exact arithmetic on those values:
 *   T_1 = 1, T_{j+1} = T_j (1 - alpha_j) (front-to-back transmittance), T_f = T_{L+1};
 *   colour C_k = sum_j c_jk alpha_j T_j + T_f bg_k,  alpha = 1 - T_f;
 *   S_jk = sum_{l > j} c_lk alpha_l T_l + T_f bg_k (the suffix sum behind splat j), so that
 *   dC_k / d alpha_j = c_jk T_j - S_jk / (1 - alpha_j),  d alpha / d alpha_j = T_f / (1 - alpha_j);
 *   dL/d alpha_j = sum_k g_k dC_k/d alpha_j + g_a T_f / (1 - alpha_j); dL/d raw_j = that, or 0 where the clamp holds
 *   (raw_j >= clamp); dL/d opacity_j += dL/d raw_j E_j; d raw / d sigma = -raw, and with d = mean - centre (exact,
 *   from the float inputs) d sigma / d mean = (a dx + b dy, c dy + b dx), d sigma / d(a, b, c) = (dx^2/2, dx dy, dy^2/2);
 *   dL/d c_jk = g_k alpha_j T_j;  dL/d bg_k = g_k T_f.
 * Evaluated in double: T by products from the front, S by sums from the back (so no division rebuilds a
 * transmittance). g_means_abs (nullable) receives per splat and axis the sum over pixels of |dL/d mean|.
 *
 * Error bound for a float32 evaluation of the same gradient by the pages' recurrence (transmittance rebuilt back to
 * front from 1 - render_alpha by divisions, the colour behind a splat and the transmittance behind it updated step by
 * step, the pages' operation order for each term). With u = 2^-24 and, per pixel, phi = (8 L + K + 12) u + u / T_f:
 * every term t of that pixel is within phi * M(t) of its exact value, where M(t) is t with every sum replaced by the
 * sum of magnitudes (|g_k| (|c_jk| T_j + |S|_jk / (1 - alpha_j)) + |g_a| T_f / (1 - alpha_j) in place of dL/d alpha_j,
 * |a dx| + |b dy| in place of a dx + b dy, and so on). The u / T_f part is the rounding of render_alpha = 1 - T_f,
 * which every rebuilt transmittance of the pixel inherits; 2L + 1 rounding steps come from the forward's and the
 * backward's transmittance chains each, 4L from the colour-behind recurrence, K + 12 from the term's own operations.
 * abs_* receive the sums of |t| over the terms of each entry and err_* the sums of phi * M(t) (all nullable); a float
 * sum of the terms in any order with at most D additions on a path then lies within err + D u abs (to first order).
 * g_bg, abs_bg and err_bg may be NULL (no background gradient). masks (nullable, [C, th, tw]): a tile whose mask is 0
 * contributes only its pixels' background terms.
 * Returns 0, -1 for a bad argument, -2 if an allocation failed. */
typedef struct {
    int64_t g;
    double alpha, raw, E, T, dx, dy;
    int unclamped;
} orc_bwd_step;

static void orc_acc(double *g, double *abs_sum, double *err, int64_t at, double term, double magnitude,
                    double phi)
{
    g[at] += term;
    if (abs_sum) abs_sum[at] += fabs(term);
    if (err) err[at] += phi * magnitude;
}

int orc_rasterize_bwd(const float *means2d, const float *conics, const float *colors, const float *opacities,
                      const float *backgrounds, int64_t C, int64_t N, int K, int width, int height, int tile_size,
                      int tile_width, int tile_height, const int32_t *offsets, const int32_t *flatten_ids,
                      int64_t n_isects, const int32_t *masks, float alpha_cutoff, float alpha_clamp,
                      const float *render_alphas, const int32_t *last_ids, const float *grad_colors_px,
                      const float *grad_alphas_px,
                      double *g_means, double *g_conics, double *g_colors, double *g_opacities, double *g_bg,
                      double *g_means_abs, double *abs_means, double *abs_conics, double *abs_colors,
                      double *abs_opacities, double *abs_bg, double *err_means, double *err_conics,
                      double *err_colors, double *err_opacities, double *err_bg)
{
    const double u = ldexp(1.0, -24);
    int64_t per_camera = (int64_t)tile_width * tile_height;
    int64_t total_tiles = C * per_camera;
    if (K < 1 || K > 64 || N < 0 || C < 1) return -1;
    int64_t longest = 1;
    for (int64_t t = 0; t < total_tiles; ++t) {
        int64_t e = t + 1 < total_tiles ? offsets[t + 1] : n_isects;
        if (e - offsets[t] > longest) longest = e - offsets[t];
    }
    orc_bwd_step *steps = (orc_bwd_step *)malloc((size_t)longest * sizeof(orc_bwd_step));
    if (!steps) return -2;
    double S[64], S_abs[64];
    for (int64_t t = 0; t < total_tiles; ++t) {
        int64_t camera = t / per_camera;
        int64_t local = t % per_camera;
        int ty = (int)(local / tile_width), tx = (int)(local % tile_width);
        int64_t start = offsets[t];
        int64_t end = t + 1 < total_tiles ? offsets[t + 1] : n_isects;
        if (masks && masks[t] == 0) end = start;
        for (int y = ty * tile_size; y < (ty + 1) * tile_size && y < height; ++y) {
            for (int x = tx * tile_size; x < (tx + 1) * tile_size && x < width; ++x) {
                int64_t pixel = (camera * height + y) * (int64_t)width + x;
                const float *gk = grad_colors_px + pixel * K;
                double ga = grad_alphas_px[pixel];
                float px = (float)x + 0.5f, py = (float)y + 0.5f;
                /* the composited splats, front to back, with the transmittance in front of each */
                int64_t stop = (int64_t)last_ids[pixel] + 1;
                if (!(render_alphas[pixel] > 0.0f)) stop = start;
                if (stop > end) stop = end;
                int64_t L = 0;
                double T = 1.0;
                for (int64_t i = start; i < stop; ++i) {
                    int64_t g = flatten_ids[i];
                    orc_eval e = orc_evaluate(means2d, conics, opacities, g, px, py, alpha_clamp);
                    if (!(e.sigma >= 0.0f) || !(e.alpha >= alpha_cutoff) || !(e.alpha < 1.0f)) continue;
                    orc_bwd_step *st = &steps[L++];
                    st->g = g;
                    st->alpha = e.alpha;
                    st->raw = e.raw;
                    st->E = e.E;
                    st->T = T;
                    st->dx = (double)means2d[g * 2] - (double)px;
                    st->dy = (double)means2d[g * 2 + 1] - (double)py;
                    st->unclamped = e.raw < alpha_clamp;
                    T *= 1.0 - (double)e.alpha;
                }
                const double T_f = T;
                const double phi = (8.0 * (double)L + (double)K + 12.0) * u + u / T_f;
                for (int k = 0; k < K; ++k) {
                    double bg = backgrounds ? backgrounds[camera * K + k] : 0.0;
                    S[k] = T_f * bg;
                    S_abs[k] = T_f * fabs(bg);
                    if (g_bg) orc_acc(g_bg, abs_bg, err_bg, camera * K + k, gk[k] * T_f, fabs(gk[k]) * T_f, phi);
                }
                /* back to front: each splat's gradient from the suffix sums behind it */
                for (int64_t j = L - 1; j >= 0; --j) {
                    const orc_bwd_step *st = &steps[j];
                    const int64_t g = st->g;
                    const float *col = colors + g * K;
                    const double one_minus = 1.0 - st->alpha, w = st->alpha * st->T;
                    double d_alpha = ga * T_f / one_minus;
                    double m_alpha = fabs(ga) * T_f / one_minus;
                    for (int k = 0; k < K; ++k) {
                        d_alpha += gk[k] * (col[k] * st->T - S[k] / one_minus);
                        m_alpha += fabs(gk[k]) * (fabs(col[k]) * st->T + S_abs[k] / one_minus);
                        orc_acc(g_colors, abs_colors, err_colors, g * K + k, gk[k] * w, fabs(gk[k]) * w, phi);
                    }
                    const double d_raw = st->unclamped ? d_alpha : 0.0;
                    const double m_raw = st->unclamped ? m_alpha : 0.0;
                    orc_acc(g_opacities, abs_opacities, err_opacities, g, d_raw * st->E, m_raw * st->E, phi);
                    const double d_sigma = -d_raw * st->raw, m_sigma = m_raw * st->raw;
                    const double a = conics[g * 3], b = conics[g * 3 + 1], c = conics[g * 3 + 2];
                    const double dx = st->dx, dy = st->dy;
                    const double mean_x = d_sigma * (a * dx + b * dy), mean_y = d_sigma * (c * dy + b * dx);
                    orc_acc(g_means, abs_means, err_means, g * 2, mean_x, m_sigma * (fabs(a * dx) + fabs(b * dy)), phi);
                    orc_acc(g_means, abs_means, err_means, g * 2 + 1, mean_y,
                            m_sigma * (fabs(c * dy) + fabs(b * dx)), phi);
                    if (g_means_abs) {
                        g_means_abs[g * 2] += fabs(mean_x);
                        g_means_abs[g * 2 + 1] += fabs(mean_y);
                    }
                    orc_acc(g_conics, abs_conics, err_conics, g * 3, d_sigma * 0.5 * dx * dx, m_sigma * 0.5 * dx * dx,
                            phi);
                    orc_acc(g_conics, abs_conics, err_conics, g * 3 + 1, d_sigma * dx * dy, m_sigma * fabs(dx * dy),
                            phi);
                    orc_acc(g_conics, abs_conics, err_conics, g * 3 + 2, d_sigma * 0.5 * dy * dy,
                            m_sigma * 0.5 * dy * dy, phi);
                    /* splat j now lies behind the splats in front of it */
                    for (int k = 0; k < K; ++k) {
                        S[k] += col[k] * w;
                        S_abs[k] += fabs(col[k]) * w;
                    }
                }
            }
        }
    }
    free(steps);
    return 0;
}

/* 3x3 product left * right, each entry summed from 0 over the inner index in order ([gsplat-proj] gs_mat3_product). */
static void orc_mat3_product(const float *left, const float *right, float *out)
{
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) {
            float v = 0.0f;
            for (int k = 0; k < 3; ++k) v += left[r * 3 + k] * right[k * 3 + c];
            out[r * 3 + c] = v;
        }
}

/* ceil of a float as int32, clamped to [0, 2^31 - 1] first (NaN -> 0) so that the conversion is defined; equal to
 * (int32_t)ceilf(v) for every v in range. */
static int32_t orc_ceil_radius(float v)
{
    float c = ceilf(v);
    if (!(c > 0.0f)) return 0;
    if (c >= 2147483648.0f) return 2147483647;
    return (int32_t)c;
}

/* EWA projection of N 3D Gaussians into C cameras ([gsplat-proj] gs_project_one), per (camera c, Gaussian g):
 *   R = the view's upper-left 3x3, t its last column; mean_c = R mean + t (each row summed left to right, then t);
 *   cov_c = (R cov) R^T (orc_mat3_product twice); depth = mean_c.z;
 *   z = depth unless depth <= near or >= far (then 1);
 *   perspective: the camera-space x/z and y/z are clipped to the image widened by 15% on each side, and
 *     J = [[fx / z, 0, -fx x_clipped / z^2], [0, fy / z, -fy y_clipped / z^2]], with x_clipped = clip(x / z) z;
 *     mean2d = ((K00 x + K01 y + K02 z) / z, (K10 x + K11 y + K12 z) / z);
 *   orthographic: J = [[fx, 0, 0], [0, fy, 0]], mean2d = (x fx + cx, y fy + cy);
 *   cov2d = J cov_c J^T (each entry summed over (left, right) in order from 0), det0 = its determinant;
 *   eps2d is added to the diagonal, det = the new determinant, safe = det <= 0 ? 1e-10 : det;
 *   r = ceil(3.33 sqrt(max(diagonal, 0))) per axis; visible iff det > 0, near < depth < far, some r > radius_clip
 *   and the box mean2d +- r overlaps the image; radii = visible ? r : 0;
 *   conic = (cov2d_11 / safe, -(cov2d_01 + cov2d_10) / (2 safe), cov2d_00 / safe);
 *   compensation (nullable) = sqrt(max(det0 / safe, 0)).
 * Float32 in the page's operation order. Outputs: radii [C, N, 2] int32, means2d [C, N, 2], depths [C, N],
 * conics [C, N, 3]. */
void orc_project(const float *means, const float *covars, const float *views, const float *Ks, int64_t C,
                 int64_t N, int width, int height, float eps2d, float near_plane, float far_plane, float radius_clip,
                 int orthographic, int32_t *radii, float *means2d, float *depths, float *conics, float *comps)
{
    for (int64_t c = 0; c < C; ++c) {
        const float *view = views + c * 16;
        const float *K = Ks + c * 9;
        float R[9] = {view[0], view[1], view[2], view[4], view[5], view[6], view[8], view[9], view[10]};
        float Rt[9];
        for (int r = 0; r < 3; ++r)
            for (int q = 0; q < 3; ++q) Rt[r * 3 + q] = R[q * 3 + r];
        for (int64_t g = 0; g < N; ++g) {
            const float *m = means + g * 3;
            const float *cov = covars + g * 9;
            float mc[3];
            for (int r = 0; r < 3; ++r) mc[r] = R[r * 3] * m[0] + R[r * 3 + 1] * m[1] + R[r * 3 + 2] * m[2] + view[r * 4 + 3];
            float tmp[9], cc[9];
            orc_mat3_product(R, cov, tmp);
            orc_mat3_product(tmp, Rt, cc);
            float depth = mc[2];
            float z = (depth <= near_plane || depth >= far_plane) ? 1.0f : depth;
            float J[6] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            float p0, p1;
            if (orthographic) {
                J[0] = K[0];
                J[4] = K[4];
                p0 = mc[0] * K[0] + K[2];
                p1 = mc[1] * K[4] + K[5];
            } else {
                float w = (float)width, h = (float)height;
                float min_x = -(K[2] / K[0] + 0.15f * w / K[0]);
                float max_x = (w - K[2]) / K[0] + 0.15f * w / K[0];
                float min_y = -(K[5] / K[4] + 0.15f * h / K[4]);
                float max_y = (h - K[5]) / K[4] + 0.15f * h / K[4];
                float cx = fminf(fmaxf(mc[0] / z, min_x), max_x) * z;
                float cy = fminf(fmaxf(mc[1] / z, min_y), max_y) * z;
                J[0] = K[0] / z;
                J[2] = -K[0] * cx / (z * z);
                J[4] = K[4] / z;
                J[5] = -K[4] * cy / (z * z);
                p0 = (K[0] * mc[0] + K[1] * mc[1] + K[2] * z) / z;
                p1 = (K[3] * mc[0] + K[4] * mc[1] + K[5] * z) / z;
            }
            float c2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int r = 0; r < 2; ++r)
                for (int q = 0; q < 2; ++q)
                    for (int a = 0; a < 3; ++a)
                        for (int b = 0; b < 3; ++b) c2[r * 2 + q] += J[r * 3 + a] * cc[a * 3 + b] * J[q * 3 + b];
            float det0 = c2[0] * c2[3] - c2[1] * c2[2];
            c2[0] += eps2d;
            c2[3] += eps2d;
            float det = c2[0] * c2[3] - c2[1] * c2[2];
            float safe = det <= 0.0f ? 1e-10f : det;
            int32_t rx = orc_ceil_radius(3.33f * sqrtf(fmaxf(c2[0], 0.0f)));
            int32_t ry = orc_ceil_radius(3.33f * sqrtf(fmaxf(c2[3], 0.0f)));
            int visible = det > 0.0f && depth > near_plane && depth < far_plane &&
                          ((float)rx > radius_clip || (float)ry > radius_clip) && p0 + (float)rx > 0.0f &&
                          p0 - (float)rx < (float)width && p1 + (float)ry > 0.0f && p1 - (float)ry < (float)height;
            int64_t i = c * N + g;
            radii[i * 2] = visible ? rx : 0;
            radii[i * 2 + 1] = visible ? ry : 0;
            means2d[i * 2] = p0;
            means2d[i * 2 + 1] = p1;
            depths[i] = depth;
            conics[i * 3] = c2[3] / safe;
            conics[i * 3 + 1] = -(c2[1] + c2[2]) / (2.0f * safe);
            conics[i * 3 + 2] = c2[0] / safe;
            if (comps) comps[i] = sqrtf(fmaxf(det0 / safe, 0.0f));
        }
    }
}

/* Tile rectangles [x0, y0, x1, y1] of every (camera, splat), for vectorised membership checks. */
void orc_rects(const float *means2d, const float *radii, int radii_per_gauss, int64_t M, int tile_size,
               int tile_width, int tile_height, int32_t *rects)
{
    for (int64_t i = 0; i < M; ++i)
        orc_bounds_of(means2d, radii, radii_per_gauss, i, tile_size, tile_width, tile_height, rects + 4 * i);
}

/* Per-tile lists straight from the definition, for sampled checks at sizes where a full sort is too slow:
 * for each requested global tile, every (camera, splat) whose rectangle contains it, ordered by
 * (depth bit pattern, flat id). Call once with out_ids == NULL to fill out_counts[n_tiles] and get the total,
 * then again with out_ids sized to that total (tile by tile, in the order of `tiles`). */
int64_t orc_tile_lists(const float *means2d, const float *radii, int radii_per_gauss, const float *depths,
                       int64_t C, int64_t N, int tile_size, int tile_width, int tile_height, const int64_t *tiles,
                       int64_t n_tiles, int64_t *out_counts, int32_t *out_ids)
{
    int64_t per_camera = (int64_t)tile_width * tile_height;
    int64_t *cursor = (int64_t *)calloc((size_t)(n_tiles > 0 ? n_tiles : 1), sizeof(int64_t));
    if (!cursor) return -1;
    if (out_ids) {
        int64_t running = 0;
        for (int64_t j = 0; j < n_tiles; ++j) {
            cursor[j] = running;
            running += out_counts[j];
        }
    } else {
        for (int64_t j = 0; j < n_tiles; ++j) out_counts[j] = 0;
    }
    for (int64_t index = 0; index < C * N; ++index) {
        int64_t camera = index / N;
        int32_t b[4];
        orc_bounds_of(means2d, radii, radii_per_gauss, index, tile_size, tile_width, tile_height, b);
        if (b[0] == b[2] || b[1] == b[3]) continue;
        for (int64_t j = 0; j < n_tiles; ++j) {
            int64_t t = tiles[j];
            if (t / per_camera != camera) continue;
            int64_t local = t % per_camera;
            int ty = (int)(local / tile_width), tx = (int)(local % tile_width);
            if (tx >= b[0] && tx < b[2] && ty >= b[1] && ty < b[3]) {
                if (out_ids) out_ids[cursor[j]++] = (int32_t)index;
                else out_counts[j] += 1;
            }
        }
    }
    int64_t total = 0;
    for (int64_t j = 0; j < n_tiles; ++j) {
        int64_t start = total;
        total += out_counts[j];
        if (!out_ids) continue;
        /* insertion sort of this tile's ids by (depth bits, id); ids arrive ascending, so equal depths keep
         * ascending id */
        for (int64_t i = start + 1; i < total; ++i) {
            int32_t v = out_ids[i];
            uint32_t dv;
            memcpy(&dv, &depths[v], sizeof dv);
            int64_t p = i;
            while (p > start) {
                uint32_t du;
                memcpy(&du, &depths[out_ids[p - 1]], sizeof du);
                if (du <= dv) break;
                out_ids[p] = out_ids[p - 1];
                --p;
            }
            out_ids[p] = v;
        }
    }
    free(cursor);
    return total;
}

/* Fixed-capacity per-tile bins, the alternative to sort-based binning (the bin list layout of [pytorch3d-fine]
 * RasterizeMeshesFineCudaKernel: bins [C, th, tw, capacity] int32 with -1 marking empty slots; the step that fills
 * them is not on the page). Definition used here: bin t holds the (camera, splat) flat ids whose rectangle
 * ([gsplat] gs_bounds) contains tile t, ordered by (depth bit pattern, flat id) - the order of the sorted
 * intersection list - the first min(count, capacity) of them, then -1 in every remaining slot; bin_counts[t] is
 * the full count (greater than capacity when the bin overflowed). Returns the largest count, or -1 on a bad
 * argument or allocation failure. */
int64_t orc_bin_tiles(const float *means2d, const float *radii, int radii_per_gauss, const float *depths,
                      int64_t C, int64_t N, int tile_size, int tile_width, int tile_height, int64_t capacity,
                      int32_t *bin_ids, int32_t *bin_counts)
{
    int64_t per_camera = (int64_t)tile_width * tile_height;
    int64_t total_tiles = C * per_camera;
    if (capacity < 1 || C < 1 || N < 0) return -1;
    int64_t *count = (int64_t *)calloc((size_t)total_tiles + 1, sizeof(int64_t));
    if (!count) return -1;
    /* pass 1: every (camera, splat) rectangle, counted per tile */
    for (int64_t index = 0; index < C * N; ++index) {
        int64_t camera = index / N;
        int32_t b[4];
        orc_bounds_of(means2d, radii, radii_per_gauss, index, tile_size, tile_width, tile_height, b);
        for (int ty = b[1]; ty < b[3]; ++ty)
            for (int tx = b[0]; tx < b[2]; ++tx) count[camera * per_camera + (int64_t)ty * tile_width + tx] += 1;
    }
    int64_t *start = (int64_t *)malloc(((size_t)total_tiles + 1) * sizeof(int64_t));
    if (!start) {
        free(count);
        return -1;
    }
    start[0] = 0;
    for (int64_t t = 0; t < total_tiles; ++t) start[t + 1] = start[t] + count[t];
    int32_t *all = (int32_t *)malloc(((size_t)start[total_tiles] + 1) * sizeof(int32_t));
    int64_t *cursor = (int64_t *)malloc(((size_t)total_tiles + 1) * sizeof(int64_t));
    if (!all || !cursor) {
        free(count);
        free(start);
        free(all);
        free(cursor);
        return -1;
    }
    memcpy(cursor, start, (size_t)total_tiles * sizeof(int64_t));
    /* pass 2: the same rectangles, ids appended per tile in ascending order */
    for (int64_t index = 0; index < C * N; ++index) {
        int64_t camera = index / N;
        int32_t b[4];
        orc_bounds_of(means2d, radii, radii_per_gauss, index, tile_size, tile_width, tile_height, b);
        for (int ty = b[1]; ty < b[3]; ++ty)
            for (int tx = b[0]; tx < b[2]; ++tx)
                all[cursor[camera * per_camera + (int64_t)ty * tile_width + tx]++] = (int32_t)index;
    }
    int64_t largest = 0;
    for (int64_t t = 0; t < total_tiles; ++t) {
        int32_t *list = all + start[t];
        int64_t n = count[t];
        /* stable insertion sort by depth bits: ids arrived ascending, so equal depths keep ascending id */
        for (int64_t i = 1; i < n; ++i) {
            int32_t v = list[i];
            uint32_t dv;
            memcpy(&dv, &depths[v], sizeof dv);
            int64_t p = i;
            while (p > 0) {
                uint32_t du;
                memcpy(&du, &depths[list[p - 1]], sizeof du);
                if (du <= dv) break;
                list[p] = list[p - 1];
                --p;
            }
            list[p] = v;
        }
        for (int64_t m = 0; m < capacity; ++m) bin_ids[t * capacity + m] = m < n ? list[m] : -1;
        bin_counts[t] = (int32_t)n;
        if (n > largest) largest = n;
    }
    free(count);
    free(start);
    free(all);
    free(cursor);
    return largest;
}

/* Compositing over fixed-capacity bins, following [pytorch3d-fine] RasterizeMeshesFineCudaKernel's walk: every
 * slot m in [0, capacity) of the pixel's bin in order, a negative entry (the -1 sentinel) skipped wherever it
 * stands; every other entry composited by the rule of orc_composite_pixel. last_ids holds the bin position
 * t * capacity + m of the last composited entry (-1 if none). Returns the number of sigma evaluations, or -1. */
int64_t orc_rasterize_bins(const float *means2d, const float *conics, const float *colors, const float *opacities,
                           const float *backgrounds, int64_t C, int K, int width, int height, int tile_size,
                           int tile_width, int tile_height, const int32_t *bin_ids, int64_t capacity,
                           float alpha_cutoff, float alpha_clamp, float transmittance_threshold,
                           float *render_colors, float *render_alphas, float *render_T, int32_t *last_ids)
{
    int64_t per_camera = (int64_t)tile_width * tile_height;
    int64_t total_tiles = C * per_camera;
    int64_t n_eval = 0;
    float acc[64];
    if (K < 1 || K > 64 || capacity < 1) return -1;
    int32_t *list = (int32_t *)malloc((size_t)capacity * sizeof(int32_t));
    int64_t *where = (int64_t *)malloc((size_t)capacity * sizeof(int64_t));
    if (!list || !where) {
        free(list);
        free(where);
        return -1;
    }
    for (int64_t t = 0; t < total_tiles; ++t) {
        int64_t camera = t / per_camera;
        int64_t local = t % per_camera;
        int ty = (int)(local / tile_width), tx = (int)(local % tile_width);
        /* the bin's entries with the sentinels taken out, and where each one stood */
        int64_t n = 0;
        for (int64_t m = 0; m < capacity; ++m) {
            int32_t g = bin_ids[t * capacity + m];
            if (g < 0) continue;
            list[n] = g;
            where[n] = t * capacity + m;
            ++n;
        }
        for (int y = ty * tile_size; y < (ty + 1) * tile_size && y < height; ++y) {
            for (int x = tx * tile_size; x < (tx + 1) * tile_size && x < width; ++x) {
                float T;
                int64_t last;
                orc_composite_pixel(means2d, conics, colors, opacities, K, list, 0, n, x, y, alpha_cutoff,
                                    alpha_clamp, transmittance_threshold, acc, &T, &last, &n_eval);
                int64_t pixel = (camera * height + y) * (int64_t)width + x;
                for (int k = 0; k < K; ++k) {
                    float bg = backgrounds ? backgrounds[camera * K + k] : 0.0f;
                    render_colors[pixel * K + k] = acc[k] + T * bg;
                }
                render_alphas[pixel] = 1.0f - T;
                if (render_T) render_T[pixel] = T;
                if (last_ids) last_ids[pixel] = last >= 0 ? (int32_t)where[last] : -1;
            }
        }
    }
    free(list);
    free(where);
    return n_eval;
}

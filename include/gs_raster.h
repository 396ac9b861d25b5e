/*
 * gs_raster.h: C ABI of the MI355X (gfx950) tile-binned splat rasterizer.
 *
 * A frame runs the first four entry points in order; the others extend it:
 *   gs_isect_tiles    splat -> tile intersections and their 64-bit keys (optionally sorted),
 *   gs_sort_keys      stable radix sort of (key, id) pairs over the populated low key bits,
 *   gs_tile_ranges    per-tile [start, end) ranges of a sorted key array,
 *   gs_rasterize_fwd  per-tile front-to-back alpha compositing (gs_rasterize_fwd_traced: with a per-pixel
 *                     trace, a per-pixel step cap and a per-tile list cap),
 *   gs_rasterize_bwd  its backward,
 *   gs_project_fwd    the EWA projection of 3D Gaussians that feeds the intersection step,
 *   gs_bin_tiles      fixed-capacity per-tile bins (the alternative to the first three steps), composited by
 *                     gs_rasterize_fwd_bins.
 *
 * Definitions follow these pages:
 *   [gsplat]     gsplat 1.0.0 Ruby gem, native C extension, intersections.c (gs_tile_bits, gs_bounds,
 *                gs_radix_sort_without_gvl, gs_isect_tiles, gs_offset_encode);
 *   [gsplat-bwd] the same gem's raster_backward.c (gs_raster_backward_pixel, gs_raster_backward_without_gvl),
 *                whose per-splat terms fix what the forward computes, and raster_backward_bridge.c
 *                (gs_raster_backward), which lists the forward's arguments;
 *   [rlx-metal]  rlx-metal 0.2.9 splat_training.rs (training_forward_metal_traced): alpha_cutoff and
 *                transmittance_threshold as forward parameters;
 *   [gsplat-proj] the gem's projection.c (gs_project_one): the projection of 3D Gaussians into cameras;
 *   [pytorch3d-fine] PyTorch3D rasterize_meshes.cu (RasterizeMeshesFineCudaKernel): the -1-sentinel bin layout.
 *
 * Conventions for every entry point.
 *   - Device pointers point to memory on the current HIP device; every array is dense and C-ordered.
 *     The caller allocates and owns every buffer, workspace included; the library never allocates or frees
 *     device memory. State kept between calls: a thread-local error message, the sort's process-wide spin limit
 *     and one 4-byte device error word per GPU (gs_set_spin_limit, gs_device_check).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Calls are asynchronous on it unless
 *     stated otherwise; inputs must stay valid until the stream has run the work.
 *   - On any error nothing is launched (argument checks run on the host first), the return value says why,
 *     and gs_last_error() describes it. GS_ERR_DEVICE means a HIP runtime call or launch failed.
 *   - Keys are 64-bit unsigned; callers holding them in int64 storage (as the pages do) pass the same bits.
 *   - Floating-point results are float32 with a fixed operation order (no contraction), so the same inputs
 *     give the same bits on every run.
 */
#ifndef GS_RASTER_H
#define GS_RASTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gs_status {
    GS_OK = 0,
    GS_ERR_INVALID_ARG = 1, /* bad shape, size, pointer or option ([gsplat] raises ArgError for these) */
    GS_ERR_OUT_OF_GRID = 2, /* a key decodes outside the tile grid ([gsplat] gs_offset_encode) */
    GS_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than the matching *_workspace_bytes() */
    GS_ERR_DEVICE = 4       /* a HIP runtime call or kernel launch failed */
} gs_status;

/* Message for the last non-OK status returned on this thread ("" if none). Valid until the next call. */
const char *gs_last_error(void);

/* ------------------------------------------------------------------------------------------------------------
 * Intersections ([gsplat] gs_isect_tiles, with gs_bounds and gs_tile_bits).
 *
 * For every camera c < C and splat g < N (flat index i = c*N + g) the tile rectangle is
 *   x0 = clamp(floor((mx - rx) / ts), 0, tw)    x1 = clamp(ceil((mx + rx) / ts), 0, tw)
 *   y0 = clamp(floor((my - ry) / ts), 0, th)    y1 = clamp(ceil((my + ry) / ts), 0, th)
 * in float32 with IEEE division (empty when rx <= 0 or ry <= 0, or when an input is NaN), its tile count is
 * (x1 - x0) * (y1 - y0), and each covered tile (ty, tx) yields one intersection
 *   key = ((c << tile_bits) | (ty * tw + tx)) << 32 | bits(depth[i]),   id = i,
 * with tile_bits = ceil(log2(tw * th)) (0 for one tile). Unsorted output is in (c, g, ty, tx) order; sorted
 * output is the stable ascending order by key, i.e. by (camera, tile, depth bits, id).
 *
 * Two phases, because the output size depends on the data:
 *   1. keys == NULL: count. Writes tiles_per_gauss[C*N] (int32), gauss_offsets[C*N] (int32 exclusive prefix
 *      of the counts, the first output slot of each splat) and *n_isects_out (host memory), then SYNCHRONISES
 *      the stream to return the count. n_isects is ignored.
 *   2. keys != NULL: emit. Needs gauss_offsets from phase 1 unchanged and n_isects = phase 1's count; writes
 *      keys[n_isects] and flatten_ids[n_isects]; when sort != 0 and n_isects > 1 also sorts them (as
 *      gs_sort_keys with end_bit = 32 + tile_bits + camera_bits). Asynchronous. tiles_per_gauss and
 *      n_isects_out are ignored.
 *
 * means2d     [C, N, 2] float32 (pixel coordinates)
 * radii       [C, N] float32 if radii_per_gauss == 1 (isotropic), [C, N, 2] if 2 (x and y extents)
 * depths      [C, N] float32; only the bit pattern is used (it forms the key's low 32 bits)
 * tile_size   > 0 pixels; tile_width, tile_height > 0 tiles (any grid; not tied to an image size here)
 * Limits (GS_ERR_INVALID_ARG): C >= 1, N >= 0, C*N < 2^31, tile_width*tile_height < 2^31,
 *   tile_bits + camera_bits <= 32 (camera_bits = ceil(log2 C)), total intersections < 2^31 (phase 1 returns
 *   the error and still writes *n_isects_out), and with sort != 0 at most 2^30 - 1 splats and intersections.
 * workspace: gs_isect_workspace_bytes(C, N, n, tile_width, tile_height, sort) bytes; n = 0 sizes phase 1.
 *   With sort != 0, phase 1 also puts the splats in (depth bits, id) order and computes each one's first output
 *   slot in that order, into the first gs_isect_workspace_bytes(C, N, 0, tile_width, tile_height, 1) bytes of
 *   the workspace. When n_isects_out is page-locked host memory (hipHostMalloc, or a pinned torch tensor) the
 *   count kernel writes the total there itself and the host waits for that word alone, so this work, queued
 *   behind the count, runs while the host returns; with pageable memory a copy call waits for the count first.
 *   Phase 2 must then receive a workspace that starts with those bytes unchanged: the same buffer (sized for
 *   phase 2 from the start), or a larger one into which the caller copied them on the same stream. A workspace
 *   without them gives a wrong order (never an access outside the buffers). Phase 2 accumulates the tile sort's
 *   digit counts in those bytes and zeroes them again as it reads them, so they serve a later phase 2 too.
 */
size_t gs_isect_workspace_bytes(int64_t C, int64_t N, int64_t n_isects, int tile_width, int tile_height, int sort);

gs_status gs_isect_tiles(const float *means2d, const float *radii, int radii_per_gauss, const float *depths,
                         int64_t C, int64_t N, int tile_size, int tile_width, int tile_height, int sort,
                         int32_t *tiles_per_gauss, int32_t *gauss_offsets, int64_t *n_isects_out,
                         uint64_t *keys, int32_t *flatten_ids, int64_t n_isects,
                         void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * Stable sort ([gsplat] gs_radix_sort_without_gvl: a stable LSD radix sort of (key, id) pairs).
 *
 * Reorders keys[n] and flatten_ids[n] in place into ascending order of (key mod 2^end_bit); equal values keep
 * their input order, so the result is unique. Bits at and above end_bit take no part and travel with their
 * key (for intersection keys they are zero). 0 <= end_bit <= 64; n <= 2^30 - 1. Passes of at most 8 bits
 * cover [0, end_bit); the workspace holds the alternate buffers and the per-pass counters.
 */
size_t gs_sort_workspace_bytes(int64_t n, int end_bit);

gs_status gs_sort_keys(uint64_t *keys, int32_t *flatten_ids, int64_t n, int end_bit, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * gs_sort_keys without a workspace, for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * The same stable sort as gs_sort_keys (same arguments and result), with its alternate buffers, digit histograms and
 * look-back words in a file-scope device array of the library (about 52 MB per GPU, held until the process ends)
 * instead of a caller workspace. n is limited to 2^22 pairs (GS_ERR_INVALID_ARG above that, before any launch). The
 * call allocates nothing. Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and give wrong orders; serialize them. Errors as gs_sort_keys.
 */
gs_status gs_sort_keys_static(uint64_t *keys, int32_t *flatten_ids, int64_t n, int end_bit, void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * Device-side failure of the sort and the count scans ([gsplat] gs_isect_tiles turns a failure of its sort into
 * an error status, NoMemError; here the only device-side failure is a wait that does not end).
 *
 * Each digit pass of the sort (gs_sort_keys, and gs_isect_tiles with sort != 0, whose last depth pass also scans
 * the counts in depth order) and the scan of the counts in splat order in gs_isect_tiles' phase 1 let a partition
 * wait for the counts of the partitions before it. The wait is bounded: after `limit` rounds (one round is one
 * device-coherent load plus a short sleep; the default, 2^20, is about a second) the partition gives up, sets the
 * library's device error word of the current GPU and finishes, so the kernel always completes; that call's output
 * is then invalid (every access still stays inside the caller's buffers).
 * gs_set_spin_limit: sets the limit used by passes launched after the call (process-wide) and returns the
 *   previous one. 0 makes every partition that does not find its predecessors' counts at the first look give up
 *   (for testing the failure path).
 * gs_device_check: SYNCHRONISES `stream`, then reads and clears the device error word of the current GPU;
 *   GS_ERR_DEVICE if a wait gave up since the last check (on any stream of that GPU), GS_OK otherwise.
 */
uint32_t gs_set_spin_limit(uint32_t limit);

gs_status gs_device_check(void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * Tile ranges ([gsplat] gs_offset_encode for the output, [gsplat-bwd] gs_raster_backward_without_gvl for how
 * a range is read).
 *
 * For keys sorted by their upper 32 bits, writes isect_offsets[C, th, tw] (int32): entry t is the number of
 * keys whose global tile camera * (tw * th) + (upper & (2^tile_bits - 1)) is below t, with
 * upper = key >> 32 and camera = upper >> tile_bits. Tile t's intersections are then
 * [offsets[t], t + 1 < C*th*tw ? offsets[t + 1] : n). Computed by boundary detection over the sorted keys.
 * validate != 0: also checks every key decodes inside the grid (camera < C, tile < tw * th) and that the
 *   keys' global tiles do not decrease, then SYNCHRONISES; returns GS_ERR_OUT_OF_GRID or GS_ERR_INVALID_ARG
 *   (unsorted) if not. validate == 0 trusts the input (writes stay in bounds either way) and is asynchronous.
 * n may be 0 (all offsets 0). workspace: gs_tile_ranges_workspace_bytes() bytes (an error flag).
 */
size_t gs_tile_ranges_workspace_bytes(void);

gs_status gs_tile_ranges(const uint64_t *sorted_keys, int64_t n, int64_t C, int tile_width, int tile_height,
                         int32_t *isect_offsets, int validate, void *workspace, size_t workspace_bytes,
                         void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * Forward compositing (the front-to-back inverse of [gsplat-bwd] gs_raster_backward_pixel, with the
 * [rlx-metal] alpha_cutoff and transmittance_threshold).
 *
 * For each camera c, tile t = (c * th + ty) * tw + tx and pixel (x, y) of the tile inside width x height,
 * walking i over [offsets[t], end of t) with g = flatten_ids[i], starting from T = 1, colour 0, last = -1:
 *   dx = means2d[g].x - (x + 0.5),  dy = means2d[g].y - (y + 0.5),
 *   sigma = 0.5 * (a dx dx + c dy dy) + b dx dy  with (a, b, c) = conics[g], each operation rounded to float;
 *   skip if sigma < 0;  alpha = min(alpha_clamp, opacities[g] * E(sigma));  skip if alpha < alpha_cutoff;
 *   T' = T * (1 - alpha); stop before this splat if T' <= transmittance_threshold;
 *   colour += colors[g] * (alpha * T); T = T'; last = i.
 * E(sigma) is e^-sigma computed as: 0 if sigma > 80 or NaN, else k = rint(-sigma * log2 e),
 * r = fma(-k, ln2_hi, -sigma), r = fma(-k, ln2_lo, r), a degree-7 Taylor polynomial of e^r by fma (Horner),
 * times 2^k (Cody and Waite's reduction) - the same bits on any IEEE float32 machine.
 * Outputs per pixel: render_colors [C, H, W, K] = colour + T * backgrounds[c] (backgrounds [C, K], NULL = 0),
 * render_alphas [C, H, W] = 1 - T, render_T [C, H, W] = T (nullable), last_ids [C, H, W] = last (nullable;
 * a global intersection index, -1 if nothing composited).
 * conics [C, N, 3] = (inv00, inv01, inv11) of the 2D covariance; colors [C, N, K]; opacities [C, N].
 * masks: nullable [C, th, tw] int32 per-tile mask; a tile whose mask is 0 composites nothing (its pixels get the
 *   background, render_alphas 0, T 1 and last id -1) - the backward page skips such tiles' splats.
 * eval_counts: nullable device uint64[5]; when set, the launch ADDS work counts: [0] the evaluations of sigma the
 * definition makes (per pixel, each splat of its range up to and including the one that stops it), [1] those
 * with alpha >= alpha_cutoff, [2] the splats composited, [3] the evaluations the kernel actually made (it skips
 * splats a conservative bound proves to stay below the cutoff over a wave's pixels, which cannot change any
 * output), [4] the splats staged per tile. The counting variant is a separate kernel build; with NULL nothing is
 * counted.
 * Limits: 1 <= K <= 4; 1 <= tile_size <= 32; tile_width == ceil(width / tile_size) and
 *   tile_height == ceil(height / tile_size). An entry of flatten_ids outside [0, C*N) is skipped (never read
 *   through; the -1 of an empty bin slot is one), so malformed ids cannot make the kernels address outside their
 *   inputs. gs_rasterize_bwd skips such entries the same way.
 * workspace: gs_rasterize_workspace_bytes(C, tile_width, tile_height) bytes, or NULL with 0 bytes. Reserved: the
 *   size is checked when one is given, but the current kernels neither read nor write it.
 */
size_t gs_rasterize_workspace_bytes(int64_t C, int tile_width, int tile_height);

gs_status gs_rasterize_fwd(const float *means2d, const float *conics, const float *colors, const float *opacities,
                           const float *backgrounds, int64_t C, int64_t N, int K, int width, int height,
                           int tile_size, int tile_width, int tile_height, const int32_t *isect_offsets,
                           const int32_t *flatten_ids, int64_t n_isects, const int32_t *masks,
                           float alpha_cutoff, float alpha_clamp,
                           float transmittance_threshold, float *render_colors, float *render_alphas,
                           float *render_T, int32_t *last_ids, uint64_t *eval_counts, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * gs_rasterize_fwd_hwexp: gs_rasterize_fwd with e^-sigma taken from the hardware base-2 exponential
 * (v_exp_f32 of -sigma log2 e, about one ulp; 0 for sigma > 80 or NaN) instead of the specified E(sigma). Faster,
 * and not bit-identical: an alpha within about an ulp of alpha_cutoff or alpha_clamp, or a transmittance product
 * within rounding of transmittance_threshold, can fall on the other side, which moves that pixel by up to about
 * alpha * T (reported separately from the specified mode; the backward always recomputes with E(sigma)).
 * Same arguments, outputs, limits and errors as gs_rasterize_fwd, without the workspace.
 */
gs_status gs_rasterize_fwd_hwexp(const float *means2d, const float *conics, const float *colors,
                                 const float *opacities, const float *backgrounds, int64_t C, int64_t N, int K,
                                 int width, int height, int tile_size, int tile_width, int tile_height,
                                 const int32_t *isect_offsets, const int32_t *flatten_ids, int64_t n_isects,
                                 const int32_t *masks, float alpha_cutoff, float alpha_clamp,
                                 float transmittance_threshold, float *render_colors, float *render_alphas,
                                 float *render_T, int32_t *last_ids, uint64_t *eval_counts, void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * Traced forward compositing ([rlx-metal] training_forward_metal_traced: max_splat_steps, the per-pixel trace of
 * counts and ids kept for the backward, and the tile-list cap max_list_entries). Everything gs_rasterize_fwd
 * computes, with:
 *   max_list_entries >= 0: each tile's range is cut to its first max_list_entries entries (the nearest ones)
 *     before compositing; a negative value keeps whole ranges;
 *   max_splat_steps >= 0: a step is a composited splat; a pixel stops right after its max_splat_steps-th step
 *     (at once when 0), so render_colors, render_alphas, render_T and last_ids describe exactly the traced splats;
 *   trace_ids: nullable [C, H, W, max_splat_steps] int32 - each pixel's composited flat splat ids (camera * N +
 *     Gaussian, the values of flatten_ids) in front-to-back order; entries past the pixel's count are left
 *     unwritten;
 *   trace_counts: nullable [C, H, W] int32 - the pixel's number of steps (<= max_splat_steps).
 * A pixel's trace holds every splat that changed it and nothing else: compositing the pixel over its trace alone
 * gives the same bits. The range backward (gs_rasterize_bwd) on these outputs is the gradient of the capped forward,
 * since it walks each pixel back from last_ids and recomputes which splats composited.
 * eval_counts' first entry counts evaluations up to and including the splat that stops the pixel, by the cap too.
 * Errors: as gs_rasterize_fwd, plus GS_ERR_INVALID_ARG for max_splat_steps < 0.
 */
gs_status gs_rasterize_fwd_traced(const float *means2d, const float *conics, const float *colors,
                                  const float *opacities, const float *backgrounds, int64_t C, int64_t N, int K,
                                  int width, int height, int tile_size, int tile_width, int tile_height,
                                  const int32_t *isect_offsets, const int32_t *flatten_ids, int64_t n_isects,
                                  const int32_t *masks, float alpha_cutoff, float alpha_clamp,
                                  float transmittance_threshold, int max_list_entries, int max_splat_steps,
                                  float *render_colors, float *render_alphas, float *render_T, int32_t *last_ids,
                                  int32_t *trace_ids, int32_t *trace_counts, uint64_t *eval_counts, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * Fixed-capacity per-tile bins, an alternative to sort-based binning ([pytorch3d-fine] PyTorch3D
 * rasterize_meshes.cu, RasterizeMeshesFineCudaKernel, reads bins [N, BH, BW, M] int32 with -1 in empty slots;
 * the step that fills them is not on the page).
 *
 * gs_bin_tiles: for each global tile t = (c * th + ty) * tw + tx, bin_counts[t] (int32 [C, th, tw]) receives the
 * number of (camera, splat) pairs whose rectangle ([gsplat] gs_bounds, as in gs_isect_tiles) contains the tile, and
 * bin_ids[t] (int32 [C, th, tw, capacity]) their flat ids camera * N + splat ordered by (depth bit pattern, flat
 * id) - the tile's list of the sorted intersection path - in slots [0, min(count, capacity)), then -1.
 * When a bin overflows (count > capacity) it keeps `capacity` of its splats, in that order; which ones is not
 * specified (they are claimed concurrently), and the caller detects it from bin_counts.
 * Limits: 1 <= capacity <= 16384; C * th * tw * capacity < 2^31; C*N < 2^31; radii as in gs_isect_tiles.
 * Asynchronous; needs no workspace.
 *
 * gs_rasterize_fwd_bins: gs_rasterize_fwd over such bins: tile t composites slots [0, min(bin_counts[t],
 * capacity)) of its bin in order, skipping negative entries (the sentinel); last_ids holds bin positions
 * t * capacity + m. Same outputs, limits and errors as gs_rasterize_fwd otherwise (no masks, no workspace).
 */
gs_status gs_bin_tiles(const float *means2d, const float *radii, int radii_per_gauss, const float *depths, int64_t C,
                       int64_t N, int tile_size, int tile_width, int tile_height, int capacity, int32_t *bin_ids,
                       int32_t *bin_counts, void *stream);

gs_status gs_rasterize_fwd_bins(const float *means2d, const float *conics, const float *colors,
                                const float *opacities, const float *backgrounds, int64_t C, int64_t N, int K,
                                int width, int height, int tile_size, int tile_width, int tile_height,
                                const int32_t *bin_ids, const int32_t *bin_counts, int capacity, float alpha_cutoff,
                                float alpha_clamp, float transmittance_threshold, float *render_colors,
                                float *render_alphas, float *render_T, int32_t *last_ids, uint64_t *eval_counts,
                                void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * EWA projection of 3D Gaussians ([gsplat-proj] gsplat 1.0.0 projection.c: gs_project_one, gs_mat3_product,
 * gs_camera_covar, gs_clip) - the step that produces the intersection step's inputs.
 *
 * For camera c (world-to-camera viewmats [C, 4, 4], intrinsics Ks [C, 3, 3]) and Gaussian g (means [N, 3],
 * covariances covars [N, 3, 3]): R = the view's upper 3x3, t its last column; mean_c = R mean + t;
 * cov_c = (R cov) R^T; depth = mean_c.z; z = depth unless depth <= near_plane or >= far_plane (then 1).
 * Perspective: x/z and y/z clipped to the image widened by 15% per side, J = [[fx/z, 0, -fx x_c/z^2],
 * [0, fy/z, -fy y_c/z^2]], mean2d = ((K00 x + K01 y + K02 z)/z, (K10 x + K11 y + K12 z)/z); orthographic:
 * J = [[fx, 0, 0], [0, fy, 0]], mean2d = (x fx + cx, y fy + cy). cov2d = J cov_c J^T; det0 its determinant;
 * eps2d added to the diagonal; det; safe = det <= 0 ? 1e-10 : det; r = ceil(3.33 sqrt(max(diag, 0))) per
 * axis (as int32, clamped to [0, 2^31 - 1]); visible iff det > 0, near < depth < far, some r > radius_clip and
 * mean2d +- r overlaps the image.
 * Outputs ([C, N, ...], C order): radii [C, N, 2] int32 (0 when not visible), means2d [C, N, 2], depths [C, N],
 * conics [C, N, 3] = (c11, -(c01 + c10)/2, c00) / safe, compensations [C, N] (nullable) = sqrt(max(det0 / safe,
 * 0)). Float32 in the page's operation order (no contraction): the same bits as a plain C evaluation.
 * Limits: 1 <= C <= 65535, C*N < 2^31. Asynchronous.
 */
gs_status gs_project_fwd(const float *means, const float *covars, const float *viewmats, const float *Ks, int64_t C,
                         int64_t N, int width, int height, float eps2d, float near_plane, float far_plane,
                         float radius_clip, int orthographic, int32_t *radii, float *means2d, float *depths,
                         float *conics, float *compensations, void *stream);

/* ------------------------------------------------------------------------------------------------------------
 * Backward of the composite ([gsplat-bwd] gs_raster_backward_pixel and gs_raster_backward_without_gvl).
 *
 * For L = sum(grad_render_colors * render_colors) + sum(grad_render_alphas * render_alphas) of the forward above
 * (same splats, ranges, cutoff and clamp; render_alphas and last_ids as the forward wrote them), writes the
 * gradients of means2d [C, N, 2], conics [C, N, 3], colors [C, N, K] and opacities [C, N], and of backgrounds
 * [C, K] when grad_backgrounds is not NULL (backgrounds may be NULL: a zero background). grad_means2d_abs
 * (nullable) receives per splat the sum of |d L / d mean| over its pixels, per axis.
 * Per pixel, T = 1 - render_alpha, after = 1 and rest = background; the background term is
 * grad_colour * T; then the tile's range is walked back to front and position i with splat g counts when
 * render_alpha > 0, sigma >= 0, alpha >= alpha_cutoff, i <= last_id, T < 1 and alpha < 1 (sigma, E(sigma),
 * raw = opacity * E and alpha = min(clamp, raw) exactly as in the forward). A counted splat adds, in float32:
 *   before = T / (1 - alpha), vis = before * alpha; colour: grad_colour[k] * vis;
 *   dot = sum_k grad_colour[k] * (colour[k] - rest[k]); g_alpha = before * (dot + grad_alpha * after);
 *   g_raw = raw < clamp ? g_alpha : 0; opacity: g_raw * E; g_sigma = -g_raw * raw;
 *   mean: g_sigma * (a dx + b dy), g_sigma * (c dy + b dx); conic: g_sigma * 0.5 * dx * dx, g_sigma * dx * dy,
 *   g_sigma * 0.5 * dy * dy;
 * then rest = alpha * colour + (1 - alpha) * rest, after *= 1 - alpha, T = before.
 * Every term is computed in that order; the terms of one splat are summed in an order the hardware picks (sums
 * over 16-lane rows, LDS atomics per tile, then one float atomic per splat and tile), so results agree with any
 * other summation order to within float rounding of the sum of the terms' magnitudes, and may differ in the last
 * bits from run to run.
 * masks: nullable [C, th, tw]; a tile whose mask is 0 adds only its pixels' background terms.
 * The gradient arrays are overwritten (cleared, then summed into). Limits as gs_rasterize_fwd. Asynchronous.
 */
gs_status gs_rasterize_bwd(const float *means2d, const float *conics, const float *colors, const float *opacities,
                           const float *backgrounds, int64_t C, int64_t N, int K, int width, int height,
                           int tile_size, int tile_width, int tile_height, const int32_t *isect_offsets,
                           const int32_t *flatten_ids, int64_t n_isects, const int32_t *masks,
                           float alpha_cutoff, float alpha_clamp,
                           const float *render_alphas, const int32_t *last_ids, const float *grad_render_colors,
                           const float *grad_render_alphas, float *grad_means2d, float *grad_conics,
                           float *grad_colors, float *grad_opacities, float *grad_backgrounds,
                           float *grad_means2d_abs, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GS_RASTER_H */

// Splat -> tile intersections on gfx950: a coalesced rectangle-and-count pass with a workgroup reduction, a
// device-wide exclusive prefix of the counts, and a load-balanced key emission in which every thread owns
// output slots (so the 8-byte key and 4-byte id stores are contiguous) and finds the splat that produced each
// slot by a search over the workgroup's offsets in LDS.
//
// Definitions: gsplat 1.0.0 native extension, intersections.c (gs_bounds, gs_tile_bits, gs_isect_tiles).
#include "gs_internal.hpp"

namespace gs {
namespace {

constexpr int kThreads = 256;

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

// Sum of one int64 per thread over a 256-thread workgroup (result valid in thread 0).
__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t *s_tmp) {
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_down(v, d, kWave);
    const int wave = threadIdx.x / kWave;
    if (__lane_id() == 0) s_tmp[wave] = v;
    __syncthreads();
    int64_t total = 0;
    if (threadIdx.x == 0)
        for (int w = 0; w < kThreads / kWave; ++w) total += s_tmp[w];
    return total;
}

// Exclusive prefix of one int64 per thread over a 256-thread workgroup; *total gets the sum (all threads).
__device__ __forceinline__ int64_t block_exclusive(int64_t v, int64_t *s_tmp, int64_t *total) {
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const int64_t inc = wave_inclusive_sum(v);
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        const int64_t t = s_tmp[w];
        if (w < wave) before += t;
        all += t;
    }
    *total = all;
    return before + inc - v;
}

// Phase 1a: per-splat tile count, and one partial sum per workgroup.
template <int RPG>
__global__ __launch_bounds__(kThreads) void count_kernel(const float2 *__restrict__ means,
                                                         const float *__restrict__ radii, int M, float ts, int tw,
                                                         int th, int32_t *__restrict__ tiles_per_gauss,
                                                         int64_t *__restrict__ block_sums) {
    __shared__ int64_t s_tmp[kThreads / kWave];
    const int i = blockIdx.x * kThreads + threadIdx.x;
    int64_t count = 0;
    if (i < M) {
        const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
        count = static_cast<int64_t>(r.x1 - r.x0) * static_cast<int64_t>(r.y1 - r.y0);
        if (tiles_per_gauss) tiles_per_gauss[i] = static_cast<int32_t>(count);
    }
    const int64_t total = block_sum(count, s_tmp);
    if (threadIdx.x == 0) block_sums[blockIdx.x] = total;
}

// Phase 1b: exclusive scan of the workgroup sums in place (one workgroup), total to *total_out.
__global__ __launch_bounds__(kThreads) void scan_block_sums_kernel(int64_t *__restrict__ sums, int count,
                                                                   int64_t *__restrict__ total_out) {
    __shared__ int64_t s_tmp[kThreads / kWave];
    int64_t carry = 0;
    for (int base = 0; base < count; base += kThreads) {
        const int i = base + threadIdx.x;
        const int64_t v = i < count ? sums[i] : 0;
        int64_t chunk = 0;
        const int64_t ex = block_exclusive(v, s_tmp, &chunk);
        if (i < count) sums[i] = carry + ex;
        carry += chunk;
        __syncthreads();
    }
    if (threadIdx.x == 0) *total_out = carry;
}

// Phase 1c: per-splat first output slot = workgroup prefix + exclusive scan of the counts within it.
template <int RPG>
__global__ __launch_bounds__(kThreads) void offsets_kernel(const float2 *__restrict__ means,
                                                           const float *__restrict__ radii, int M, float ts, int tw,
                                                           int th, const int64_t *__restrict__ block_prefix,
                                                           int32_t *__restrict__ gauss_offsets) {
    __shared__ int64_t s_tmp[kThreads / kWave];
    const int i = blockIdx.x * kThreads + threadIdx.x;
    int64_t count = 0;
    if (i < M) {
        const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
        count = static_cast<int64_t>(r.x1 - r.x0) * static_cast<int64_t>(r.y1 - r.y0);
    }
    int64_t unused;
    const int64_t ex = block_exclusive(count, s_tmp, &unused);
    if (i < M) gauss_offsets[i] = static_cast<int32_t>(block_prefix[blockIdx.x] + ex);
}

// Phase 2: the workgroup takes 256 consecutive splats; their outputs occupy the contiguous slots
// [start(g0), start(g0 + 256)). Each thread walks slots with stride 256, finds the owning splat (the last one
// whose start is <= slot) by binary search in LDS, and writes key and id for tile k of its rectangle in
// row-major order.
template <int RPG>
__global__ __launch_bounds__(kThreads) void emit_kernel(const float2 *__restrict__ means,
                                                        const float *__restrict__ radii,
                                                        const uint32_t *__restrict__ depth_bits, int M, int N,
                                                        float ts, int tw, int th, int tile_bits,
                                                        const int32_t *__restrict__ gauss_offsets, int n,
                                                        uint64_t *__restrict__ keys, int32_t *__restrict__ ids) {
    __shared__ int s_start[kThreads + 1];
    __shared__ int s_x0[kThreads], s_y0[kThreads], s_w[kThreads];
    __shared__ uint32_t s_upper_cam[kThreads], s_depth[kThreads];
    const int g0 = blockIdx.x * kThreads;
    const int i = g0 + threadIdx.x;
    if (i < M) {
        const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
        s_x0[threadIdx.x] = r.x0;
        s_y0[threadIdx.x] = r.y0;
        s_w[threadIdx.x] = r.x1 - r.x0;
        s_start[threadIdx.x] = gauss_offsets[i];
        s_depth[threadIdx.x] = depth_bits[i];
        s_upper_cam[threadIdx.x] = static_cast<uint32_t>(i / N) << tile_bits;
    } else {
        s_start[threadIdx.x] = n;
        s_w[threadIdx.x] = 1;
        s_x0[threadIdx.x] = s_y0[threadIdx.x] = 0;
        s_depth[threadIdx.x] = s_upper_cam[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) s_start[kThreads] = (g0 + kThreads < M) ? gauss_offsets[g0 + kThreads] : n;
    __syncthreads();
    // clamped to [0, n] so that offsets inconsistent with n can never address past the outputs
    const int out_end = min(s_start[kThreads], n);
    const int out_begin = min(s_start[0], out_end);
    for (int j = out_begin + static_cast<int>(threadIdx.x); j < out_end; j += kThreads) {
        int lo = 0, hi = kThreads - 1;  // invariant: s_start[lo] <= j, answer in [lo, hi]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_start[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        const int k = j - s_start[lo];
        const int w = s_w[lo];
        const int ry = k / w;
        const int rx = k - ry * w;
        const uint32_t tile = static_cast<uint32_t>(s_y0[lo] + ry) * static_cast<uint32_t>(tw) +
                              static_cast<uint32_t>(s_x0[lo] + rx);
        const uint64_t upper = static_cast<uint64_t>(s_upper_cam[lo] | tile);
        keys[j] = (upper << 32) | static_cast<uint64_t>(s_depth[lo]);
        ids[j] = g0 + lo;
    }
}

struct IsectLayout {
    size_t block_sums, total, sort, bytes;
};

IsectLayout isect_layout(int64_t M, int64_t n, int end_bit, int sort) {
    IsectLayout L{};
    Carver c(nullptr);
    const int64_t blocks = (M + kThreads - 1) / kThreads;
    c.take<int64_t>(static_cast<size_t>(blocks > 0 ? blocks : 1));
    L.block_sums = 0;
    L.total = align_up(c.used, 256);
    c.take<int64_t>(1);
    L.sort = align_up(c.used, 256);
    L.bytes = L.sort;
    if (sort && n > 1) L.bytes += sort_workspace_layout(n, end_bit);
    return L;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_isect_workspace_bytes(int64_t C, int64_t N, int64_t n_isects, int tile_width,
                                           int tile_height, int sort) {
    if (C < 1 || N < 0 || tile_width < 1 || tile_height < 1) return 0;
    const int end_bit = 32 + bits_for(static_cast<int64_t>(tile_width) * tile_height) + bits_for(C);
    return isect_layout(C * N, n_isects, end_bit > 64 ? 64 : end_bit, sort).bytes;
}

extern "C" gs_status gs_isect_tiles(const float *means2d, const float *radii, int radii_per_gauss,
                                    const float *depths, int64_t C, int64_t N, int tile_size, int tile_width,
                                    int tile_height, int sort, int32_t *tiles_per_gauss, int32_t *gauss_offsets,
                                    int64_t *n_isects_out, uint64_t *keys, int32_t *flatten_ids, int64_t n_isects,
                                    void *workspace, size_t workspace_bytes, void *stream_handle) {
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    if (C < 1 || N < 0) return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: need C >= 1 and N >= 0 (C=%lld N=%lld)",
                                    (long long)C, (long long)N);
    if (C * N >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: C*N = %lld does not fit the int32 flatten ids",
                    (long long)(C * N));
    if (radii_per_gauss != 1 && radii_per_gauss != 2)
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: radii_per_gauss must be 1 or 2 (got %d)", radii_per_gauss);
    if (tile_size < 1 || tile_width < 1 || tile_height < 1)
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: tile_size, tile_width and tile_height must be positive");
    const int64_t tiles = static_cast<int64_t>(tile_width) * tile_height;
    if (tiles >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: tile grid of %lld tiles is too large", (long long)tiles);
    const int tile_bits = bits_for(tiles);
    const int cam_bits = bits_for(C);
    if (tile_bits + cam_bits > 32)
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: camera bits %d + tile bits %d exceed the 32 upper key bits",
                    cam_bits, tile_bits);
    const int M = static_cast<int>(C * N);
    if (M > 0 && (!means2d || !radii || !depths))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: means2d, radii and depths are required");
    if (M > 0 && !gauss_offsets)
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: gauss_offsets is required in both phases");
    const int blocks = (M + kThreads - 1) / kThreads;
    const float ts = static_cast<float>(tile_size);
    const float2 *m2 = reinterpret_cast<const float2 *>(means2d);

    if (keys == nullptr) {  // ---------------------------------------------------------------- phase 1: count
        if (!n_isects_out) return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: n_isects_out is required to count");
        const IsectLayout L = isect_layout(M, 0, 64, 0);
        if (!workspace || workspace_bytes < L.bytes)
            return fail(GS_ERR_WORKSPACE, "gs_isect_tiles: count needs %zu workspace bytes (got %zu)", L.bytes,
                        workspace_bytes);
        if (M == 0) {
            *n_isects_out = 0;
            return ok();
        }
        int64_t *block_sums = reinterpret_cast<int64_t *>(static_cast<char *>(workspace) + L.block_sums);
        int64_t *total = reinterpret_cast<int64_t *>(static_cast<char *>(workspace) + L.total);
        if (radii_per_gauss == 2)
            hipLaunchKernelGGL(count_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, M, ts,
                               tile_width, tile_height, tiles_per_gauss, block_sums);
        else
            hipLaunchKernelGGL(count_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, M, ts,
                               tile_width, tile_height, tiles_per_gauss, block_sums);
        GS_LAUNCH_TRY("count_kernel");
        hipLaunchKernelGGL(scan_block_sums_kernel, dim3(1), dim3(kThreads), 0, stream, block_sums, blocks, total);
        GS_LAUNCH_TRY("scan_block_sums_kernel");
        if (radii_per_gauss == 2)
            hipLaunchKernelGGL(offsets_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, M, ts,
                               tile_width, tile_height, block_sums, gauss_offsets);
        else
            hipLaunchKernelGGL(offsets_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, M, ts,
                               tile_width, tile_height, block_sums, gauss_offsets);
        GS_LAUNCH_TRY("offsets_kernel");
        int64_t host_total = 0;
        GS_HIP_TRY(hipMemcpyAsync(&host_total, total, sizeof host_total, hipMemcpyDeviceToHost, stream));
        GS_HIP_TRY(hipStreamSynchronize(stream));
        *n_isects_out = host_total;
        if (host_total >= (int64_t(1) << 31))
            return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: %lld intersections exceed the int32 offsets",
                        (long long)host_total);
        return ok();
    }

    // ------------------------------------------------------------------------------------------ phase 2: emit
    if (!flatten_ids) return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: flatten_ids is required to emit");
    if (n_isects < 0 || n_isects >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: n_isects = %lld out of range", (long long)n_isects);
    const int end_bit = 32 + tile_bits + cam_bits;
    if (sort && n_isects > 1 && n_isects >= (int64_t(1) << 30))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: sorting supports at most 2^30 - 1 intersections");
    const IsectLayout L = isect_layout(M, n_isects, end_bit, sort);
    if (!workspace || workspace_bytes < L.bytes)
        return fail(GS_ERR_WORKSPACE, "gs_isect_tiles: emit needs %zu workspace bytes (got %zu)", L.bytes,
                    workspace_bytes);
    if (M == 0 || n_isects == 0) return ok();
    const uint32_t *dbits = reinterpret_cast<const uint32_t *>(depths);
    if (radii_per_gauss == 2)
        hipLaunchKernelGGL(emit_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, dbits, M,
                           static_cast<int>(N), ts, tile_width, tile_height, tile_bits, gauss_offsets,
                           static_cast<int>(n_isects), keys, flatten_ids);
    else
        hipLaunchKernelGGL(emit_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, dbits, M,
                           static_cast<int>(N), ts, tile_width, tile_height, tile_bits, gauss_offsets,
                           static_cast<int>(n_isects), keys, flatten_ids);
    GS_LAUNCH_TRY("emit_kernel");
    if (sort && n_isects > 1)
        return sort_pairs_u64(keys, flatten_ids, n_isects, end_bit, static_cast<char *>(workspace) + L.sort,
                              stream);
    return ok();
}

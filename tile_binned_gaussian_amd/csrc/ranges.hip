// Per-tile ranges of a sorted intersection array by boundary detection: position i compares the global tile of
// key i with that of key i - 1 and, when they differ, writes i as the start offset of every tile in between
// (empty tiles included). Each thread walks kPer consecutive positions (16-byte loads when the keys are 16-byte
// aligned), so it reads one key before its run and its own kPer keys. Output format and the out-of-grid error:
// gsplat 1.0.0 native extension, intersections.c, gs_offset_encode; range reading: raster_backward.c,
// gs_raster_backward_without_gvl.
#include "gs_internal.hpp"

namespace gs {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 8;  // positions per thread
constexpr uint32_t kErrOutOfGrid = 1u;
constexpr uint32_t kErrUnsorted = 2u;

struct Grid {
    int tile_bits;
    uint32_t tile_mask;
    int64_t per_camera;
    int64_t C;
    int64_t total;  // C * per_camera
};

// Global tile of a key, or `g.total` (one past the end) with *err set when it decodes outside the grid.
__device__ __forceinline__ int64_t global_tile(uint64_t key, const Grid &g, uint32_t *err) {
    const uint64_t upper = key >> 32;
    const uint64_t camera = upper >> g.tile_bits;
    const uint64_t tile = upper & g.tile_mask;
    if (camera >= static_cast<uint64_t>(g.C) || tile >= static_cast<uint64_t>(g.per_camera)) {
        *err |= kErrOutOfGrid;
        return g.total;
    }
    return static_cast<int64_t>(camera) * g.per_camera + static_cast<int64_t>(tile);
}

template <bool kVec>
__global__ __launch_bounds__(kThreads) void ranges_kernel(const uint64_t *__restrict__ keys, int64_t n, Grid g,
                                                          int32_t *__restrict__ offsets, uint32_t *__restrict__ flag) {
    const int64_t base = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * kPer;
    if (base >= n) return;
    uint64_t k[kPer];
    if (kVec && base + kPer <= n) {
        const ulonglong2 *v = reinterpret_cast<const ulonglong2 *>(keys + base);
#pragma unroll
        for (int j = 0; j < kPer / 2; ++j) {
            const ulonglong2 x = v[j];
            k[2 * j] = x.x;
            k[2 * j + 1] = x.y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) k[j] = base + j < n ? keys[base + j] : 0ull;
    }
    uint32_t err = 0;
    int64_t prev = (base == 0) ? -1 : global_tile(keys[base - 1], g, &err);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = base + j;
        if (i >= n) break;
        const int64_t cur = global_tile(k[j], g, &err);
        if (prev > cur) err |= kErrUnsorted;
        // tiles (prev, cur] start at i
        const int64_t hi = cur < g.total ? cur : g.total - 1;
        for (int64_t t = prev + 1; t <= hi; ++t) offsets[t] = static_cast<int32_t>(i);
        if (i == n - 1)
            for (int64_t t = (cur > prev ? cur : prev) + 1; t < g.total; ++t) offsets[t] = static_cast<int32_t>(n);
        prev = cur;
    }
    if (err && flag) atomicOr(flag, err);
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_tile_ranges_workspace_bytes(void) { return 256; }

extern "C" gs_status gs_tile_ranges(const uint64_t *sorted_keys, int64_t n, int64_t C, int tile_width,
                                    int tile_height, int32_t *isect_offsets, int validate, void *workspace,
                                    size_t workspace_bytes, void *stream_handle) {
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    if (C < 1 || tile_width < 1 || tile_height < 1)
        return fail(GS_ERR_INVALID_ARG, "gs_tile_ranges: need C, tile_width, tile_height >= 1");
    const int64_t per_camera = static_cast<int64_t>(tile_width) * tile_height;
    const int tile_bits = bits_for(per_camera);
    if (tile_bits + bits_for(C) > 32 || C * per_camera >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_tile_ranges: the grid does not fit the key's upper 32 bits");
    if (n < 0 || n >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_tile_ranges: n = %lld outside [0, 2^31)", (long long)n);
    if (!isect_offsets || (n > 0 && !sorted_keys))
        return fail(GS_ERR_INVALID_ARG, "gs_tile_ranges: keys and isect_offsets are required");
    if (!workspace || workspace_bytes < gs_tile_ranges_workspace_bytes())
        return fail(GS_ERR_WORKSPACE, "gs_tile_ranges: needs %zu workspace bytes", gs_tile_ranges_workspace_bytes());
    uint32_t *flag = static_cast<uint32_t *>(workspace);
    Grid g{tile_bits, tile_bits == 0 ? 0u : static_cast<uint32_t>((uint64_t(1) << tile_bits) - 1), per_camera, C,
           C * per_camera};
    if (n == 0) {
        GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(isect_offsets), 0, static_cast<size_t>(g.total), stream));
        return ok();
    }
    if (validate) GS_HIP_TRY(fill_u32(flag, 0, 1, stream));
    const int64_t per_block = static_cast<int64_t>(kThreads) * kPer;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (reinterpret_cast<uintptr_t>(sorted_keys) % 16 == 0)
        hipLaunchKernelGGL(ranges_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                           sorted_keys, n, g, isect_offsets, validate ? flag : nullptr);
    else
        hipLaunchKernelGGL(ranges_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                           sorted_keys, n, g, isect_offsets, validate ? flag : nullptr);
    GS_LAUNCH_TRY("ranges_kernel");
    if (validate) {
        uint32_t host_flag = 0;
        GS_HIP_TRY(hipMemcpyAsync(&host_flag, flag, sizeof host_flag, hipMemcpyDeviceToHost, stream));
        GS_HIP_TRY(hipStreamSynchronize(stream));
        if (host_flag & kErrOutOfGrid)
            return fail(GS_ERR_OUT_OF_GRID, "gs_tile_ranges: intersection key is outside the tile grid");
        if (host_flag & kErrUnsorted)
            return fail(GS_ERR_INVALID_ARG, "gs_tile_ranges: keys are not sorted by tile");
    }
    return ok();
}

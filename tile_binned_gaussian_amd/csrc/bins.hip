// Fixed-capacity per-tile bins on gfx950, the alternative to sort-based binning: every (camera, splat) claims a
// slot in each bin its rectangle covers by atomic adds on the bin's counter (no global sort, no prefix sums;
// aggregated per workgroup in LDS when the tile counters fit there), then one workgroup per bin orders the bin's
// entries in LDS by (depth bit pattern, flat id) with a bitonic network and writes them back followed by -1
// sentinels. The result holds, bin by bin, the same list
// as the sorted intersection path (when no bin overflows).
//
// Layout: the -1-sentinel bins [C, th, tw, capacity] int32 read by PyTorch3D rasterize_meshes.cu
// (RasterizeMeshesFineCudaKernel); the rectangles are gsplat 1.0.0 intersections.c gs_bounds.
#include "gs_rect.hpp"

namespace gs {
namespace {

constexpr int kFillThreads = 256;
constexpr int kChunkThreads = 1024;
constexpr int kChunkBlocks = 256;    // one chunk of splats per CU
constexpr int kLdsTiles = 32768;     // the chunked fill keeps one 4-byte counter per tile in LDS (128 KB at most)
constexpr int kSortThreads = 1024;
constexpr int kMaxCapacity = 16384;  // the bitonic sort holds a bin's 8-byte keys in LDS (128 KB at most)

// One thread per (camera, splat): a slot per covered tile, claimed with an atomic add on the tile's count.
// The count keeps growing past the capacity, so it ends as the tile's full count; slots past the capacity are
// not written.
template <int RPG>
__global__ __launch_bounds__(kFillThreads) void bin_fill_kernel(const float2 *__restrict__ means,
                                                                const float *__restrict__ radii, int M, int N,
                                                                float ts, int tw, int th, int capacity,
                                                                int32_t *__restrict__ bin_ids,
                                                                int32_t *__restrict__ bin_counts) {
    const int i = blockIdx.x * kFillThreads + threadIdx.x;
    if (i >= M) return;
    const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
    const int64_t base = static_cast<int64_t>(i / N) * tw * th;
    for (int ty = r.y0; ty < r.y1; ++ty)
        for (int tx = r.x0; tx < r.x1; ++tx) {
            const int64_t t = base + static_cast<int64_t>(ty) * tw + tx;
            const int slot = atomicAdd(&bin_counts[t], 1);
            if (slot < capacity) bin_ids[t * capacity + slot] = i;
        }
}

// The same slot claims with one global atomic per (workgroup, touched tile) instead of one per (splat, tile):
// each workgroup takes a contiguous chunk of splats, counts its (splat, tile) pairs per tile with LDS atomics,
// reserves each touched tile's share of the bin with one global atomic add, then walks the chunk again and hands
// out slots from the reserved bases with LDS atomics. Needs C * th * tw <= kLdsTiles.
template <int RPG>
__global__ __launch_bounds__(kChunkThreads) void bin_fill_chunked_kernel(const float2 *__restrict__ means,
                                                                         const float *__restrict__ radii, int M, int N,
                                                                         int chunk, float ts, int tw, int th,
                                                                         int tiles, int capacity,
                                                                         int32_t *__restrict__ bin_ids,
                                                                         int32_t *__restrict__ bin_counts) {
    extern __shared__ int32_t s_cursor[];  // [tiles]: the chunk's count per tile, then its next slot
    const int c0 = blockIdx.x * chunk;
    const int c1 = c0 + chunk < M ? c0 + chunk : M;
    for (int t = threadIdx.x; t < tiles; t += kChunkThreads) s_cursor[t] = 0;
    __syncthreads();
    for (int i = c0 + threadIdx.x; i < c1; i += kChunkThreads) {
        const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
        const int base = (i / N) * tw * th;
        for (int ty = r.y0; ty < r.y1; ++ty)
            for (int tx = r.x0; tx < r.x1; ++tx) atomicAdd(&s_cursor[base + ty * tw + tx], 1);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < tiles; t += kChunkThreads) {
        const int n = s_cursor[t];
        if (n > 0) s_cursor[t] = atomicAdd(&bin_counts[t], n);
    }
    __syncthreads();
    for (int i = c0 + threadIdx.x; i < c1; i += kChunkThreads) {
        const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
        const int base = (i / N) * tw * th;
        for (int ty = r.y0; ty < r.y1; ++ty)
            for (int tx = r.x0; tx < r.x1; ++tx) {
                const int t = base + ty * tw + tx;
                const int slot = atomicAdd(&s_cursor[t], 1);
                if (slot < capacity) bin_ids[static_cast<int64_t>(t) * capacity + slot] = i;
            }
    }
}

// One workgroup per bin: keys (depth bits << 32 | flat id) of the bin's min(count, capacity) entries, padded
// to a power of two with all-ones keys, sorted ascending by a bitonic network in LDS; the ids are written back
// in that order and every further slot gets -1. Keys are unique (ids are), so the order is unique.
__global__ __launch_bounds__(kSortThreads) void bin_sort_kernel(const float *__restrict__ depths, int capacity,
                                                                int32_t *__restrict__ bin_ids,
                                                                const int32_t *__restrict__ bin_counts) {
    extern __shared__ uint64_t s_keys[];
    const int64_t t = blockIdx.x;
    int32_t *bin = bin_ids + t * capacity;
    int n = bin_counts[t];
    n = n < capacity ? n : capacity;
    int P = 1;
    while (P < n) P <<= 1;
    for (int i = threadIdx.x; i < P; i += kSortThreads) {
        uint64_t key = ~0ull;
        if (i < n) {
            const int g = bin[i];
            key = (static_cast<uint64_t>(__float_as_uint(depths[g])) << 32) | static_cast<uint32_t>(g);
        }
        s_keys[i] = key;
    }
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < P / 2; i += kSortThreads) {
                const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));  // i-th pair: (lo, lo + j)
                const int hi = lo + j;
                const bool ascending = (lo & k) == 0;
                const uint64_t x = s_keys[lo], y = s_keys[hi];
                if ((x > y) == ascending) {
                    s_keys[lo] = y;
                    s_keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < capacity; i += kSortThreads)
        bin[i] = i < n ? static_cast<int32_t>(static_cast<uint32_t>(s_keys[i])) : -1;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" gs_status gs_bin_tiles(const float *means2d, const float *radii, int radii_per_gauss, const float *depths,
                                  int64_t C, int64_t N, int tile_size, int tile_width, int tile_height, int capacity,
                                  int32_t *bin_ids, int32_t *bin_counts, void *stream_handle) {
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    if (C < 1 || N < 0 || C * N >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_bin_tiles: need C >= 1, N >= 0 and C*N < 2^31");
    if (radii_per_gauss != 1 && radii_per_gauss != 2)
        return fail(GS_ERR_INVALID_ARG, "gs_bin_tiles: radii_per_gauss must be 1 or 2");
    if (tile_size < 1 || tile_width < 1 || tile_height < 1)
        return fail(GS_ERR_INVALID_ARG, "gs_bin_tiles: tile_size, tile_width and tile_height must be >= 1");
    if (capacity < 1 || capacity > kMaxCapacity)
        return fail(GS_ERR_INVALID_ARG, "gs_bin_tiles: capacity = %d outside [1, %d]", capacity, kMaxCapacity);
    const int64_t tiles = C * tile_width * tile_height;
    if (tiles * capacity >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_bin_tiles: C * tile_height * tile_width * capacity must be < 2^31");
    if (!bin_ids || !bin_counts || (N > 0 && (!means2d || !radii || !depths)))
        return fail(GS_ERR_INVALID_ARG, "gs_bin_tiles: a required pointer is NULL");
    GS_HIP_TRY(fill_u32(reinterpret_cast<uint32_t *>(bin_counts), 0u, static_cast<size_t>(tiles), stream));
    const int M = static_cast<int>(C * N);
    const float ts = static_cast<float>(tile_size);
    const float2 *m = reinterpret_cast<const float2 *>(means2d);
    if (M > 0 && tiles <= kLdsTiles) {
        const int chunk = (M + kChunkBlocks - 1) / kChunkBlocks;
        const dim3 grid(static_cast<unsigned>((M + chunk - 1) / chunk));
        const size_t lds = static_cast<size_t>(tiles) * sizeof(int32_t);
        if (radii_per_gauss == 2) {
            if (lds > 65536)
                GS_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(bin_fill_chunked_kernel<2>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)));
            hipLaunchKernelGGL(bin_fill_chunked_kernel<2>, grid, dim3(kChunkThreads), lds, stream, m, radii, M,
                               static_cast<int>(N), chunk, ts, tile_width, tile_height, static_cast<int>(tiles),
                               capacity, bin_ids, bin_counts);
        } else {
            if (lds > 65536)
                GS_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(bin_fill_chunked_kernel<1>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)));
            hipLaunchKernelGGL(bin_fill_chunked_kernel<1>, grid, dim3(kChunkThreads), lds, stream, m, radii, M,
                               static_cast<int>(N), chunk, ts, tile_width, tile_height, static_cast<int>(tiles),
                               capacity, bin_ids, bin_counts);
        }
        GS_LAUNCH_TRY("bin_fill_chunked_kernel");
    } else if (M > 0) {
        const dim3 grid(static_cast<unsigned>((M + kFillThreads - 1) / kFillThreads));
        if (radii_per_gauss == 2)
            hipLaunchKernelGGL(bin_fill_kernel<2>, grid, dim3(kFillThreads), 0, stream, m, radii, M,
                               static_cast<int>(N), ts, tile_width, tile_height, capacity, bin_ids, bin_counts);
        else
            hipLaunchKernelGGL(bin_fill_kernel<1>, grid, dim3(kFillThreads), 0, stream, m, radii, M,
                               static_cast<int>(N), ts, tile_width, tile_height, capacity, bin_ids, bin_counts);
        GS_LAUNCH_TRY("bin_fill_kernel");
    }
    int P = 1;
    while (P < capacity) P <<= 1;
    const size_t lds = static_cast<size_t>(P) * sizeof(uint64_t);
    if (lds > 65536)
        GS_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(bin_sort_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)));
    hipLaunchKernelGGL(bin_sort_kernel, dim3(static_cast<unsigned>(tiles)), dim3(kSortThreads), lds, stream, depths,
                       capacity, bin_ids, bin_counts);
    GS_LAUNCH_TRY("bin_sort_kernel");
    return ok();
}

// Splat -> tile intersections on gfx950: a coalesced rectangle-and-count pass with a workgroup reduction, a
// device-wide exclusive prefix of the counts, and a load-balanced key emission in which every thread owns
// output slots (so the 8-byte key and 4-byte id stores are contiguous) and finds the splat that produced each
// slot by a search over the workgroup's offsets in LDS.
//
// Definitions: gsplat 1.0.0 native extension, intersections.c (gs_bounds, gs_tile_bits, gs_isect_tiles).
#include "gs_rect.hpp"
#include "gs_sort.hpp"

namespace gs {
namespace {

constexpr int kThreads = 256;
// emission workgroups: 16 per CU, each striding over chunks of splats (4096 emitted 13M intersections 12% faster
// than 2048; 8192 were no faster)
constexpr int kEmitBlocks = 4096;

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

// Phase 1a: per-splat tile count, and one partial sum per workgroup. rects (nullable) receives each splat's
// rectangle as (x0, y0, width, height) in tiles, for the depth-ordered steps.
template <int RPG>
__global__ __launch_bounds__(kThreads) void count_kernel(const float2 *__restrict__ means,
                                                         const float *__restrict__ radii, int M, float ts, int tw,
                                                         int th, int32_t *__restrict__ tiles_per_gauss,
                                                         int4 *__restrict__ rects, int64_t *__restrict__ block_sums) {
    __shared__ int64_t s_tmp[kThreads / kWave];
    const int j = blockIdx.x * kThreads + threadIdx.x;
    int64_t count = 0;
    if (j < M) {
        const Rect r = rect_of<RPG>(means, radii, j, ts, tw, th);
        count = static_cast<int64_t>(r.x1 - r.x0) * static_cast<int64_t>(r.y1 - r.y0);
        tiles_per_gauss[j] = static_cast<int32_t>(count);
        if (rects) rects[j] = make_int4(r.x0, r.y0, r.x1 - r.x0, r.y1 - r.y0);
    }
    const int64_t total = block_sum(count, s_tmp);
    if (threadIdx.x == 0) block_sums[blockIdx.x] = total;
}

// Phase 1b: exclusive scan of the workgroup sums in place (one workgroup), total to *total_out. The sums pass
// through LDS in chunks of 16 per thread: each thread adds its 16 consecutive values, one workgroup scan spreads
// the partial sums, and each thread writes its 16 prefixes (LDS rows padded by one word against bank conflicts).
constexpr int kScanPer = 16;
constexpr int kScanChunk = kThreads * kScanPer;
__device__ __forceinline__ int scan_slot(int i) { return i + i / kScanPer; }

__global__ __launch_bounds__(kThreads) void scan_block_sums_kernel(int64_t *__restrict__ sums, int count,
                                                                   int64_t *__restrict__ total_out) {
    __shared__ int64_t s_v[kScanChunk + kScanChunk / kScanPer];
    __shared__ int64_t s_tmp[kThreads / kWave];
    int64_t carry = 0;
    for (int base = 0; base < count; base += kScanChunk) {
        const int len = count - base < kScanChunk ? count - base : kScanChunk;
        for (int i = threadIdx.x; i < len; i += kThreads) s_v[scan_slot(i)] = sums[base + i];
        __syncthreads();
        const int first = static_cast<int>(threadIdx.x) * kScanPer;
        int64_t local = 0;
#pragma unroll
        for (int i = 0; i < kScanPer; ++i)
            if (first + i < len) local += s_v[scan_slot(first + i)];
        int64_t chunk_total;
        int64_t run = carry + block_exclusive(local, s_tmp, &chunk_total);
#pragma unroll
        for (int i = 0; i < kScanPer; ++i) {
            if (first + i < len) {
                const int64_t v = s_v[scan_slot(first + i)];
                s_v[scan_slot(first + i)] = run;
                run += v;
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < len; i += kThreads) sums[base + i] = s_v[scan_slot(i)];
        carry += chunk_total;
        __syncthreads();
    }
    if (threadIdx.x == 0) *total_out = carry;
}

// Phase 1c: per-splat first output slot = workgroup prefix + exclusive scan of the counts within it (the counts
// are read back from phase 1a, coalesced).
__global__ __launch_bounds__(kThreads) void offsets_kernel(const int32_t *__restrict__ tiles_per_gauss, int M,
                                                           const int64_t *__restrict__ block_prefix,
                                                           int32_t *__restrict__ gauss_offsets) {
    __shared__ int64_t s_tmp[kThreads / kWave];
    const int j = blockIdx.x * kThreads + threadIdx.x;
    const int64_t count = j < M ? static_cast<int64_t>(tiles_per_gauss[j]) : 0;
    int64_t unused;
    const int64_t ex = block_exclusive(count, s_tmp, &unused);
    if (j < M) gauss_offsets[j] = static_cast<int32_t>(block_prefix[blockIdx.x] + ex);
}

// Depth order, step 1: position j holds splat perm[j]; its rectangle is gathered once into depth order and its
// count summed per workgroup. A perm entry outside [0, M) - only possible with a corrupted workspace - gives an
// empty rectangle.
__global__ __launch_bounds__(kThreads) void perm_rects_kernel(const int32_t *__restrict__ perm,
                                                              const int4 *__restrict__ rects, int M,
                                                              int4 *__restrict__ sorted_rects,
                                                              int64_t *__restrict__ block_sums) {
    __shared__ int64_t s_tmp[kThreads / kWave];
    const int j = blockIdx.x * kThreads + threadIdx.x;
    int64_t count = 0;
    if (j < M) {
        const int i = perm[j];
        const int4 r = static_cast<unsigned>(i) < static_cast<unsigned>(M) ? rects[i] : make_int4(0, 0, 0, 0);
        sorted_rects[j] = r;
        count = static_cast<int64_t>(r.z) * static_cast<int64_t>(r.w);
    }
    const int64_t sum = block_sum(count, s_tmp);
    if (threadIdx.x == 0) block_sums[blockIdx.x] = sum;
}

// Depth order, step 2: first output slot per position = workgroup prefix + exclusive scan within the workgroup.
__global__ __launch_bounds__(kThreads) void perm_offsets_kernel(const int4 *__restrict__ sorted_rects, int M,
                                                                const int64_t *__restrict__ block_prefix,
                                                                int32_t *__restrict__ sorted_offsets) {
    __shared__ int64_t s_tmp[kThreads / kWave];
    const int j = blockIdx.x * kThreads + threadIdx.x;
    int64_t count = 0;
    if (j < M) {
        const int4 r = sorted_rects[j];
        count = static_cast<int64_t>(r.z) * static_cast<int64_t>(r.w);
    }
    int64_t unused;
    const int64_t ex = block_exclusive(count, s_tmp, &unused);
    if (j < M) sorted_offsets[j] = static_cast<int32_t>(block_prefix[blockIdx.x] + ex);
}

// floor(k / w) for w >= 1, given rcp_w = 1.0f / w correctly rounded. For 0 <= k < 2^22 the float product is within
// 0.75 of k / w (relative error below 1.5 * 2^-23 on a quotient below 2^22), so truncating it is off by at most one
// and one remainder test in each direction makes it exact; other k take the integer division.
__device__ __forceinline__ int floor_div(int k, int w, float rcp_w) {
    if (static_cast<unsigned>(k) >= (1u << 22)) return k / w;
    int q = static_cast<int>(static_cast<float>(k) * rcp_w);
    const int r = k - q * w;
    q += (r >= w ? 1 : 0) - (r < 0 ? 1 : 0);
    return q;
}

// Phase 2: a chunk is 256 consecutive positions (splat perm[j], or j without a permutation); their outputs occupy
// the contiguous slots [start(g0), start(g0 + 256)). Each thread walks slots with stride 256, finds the owning
// position (the last one whose start is <= slot) by an unrolled branchless binary search in LDS, and writes key and
// id for tile k of that splat's rectangle in row-major order (row = k / width by a float reciprocal kept per
// position, corrected to the exact quotient). With a permutation, sorted_depth[j] holds the depth bits of splat
// perm[j] (read in order instead of gathered), and sorted_rects[j] its rectangle, so no splat data is gathered.
// Workgroups stride over chunks, so the digit histograms (hist non-null) are flushed to global memory once per
// workgroup, into the histogram copy of that workgroup.
static_assert(kThreads * kMaxPasses == kHistCopyWords, "one emission thread per digit of the histograms");
template <int RPG>
__global__ __launch_bounds__(kThreads) void emit_kernel(const float2 *__restrict__ means,
                                                        const float *__restrict__ radii,
                                                        const uint32_t *__restrict__ depth_bits, int M, int N,
                                                        float ts, int tw, int th, int tile_bits,
                                                        const int32_t *__restrict__ perm,
                                                        const uint32_t *__restrict__ sorted_depth,
                                                        const int4 *__restrict__ sorted_rects,
                                                        const int32_t *__restrict__ gauss_offsets, int n,
                                                        uint64_t *__restrict__ keys, int32_t *__restrict__ ids,
                                                        uint32_t *__restrict__ hist, PassPlan hplan) {
    __shared__ uint32_t s_hist[kMaxPasses][kThreads];
    __shared__ int s_start[kThreads + 1];
    __shared__ int s_x0[kThreads], s_y0[kThreads], s_w[kThreads], s_id[kThreads];
    __shared__ float s_rcp_w[kThreads];
    __shared__ uint32_t s_upper_cam[kThreads], s_depth[kThreads];
    const int lane = __lane_id();
    const uint64_t above_mask = lane == kWave - 1 ? 0ull : (~0ull << (lane + 1));
    if (hist)
        for (int p = 0; p < hplan.passes; ++p) s_hist[p][threadIdx.x] = 0;
    const int chunks = (M + kThreads - 1) / kThreads;
    for (int chunk = blockIdx.x; chunk < chunks; chunk += gridDim.x) {
        const int g0 = chunk * kThreads;
        const int j = g0 + threadIdx.x;
        __syncthreads();  // the previous chunk's LDS reads are done
        if (j < M) {
            int i = perm ? perm[j] : j;
            if (static_cast<unsigned>(i) >= static_cast<unsigned>(M)) i = 0;  // only with a corrupted workspace
            if (sorted_rects) {
                const int4 r = sorted_rects[j];
                s_x0[threadIdx.x] = r.x;
                s_y0[threadIdx.x] = r.y;
                s_w[threadIdx.x] = r.z;
            } else {
                const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
                s_x0[threadIdx.x] = r.x0;
                s_y0[threadIdx.x] = r.y0;
                s_w[threadIdx.x] = r.x1 - r.x0;
            }
            // a slot never maps to an empty rectangle unless the offsets are corrupt; width 1 keeps the division
            // defined
            const int w = max(s_w[threadIdx.x], 1);
            s_w[threadIdx.x] = w;
            s_rcp_w[threadIdx.x] = 1.0f / static_cast<float>(w);
            s_start[threadIdx.x] = gauss_offsets[j];
            s_depth[threadIdx.x] = sorted_depth ? sorted_depth[j] : depth_bits[i];
            s_upper_cam[threadIdx.x] = static_cast<uint32_t>(i / N) << tile_bits;
            s_id[threadIdx.x] = i;
        } else {
            s_start[threadIdx.x] = n;
            s_w[threadIdx.x] = 1;
            s_rcp_w[threadIdx.x] = 1.0f;
            s_x0[threadIdx.x] = s_y0[threadIdx.x] = 0;
            s_depth[threadIdx.x] = s_upper_cam[threadIdx.x] = 0;
            s_id[threadIdx.x] = 0;
        }
        if (threadIdx.x == 0) s_start[kThreads] = (g0 + kThreads < M) ? gauss_offsets[g0 + kThreads] : n;
        __syncthreads();
        // clamped to [0, n] so that offsets inconsistent with n can never address past the outputs
        const int out_end = min(s_start[kThreads], n);
        const int out_begin = min(s_start[0], out_end);
        // every lane runs every round (the histogram's neighbour exchange needs the whole wave)
        for (int round = out_begin; round < out_end; round += kThreads) {
            const int slot = round + static_cast<int>(threadIdx.x);
            const bool in = slot < out_end;
            const int sl = in ? slot : out_end - 1;
            // the largest lo with s_start[lo] <= sl (starts are non-decreasing and s_start[0] <= sl); an empty
            // rectangle shares its start with the next position, so lo never lands on one
            int lo = 0;
#pragma unroll
            for (int step = kThreads / 2; step > 0; step >>= 1)
                if (s_start[lo + step] <= sl) lo += step;
            const int k = sl - s_start[lo];
            const int w = s_w[lo];
            const int ry = floor_div(k, w, s_rcp_w[lo]);
            const int rx = k - ry * w;
            const uint32_t tile = static_cast<uint32_t>(s_y0[lo] + ry) * static_cast<uint32_t>(tw) +
                                  static_cast<uint32_t>(s_x0[lo] + rx);
            const uint64_t upper = static_cast<uint64_t>(s_upper_cam[lo] | tile);
            const uint64_t key = (upper << 32) | static_cast<uint64_t>(s_depth[lo]);
            if (in) {
                keys[slot] = key;
                ids[slot] = s_id[lo];
            }
            if (hist) {
                // consecutive lanes hold consecutive slots: a run of equal digits adds its length once
#pragma unroll
                for (int p = 0; p < kMaxPasses; ++p) {
                    if (p >= hplan.passes) break;
                    const uint32_t d =
                        in ? static_cast<uint32_t>(key >> hplan.shift[p]) & ((1u << hplan.bits[p]) - 1u) : 0xffffffffu;
                    const uint32_t prev = __builtin_amdgcn_update_dpp(0xffffffffu, d, 0x138, 0xf, 0xf, false);
                    const bool start = lane == 0 || d != prev;
                    const uint64_t starts = __ballot(start);
                    if (start && in) {
                        const uint64_t later = starts & above_mask;
                        const int next = later ? __builtin_ctzll(later) : kWave;
                        atomicAdd(&s_hist[p][d], static_cast<uint32_t>(next - lane));
                    }
                }
            }
        }
    }
    // digit histograms of the keys just written, for the sort passes that follow
    if (hist) {
        __syncthreads();
        uint32_t *copy = hist_copy(hist, blockIdx.x);
        for (int p = 0; p < hplan.passes; ++p) {
            const uint32_t c = s_hist[p][threadIdx.x];
            if (c) atomicAdd(&copy[p * kThreads + threadIdx.x], c);
        }
    }
}

// Workspace of gs_isect_tiles. The prefix [0, prefix) depends on M and the sort flag only, so phase 1 and phase 2
// see it at the same offsets: the workgroup sums, the total and, when sorting, the depth order of the splats
// (two u32/i32 ping-pong pairs of M), the rectangles (row-major and in depth order), the per-position offsets in
// that order and the depth sort's scratch. Phase 1
// fills it; phase 2 reads it and adds, when sorting more than one intersection, the alternate intersection buffers
// and the tile sort's scratch.
struct IsectLayout {
    size_t block_sums, total, dkeys_a, dids_a, dkeys_b, dids_b, rects, sorted_rects, sorted_offsets, depth_scratch,
        prefix;
    size_t alt_keys, alt_ids, tile_scratch, bytes;
};

IsectLayout isect_layout(int64_t M, int64_t n, int sort) {
    IsectLayout L{};
    Carver c(nullptr);
    const int64_t blocks = (M + kThreads - 1) / kThreads;
    L.block_sums = align_up(c.used, 256);
    c.take<int64_t>(static_cast<size_t>(blocks > 0 ? blocks : 1));
    L.total = align_up(c.used, 256);
    c.take<int64_t>(1);
    if (sort) {
        const size_t m = static_cast<size_t>(M > 0 ? M : 1);
        L.dkeys_a = align_up(c.used, 256);
        c.take<uint32_t>(m);
        L.dids_a = align_up(c.used, 256);
        c.take<int32_t>(m);
        L.dkeys_b = align_up(c.used, 256);
        c.take<uint32_t>(m);
        L.dids_b = align_up(c.used, 256);
        c.take<int32_t>(m);
        L.rects = align_up(c.used, 256);
        c.take<int4>(m);
        L.sorted_rects = align_up(c.used, 256);
        c.take<int4>(m);
        L.sorted_offsets = align_up(c.used, 256);
        c.take<int32_t>(m);
        L.depth_scratch = align_up(c.used, 256);
        c.take<char>(sort_scratch_layout(static_cast<int64_t>(m)).bytes);
    }
    L.prefix = L.bytes = align_up(c.used, 256);
    if (!(sort && n > 1)) return L;
    const size_t nn = static_cast<size_t>(n);
    L.alt_keys = align_up(c.used, 256);
    c.take<uint64_t>(nn);
    L.alt_ids = align_up(c.used, 256);
    c.take<int32_t>(nn);
    L.tile_scratch = align_up(c.used, 256);
    c.take<char>(sort_scratch_layout(n).bytes);
    L.bytes = align_up(c.used, 256);
    return L;
}

// Whether p is page-locked host memory the device can write directly (a copy into it does not block the host).
bool pinned_host(const void *p) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // an unknown host pointer is not an error here
        return false;
    }
    return attr.type == hipMemoryTypeHost;
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// count -> workgroup sums -> scan -> per-splat offsets.
gs_status launch_counts(int rpg, const float2 *m2, const float *radii, int M, float ts, int tw, int th,
                        int32_t *tiles_per_gauss, int4 *rects, int64_t *block_sums, int64_t *total,
                        int32_t *offsets, hipStream_t stream) {
    const int blocks = (M + kThreads - 1) / kThreads;
    if (rpg == 2)
        hipLaunchKernelGGL(count_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, M, ts, tw, th,
                           tiles_per_gauss, rects, block_sums);
    else
        hipLaunchKernelGGL(count_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, M, ts, tw, th,
                           tiles_per_gauss, rects, block_sums);
    GS_LAUNCH_TRY("count_kernel");
    hipLaunchKernelGGL(scan_block_sums_kernel, dim3(1), dim3(kThreads), 0, stream, block_sums, blocks, total);
    GS_LAUNCH_TRY("scan_block_sums_kernel");
    hipLaunchKernelGGL(offsets_kernel, dim3(blocks), dim3(kThreads), 0, stream, tiles_per_gauss, M, block_sums,
                       offsets);
    GS_LAUNCH_TRY("offsets_kernel");
    return ok();
}

// hist (nullable): accumulate the digit histograms of the emitted keys for the passes of hplan.
gs_status launch_emit(int rpg, const float2 *m2, const float *radii, const uint32_t *dbits, int M, int N, float ts,
                      int tw, int th, int tile_bits, const int32_t *perm, const uint32_t *sorted_depth,
                      const int4 *sorted_rects, const int32_t *offsets, int n, uint64_t *keys, int32_t *ids,
                      uint32_t *hist, const PassPlan &hplan, hipStream_t stream) {
    const int chunks = (M + kThreads - 1) / kThreads;
    const int blocks = chunks < kEmitBlocks ? chunks : kEmitBlocks;
    if (rpg == 2)
        hipLaunchKernelGGL(emit_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, dbits, M, N, ts, tw,
                           th, tile_bits, perm, sorted_depth, sorted_rects, offsets, n, keys, ids, hist, hplan);
    else
        hipLaunchKernelGGL(emit_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, dbits, M, N, ts, tw,
                           th, tile_bits, perm, sorted_depth, sorted_rects, offsets, n, keys, ids, hist, hplan);
    GS_LAUNCH_TRY("emit_kernel");
    return ok();
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_isect_workspace_bytes(int64_t C, int64_t N, int64_t n_isects, int tile_width,
                                           int tile_height, int sort) {
    if (C < 1 || N < 0 || tile_width < 1 || tile_height < 1 || n_isects < 0) return 0;
    return isect_layout(C * N, n_isects, sort).bytes;
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
    if (sort && M >= (1 << 30))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: sorting supports at most 2^30 - 1 splats (C*N = %d)", M);
    if (M > 0 && (!means2d || !radii || !depths))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: means2d, radii and depths are required");
    if (M > 0 && !gauss_offsets)
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: gauss_offsets is required in both phases");
    const float ts = static_cast<float>(tile_size);
    const float2 *m2 = reinterpret_cast<const float2 *>(means2d);

    // the depth order of the splats lands in the B pair after an even number of 8-bit passes over 32 bits
    const PassPlan depth_plan = make_pass_plan(0, 32);
    const bool depth_in_b = depth_plan.passes % 2 == 0;

    if (keys == nullptr) {  // ---------------------------------------------------------------- phase 1: count
        if (!n_isects_out) return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: n_isects_out is required to count");
        if (M > 0 && !tiles_per_gauss)
            return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: tiles_per_gauss is required to count");
        const IsectLayout L = isect_layout(M, 0, sort);
        if (!workspace || workspace_bytes < L.bytes)
            return fail(GS_ERR_WORKSPACE, "gs_isect_tiles: count needs %zu workspace bytes (got %zu)", L.bytes,
                        workspace_bytes);
        if (M == 0) {
            *n_isects_out = 0;
            return ok();
        }
        int64_t *total = at<int64_t>(workspace, L.total);
        int64_t *block_sums = at<int64_t>(workspace, L.block_sums);
        int4 *rects = sort ? at<int4>(workspace, L.rects) : nullptr;
        gs_status st = launch_counts(radii_per_gauss, m2, radii, M, ts, tile_width, tile_height, tiles_per_gauss,
                                     rects, block_sums, total, gauss_offsets, stream);
        if (st != GS_OK) return st;
        // Into page-locked memory the copy is asynchronous, so the depth-order work below is queued before the
        // host waits; into pageable memory the copy call itself waits for the count.
        const bool pinned = pinned_host(n_isects_out);
        int64_t host_total = 0;
        hipEvent_t copied = nullptr;
        GS_HIP_TRY(hipEventCreateWithFlags(&copied, hipEventDisableTiming));
        hipError_t e = hipMemcpyAsync(pinned ? n_isects_out : &host_total, total, sizeof host_total,
                                      hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipEventRecord(copied, stream);
        if (e == hipSuccess && sort) {
            // The depth order and the offsets in that order need only the splats: queue them behind the copy so
            // the device works on them while the count travels to the host and the caller prepares phase 2.
            const uint32_t *dbits = reinterpret_cast<const uint32_t *>(depths);
            int in_b = 0;
            st = radix_sort_pairs<uint32_t>(dbits, nullptr, at<uint32_t>(workspace, L.dkeys_a),
                                            at<int32_t>(workspace, L.dids_a), at<uint32_t>(workspace, L.dkeys_b),
                                            at<int32_t>(workspace, L.dids_b), M, depth_plan,
                                            at<char>(workspace, L.depth_scratch), stream, &in_b);
            const int32_t *perm = at<int32_t>(workspace, depth_in_b ? L.dids_b : L.dids_a);
            const int blocks = (M + kThreads - 1) / kThreads;
            if (st == GS_OK) {
                hipLaunchKernelGGL(perm_rects_kernel, dim3(blocks), dim3(kThreads), 0, stream, perm, rects, M,
                                   at<int4>(workspace, L.sorted_rects), block_sums);
                e = hipGetLastError();
            }
            if (st == GS_OK && e == hipSuccess) {
                // the scan rewrites the total with the same value (the same counts in another order)
                hipLaunchKernelGGL(scan_block_sums_kernel, dim3(1), dim3(kThreads), 0, stream, block_sums, blocks,
                                   total);
                e = hipGetLastError();
            }
            if (st == GS_OK && e == hipSuccess) {
                hipLaunchKernelGGL(perm_offsets_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                                   at<int4>(workspace, L.sorted_rects), M, block_sums,
                                   at<int32_t>(workspace, L.sorted_offsets));
                e = hipGetLastError();
            }
        }
        const hipError_t w = (e == hipSuccess) ? hipEventSynchronize(copied) : e;
        (void)hipEventDestroy(copied);
        if (st != GS_OK) return st;
        if (w != hipSuccess) return fail(GS_ERR_DEVICE, "gs_isect_tiles: %s", hipGetErrorString(w));
        if (pinned) host_total = *static_cast<volatile int64_t *>(n_isects_out);
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
    if (sort && n_isects > 1 && n_isects >= (int64_t(1) << 30))
        return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: sorting supports at most 2^30 - 1 intersections");
    const IsectLayout L = isect_layout(M, n_isects, sort);
    if (!workspace || workspace_bytes < L.bytes)
        return fail(GS_ERR_WORKSPACE, "gs_isect_tiles: emit needs %zu workspace bytes (got %zu)", L.bytes,
                    workspace_bytes);
    if (M == 0 || n_isects == 0) return ok();
    const uint32_t *dbits = reinterpret_cast<const uint32_t *>(depths);
    const int n = static_cast<int>(n_isects);
    if (!(sort && n > 1))  // emission in (camera, splat, tile row, tile column) order
        return launch_emit(radii_per_gauss, m2, radii, dbits, M, static_cast<int>(N), ts, tile_width, tile_height,
                           tile_bits, nullptr, nullptr, nullptr, gauss_offsets, n, keys, flatten_ids, nullptr,
                           PassPlan{}, stream);

    // Sorted output. Phase 1 put the splats in stable (depth bits, flat id) order and computed each position's
    // first output slot in that order; emitting each splat's tiles in that order makes the intersections ordered
    // by (depth bits, id) already, so a stable sort of the camera and tile bits [32, end_bit) alone completes the
    // order by the whole key - the unique stable order by key.
    const int32_t *perm = at<int32_t>(workspace, depth_in_b ? L.dids_b : L.dids_a);
    const uint32_t *sorted_depth = at<uint32_t>(workspace, depth_in_b ? L.dkeys_b : L.dkeys_a);
    const int32_t *sorted_offsets = at<int32_t>(workspace, L.sorted_offsets);
    const int4 *sorted_rects = at<int4>(workspace, L.sorted_rects);
    void *scratch = at<char>(workspace, L.tile_scratch);
    const PassPlan tile_plan = make_pass_plan(32, 32 + tile_bits + cam_bits);
    uint64_t *alt_keys = at<uint64_t>(workspace, L.alt_keys);
    int32_t *alt_ids = at<int32_t>(workspace, L.alt_ids);
    // the tile passes alternate buffers; emit where the last pass then lands in the caller's arrays
    const bool odd = (tile_plan.passes % 2) == 1;
    uint64_t *emit_keys = odd ? alt_keys : keys;
    int32_t *emit_ids = odd ? alt_ids : flatten_ids;
    if (tile_plan.passes == 0)
        return launch_emit(radii_per_gauss, m2, radii, dbits, M, static_cast<int>(N), ts, tile_width, tile_height,
                           tile_bits, perm, sorted_depth, sorted_rects, sorted_offsets, n, emit_keys, emit_ids,
                           nullptr, PassPlan{}, stream);
    // the emission also accumulates the tile passes' digit histograms, so the keys are not read again for them
    gs_status st = radix_prepare(n, scratch, stream);
    if (st != GS_OK) return st;
    st = launch_emit(radii_per_gauss, m2, radii, dbits, M, static_cast<int>(N), ts, tile_width, tile_height, tile_bits,
                     perm, sorted_depth, sorted_rects, sorted_offsets, n, emit_keys, emit_ids,
                     radix_histograms(scratch, n), tile_plan, stream);
    if (st != GS_OK) return st;
    int in_b = 0;
    if (odd)
        return radix_passes<uint64_t>(alt_keys, alt_ids, keys, flatten_ids, alt_keys, alt_ids, n, tile_plan, scratch,
                                      stream, &in_b);
    return radix_passes<uint64_t>(keys, flatten_ids, alt_keys, alt_ids, keys, flatten_ids, n, tile_plan, scratch,
                                  stream, &in_b);
}

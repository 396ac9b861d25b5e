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
// emission workgroups at most, each striding over chunks of 256 splats: a 1M-splat frame gives every chunk its own
// workgroup (3907); with 4096 the 13M intersections of that frame were emitted 12% faster than with 2048, and on the
// 6M-splat and 4 x 3M-splat frames (23K and 47K chunks) 16384 made the emission and tile sort 1.3% faster than 4096
// (8192: 1.1% and 0.7%)
constexpr int kEmitBlocks = 16384;

// ------------------------------------------------------------------------------------------------------------
// Phase 1. A single-pass scan of the tile counts in splat order over partitions of kScanTile consecutive positions
// (each splat's first output slot, and the total); when sorting, the depth sort that follows it also scans the
// counts in depth order, in its last pass. Item i of thread t is position i * kScanThreads + t of the partition, so
// every load and store of a wave is contiguous.
// Partition p is workgroup p: workgroups start in block order on each XCD, so every predecessor of a running
// partition is running or done (the bounded look-back turns any violation into a reported error, not a hang). It
// publishes its sum in its status word, and finds the sum over all predecessors by a decoupled look-back in which
// the 64 lanes of the first wave each inspect one predecessor per round. A status word holds a flag in its top two
// bits (the partition's own sum published, or its inclusive prefix published) and the value below.
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kScanTile = kScanThreads * kScanItems;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr uint64_t kStatAggregate = 1ull << 62;
constexpr uint64_t kStatInclusive = 2ull << 62;
constexpr uint64_t kStatValue = (1ull << 62) - 1;

__device__ __forceinline__ uint64_t load_status(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_status(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Exclusive prefix over the partition's positions of one value per item (item i of thread t at i * kScanThreads +
// t): v[i] is replaced by its prefix and the partition's sum is returned (every thread). The (item row, wave) sums
// are 64 values in position order, scanned by wave 0 in LDS.
static_assert(kScanItems * kScanWaves == kWave, "one lane of wave 0 per (item row, wave) sum");
__device__ __forceinline__ int64_t scan_items_exclusive(int64_t (&v)[kScanItems], int64_t *s_part_sums,
                                                        int64_t *s_total) {
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    int64_t inc[kScanItems];
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        inc[i] = wave_inclusive_sum(v[i]);
        if (lane == kWave - 1) s_part_sums[i * kScanWaves + wave] = inc[i];
    }
    __syncthreads();
    if (wave == 0) {
        const int64_t x = s_part_sums[lane];
        const int64_t x_inc = wave_inclusive_sum(x);
        s_part_sums[lane] = x_inc - x;
        if (lane == kWave - 1) *s_total = x_inc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) v[i] = s_part_sums[i * kScanWaves + wave] + inc[i] - v[i];
    return *s_total;
}

// Publishes the partition's sum and returns the sum over partitions [0, part) (wave 0 only; the other waves get 0).
// Each round every lane of wave 0 loads one predecessor's status word, newest first; the round consumes the words up
// to and including the first inclusive one, or up to the first unpublished one when that comes earlier. After
// spin_limit rounds that find the newest remaining predecessor unpublished the wait gives up: it sets the scan bit
// of *err and returns what it has (the offsets are then wrong; every access stays in bounds).
__device__ int64_t publish_and_look_back(uint64_t *status, uint32_t part, int64_t aggregate, uint32_t spin_limit,
                                         uint32_t *err) {
    if (threadIdx.x >= kWave) return 0;
    const int lane = __lane_id();
    if (lane == 0)
        store_status(status + part, (part == 0 ? kStatInclusive : kStatAggregate) | static_cast<uint64_t>(aggregate));
    if (part == 0) return 0;
    int64_t prefix = 0;
    int64_t j = static_cast<int64_t>(part) - 1;  // the newest predecessor not yet added
    uint32_t idle = 0;
    while (true) {
        const int64_t q = j - lane;
        const uint64_t w = q >= 0 ? load_status(status + q) : kStatInclusive;
        const uint64_t flag = w & ~kStatValue;
        const uint64_t pending = __ballot(flag == 0);
        const uint64_t inclusive = __ballot(flag == kStatInclusive);
        const int first_pending = pending ? __builtin_ctzll(pending) : kWave;
        const int first_inclusive = inclusive ? __builtin_ctzll(inclusive) : kWave;
        const bool done = first_inclusive < first_pending;
        const int used = done ? first_inclusive + 1 : first_pending;
        prefix += wave_sum(lane < used ? static_cast<int64_t>(w & kStatValue) : 0);
        if (done) break;
        j -= used;
        if (used == 0) {
            if (idle++ >= spin_limit) {
                if (lane == 0) atomicOr(err, kDeviceErrScanLookBack);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (lane == 0) store_status(status + part, kStatInclusive | static_cast<uint64_t>(prefix + aggregate));
    return prefix;
}

// Phase 1a: per-splat tile count (tiles_per_gauss), its exclusive prefix in splat order (gauss_offsets) and the total
// (*total; also *total_host when non-null, a device-visible address of page-locked host memory). When sorting,
// rects receives each splat's rectangle as (x0, y0, width, height) in tiles (int4, or one packed word when pk.cx is
// nonzero), and the depth sort's digit histograms
// (hplan's passes over the depth bits) are accumulated, with the tile counts summed by the last pass's digit in
// the row after them, so neither the rectangles nor the depths are read again for them.
static_assert(kScanThreads == 4 * 256, "one thread per digit of the depth sort's four 8-bit passes");
template <int RPG>
__global__ __launch_bounds__(kScanThreads) void count_scan_kernel(
    const float2 *__restrict__ means, const float *__restrict__ radii, const uint32_t *__restrict__ depth_bits, int M,
    float ts, int tw, int th, int32_t *__restrict__ tiles_per_gauss, int32_t *__restrict__ gauss_offsets,
    void *__restrict__ rects, RectPacking pk, int64_t *__restrict__ total, int64_t *total_host, uint64_t *status,
    uint32_t *__restrict__ hist, PassPlan hplan, uint32_t spin_limit, uint32_t *err) {
    __shared__ uint32_t s_hist[4][256];
    // the last pass's digits: key count (low word) and tile count sum (high word), one 64-bit LDS atomic per splat
    __shared__ uint64_t s_top[256];
    __shared__ int64_t s_part_sums[kScanItems * kScanWaves];
    __shared__ int64_t s_total;
    __shared__ int64_t s_prefix;
    if (hist) {
        (&s_hist[0][0])[threadIdx.x] = 0;
        if (threadIdx.x < 256) s_top[threadIdx.x] = 0;
    }
    __syncthreads();
    const uint32_t part = blockIdx.x;
    const int j0 = static_cast<int>(part) * kScanTile + static_cast<int>(threadIdx.x);
    // every load of the thread's splats is issued before any result is used
    float2 m[kScanItems];
    float2 rad[kScanItems];
    uint32_t bits[kScanItems];
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int j = j0 + i * kScanThreads < M ? j0 + i * kScanThreads : M - 1;
        m[i] = means[j];
        rad[i] = RPG == 2 ? reinterpret_cast<const float2 *>(radii)[j] : make_float2(radii[j], radii[j]);
        bits[i] = hist ? depth_bits[j] : 0u;
    }
    int64_t v[kScanItems];
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int j = j0 + i * kScanThreads;
        const Rect r = tile_rect(m[i].x, m[i].y, rad[i].x, rad[i].y, ts, tw, th);
        const int32_t count = j < M ? (r.x1 - r.x0) * (r.y1 - r.y0) : 0;
        v[i] = count;
        if (j < M) {
            tiles_per_gauss[j] = count;
            if (rects && pk.cx) static_cast<uint32_t *>(rects)[j] = pack_rect(r.x0, r.y0, r.x1 - r.x0, r.y1 - r.y0, pk);
            else if (rects) static_cast<int4 *>(rects)[j] = make_int4(r.x0, r.y0, r.x1 - r.x0, r.y1 - r.y0);
        }
    }
    if (hist) {
        const int last = hplan.passes - 1;
#pragma unroll
        for (int i = 0; i < kScanItems; ++i)
            if (j0 + i * kScanThreads < M) {
                for (int p = 0; p < last; ++p)
                    atomicAdd(&s_hist[p][(bits[i] >> hplan.shift[p]) & ((1u << hplan.bits[p]) - 1u)], 1u);
                atomicAdd(&s_top[(bits[i] >> hplan.shift[last]) & ((1u << hplan.bits[last]) - 1u)],
                          (static_cast<uint64_t>(v[i]) << 32) | 1u);
            }
    }
    const int64_t aggregate = scan_items_exclusive(v, s_part_sums, &s_total);
    const int64_t before = publish_and_look_back(status, part, aggregate, spin_limit, err);
    if (threadIdx.x == 0) s_prefix = before;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int j = j0 + i * kScanThreads;
        if (j < M) gauss_offsets[j] = static_cast<int32_t>(s_prefix + v[i]);
    }
    if (threadIdx.x == 0 && static_cast<int64_t>(part + 1) * kScanTile >= M) {
        const int64_t all = s_prefix + aggregate;
        *total = all;
        if (total_host) __hip_atomic_store(total_host, all, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (hist) {
        const int p = threadIdx.x / 256, d = threadIdx.x % 256, last = hplan.passes - 1;
        const uint32_t c = p < last ? s_hist[p][d] : (p == last ? static_cast<uint32_t>(s_top[d]) : 0u);
        if (c) atomicAdd(&hist_copy(hist, part)[p * 256 + d], c);
        const uint32_t w = p == 0 ? static_cast<uint32_t>(s_top[d] >> 32) : 0u;
        if (w) atomicAdd(&hist_copy(hist, part)[hplan.passes * 256 + d], w);
    }
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
// position (the last one whose start is <= slot) by an unrolled branchless binary search in LDS, reads that
// position's two 16-byte LDS records, and writes key and id for tile k of that splat's rectangle in row-major order
// (row = k / width by a float reciprocal kept per position, corrected to the exact quotient). With a permutation,
// sorted_depth[j] holds the depth bits of splat perm[j] (read in order instead of gathered), and sorted_rects[j]
// its rectangle (int4, or one packed word when pk.cx is nonzero), so no splat data is gathered. Workgroups stride
// over chunks, so the digit histograms (hist non-null) are flushed to global memory once per workgroup, into the
// histogram copy of that workgroup. The workgroups also zero clear[0, 4 * clear_quads) (the first look-back array
// of the sort that follows), so no separate clearing launch precedes it.
static_assert(kThreads * kMaxPasses == kHistCopyWords, "one emission thread per digit of the histograms");
template <int RPG>
__global__ __launch_bounds__(kThreads) void emit_kernel(const float2 *__restrict__ means,
                                                        const float *__restrict__ radii,
                                                        const uint32_t *__restrict__ depth_bits, int M, int N,
                                                        float ts, int tw, int th, int tile_bits,
                                                        const int32_t *__restrict__ perm,
                                                        const uint32_t *__restrict__ sorted_depth,
                                                        const void *__restrict__ sorted_rects, RectPacking pk,
                                                        const int32_t *__restrict__ gauss_offsets, int n,
                                                        uint64_t *__restrict__ keys, int32_t *__restrict__ ids,
                                                        uint32_t *__restrict__ hist, PassPlan hplan,
                                                        uint4 *__restrict__ clear, int clear_quads) {
    __shared__ uint32_t s_hist[kMaxPasses][kThreads];
    __shared__ int s_start[kThreads + 1];
    // per position: (start, x0, y0, width) and (1 / width, camera bits, depth bits, id), two 16-byte LDS reads
    __shared__ int4 s_pa[kThreads];
    __shared__ uint4 s_pb[kThreads];
    const RunLanes rl = run_lanes();
    if (hist)
        for (int p = 0; p < hplan.passes; ++p) s_hist[p][threadIdx.x] = 0;
    for (int q = blockIdx.x * kThreads + threadIdx.x; q < clear_quads; q += gridDim.x * kThreads)
        clear[q] = make_uint4(0u, 0u, 0u, 0u);
    const int chunks = (M + kThreads - 1) / kThreads;
    for (int chunk = blockIdx.x; chunk < chunks; chunk += gridDim.x) {
        const int g0 = chunk * kThreads;
        const int j = g0 + threadIdx.x;
        __syncthreads();  // the previous chunk's LDS reads are done
        if (j < M) {
            int i = perm ? perm[j] : j;
            if (static_cast<unsigned>(i) >= static_cast<unsigned>(M)) i = 0;  // only with a corrupted workspace
            int x0, y0, w;
            if (sorted_rects) {
                const int4 r = pk.cx ? unpack_rect(static_cast<const uint32_t *>(sorted_rects)[j], pk)
                                     : static_cast<const int4 *>(sorted_rects)[j];
                x0 = r.x;
                y0 = r.y;
                w = r.z;
            } else {
                const Rect r = rect_of<RPG>(means, radii, i, ts, tw, th);
                x0 = r.x0;
                y0 = r.y0;
                w = r.x1 - r.x0;
            }
            // a slot never maps to an empty rectangle unless the offsets are corrupt; width 1 keeps the division
            // defined
            w = max(w, 1);
            const int start = min(max(gauss_offsets[j], 0), n);
            s_start[threadIdx.x] = start;
            s_pa[threadIdx.x] = make_int4(start, x0, y0, w);
            s_pb[threadIdx.x] = make_uint4(__float_as_uint(1.0f / static_cast<float>(w)),
                                           static_cast<uint32_t>(i / N) << tile_bits,
                                           sorted_depth ? sorted_depth[j] : depth_bits[i], static_cast<uint32_t>(i));
        } else {
            s_start[threadIdx.x] = n;
            s_pa[threadIdx.x] = make_int4(n, 0, 0, 1);
            s_pb[threadIdx.x] = make_uint4(__float_as_uint(1.0f), 0u, 0u, 0u);
        }
        if (threadIdx.x == 0)
            s_start[kThreads] = (g0 + kThreads < M) ? min(max(gauss_offsets[g0 + kThreads], 0), n) : n;
        __syncthreads();
        // Every start is clamped to [0, n] as it is loaded, so offsets inconsistent with n (a workspace that phase 1
        // did not fill, or a wait that gave up) can never address outside the outputs: every slot written lies in
        // [out_begin, out_end), within [0, n). They are then not ordered either, so the search below may land on any
        // position of the chunk; it still reads only s_start[0 .. 255] and the key it builds is merely wrong.
        const int out_end = s_start[kThreads];
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
            const int4 pa = s_pa[lo];
            const uint4 pb = s_pb[lo];
            const int k = sl - pa.x;
            const int w = pa.w;
            const int ry = floor_div(k, w, __uint_as_float(pb.x));
            const int rx = k - ry * w;
            const uint32_t tile = static_cast<uint32_t>(pa.z + ry) * static_cast<uint32_t>(tw) +
                                  static_cast<uint32_t>(pa.y + rx);
            const uint64_t upper = static_cast<uint64_t>(pb.y | tile);
            const uint64_t key = (upper << 32) | static_cast<uint64_t>(pb.z);
            if (in) {
                keys[slot] = key;
                ids[slot] = static_cast<int32_t>(pb.w);
            }
            if (hist) {
                // consecutive lanes hold consecutive slots: a run of equal digits adds its length once; every
                // digit of hplan lies in the key's upper word (its shifts are at least 32, checked on the host)
                const uint32_t upper32 = static_cast<uint32_t>(upper);
#pragma unroll
                for (int p = 0; p < kMaxPasses; ++p) {
                    if (p >= hplan.passes) break;
                    const uint32_t d =
                        in ? (upper32 >> (hplan.shift[p] - 32)) & ((1u << hplan.bits[p]) - 1u) : 0xffffffffu;
                    wave_add_runs(s_hist[p], d, in, rl);
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
// see it at the same offsets: the total, the count scan's status words, and, when sorting, the look-back words of
// the depth sort's last pass, the depth sort's scratch, the depth order of the splats (two u32/i32 ping-pong pairs
// of M), the rectangles (in splat order and in depth order; 4 or 16 bytes each) and the per-position offsets in
// that order. [clear_begin, clear_end) is what phase 1 clears before it starts: the status and look-back words, the
// tile sort's histogram copies and partition counters, and the part of the depth sort's scratch that must start at
// zero. Phase 2 adds, when sorting more than one intersection, the alternate intersection buffers and the rest of
// the tile sort's scratch (its look-back arrays and digit starts).
struct IsectLayout {
    size_t total, count_status, order_status, tile_head, depth_scratch, clear_begin, clear_end;
    size_t dkeys_a, dids_a, dkeys_b, dids_b, rects, sorted_rects, sorted_offsets, prefix;
    size_t alt_keys, alt_ids, tile_scratch, bytes;
};

IsectLayout isect_layout(int64_t M, int64_t n, int sort) {
    IsectLayout L{};
    Carver c(nullptr);
    const size_t parts = static_cast<size_t>(M > 0 ? (M + kScanTile - 1) / kScanTile : 1);
    L.total = align_up(c.used, 256);
    c.take<int64_t>(1);
    L.count_status = L.clear_begin = align_up(c.used, 256);
    c.take<uint64_t>(parts);
    L.clear_end = c.used;
    if (sort) {
        const size_t m = static_cast<size_t>(M > 0 ? M : 1);
        L.order_status = align_up(c.used, 256);
        c.take<char>(depth_order_status_bytes(static_cast<int64_t>(m)));
        L.tile_head = align_up(c.used, 256);
        c.take<char>(sort_scratch_head_bytes());
        L.depth_scratch = align_up(c.used, 256);
        c.take<char>(sort_scratch_layout(static_cast<int64_t>(m)).bytes);
        L.clear_end = L.depth_scratch + radix_clear_bytes(static_cast<int64_t>(m));
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
    }
    L.prefix = L.bytes = align_up(c.used, 256);
    if (!(sort && n > 1)) return L;
    const size_t nn = static_cast<size_t>(n);
    L.alt_keys = align_up(c.used, 256);
    c.take<uint64_t>(nn);
    L.alt_ids = align_up(c.used, 256);
    c.take<int32_t>(nn);
    L.tile_scratch = align_up(c.used, 256);
    c.take<char>(sort_scratch_tail_bytes(n));
    L.bytes = align_up(c.used, 256);
    return L;
}

// The device-visible address of p when it is page-locked host memory the device can write directly, else null.
int64_t *pinned_device_address(int64_t *p) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // an unknown host pointer is not an error here
        return nullptr;
    }
    if (attr.type != hipMemoryTypeHost) return nullptr;
    return static_cast<int64_t *>(attr.devicePointer);
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// The count scan (hist non-null: with the depth sort's histograms of hplan's passes).
gs_status launch_count_scan(int rpg, const float2 *m2, const float *radii, const uint32_t *dbits, int M, float ts,
                            int tw, int th, int32_t *tiles_per_gauss, int32_t *offsets, void *rects,
                            RectPacking pk, int64_t *total,
                            int64_t *total_host, uint64_t *status, uint32_t *hist,
                            const PassPlan &hplan, uint32_t *err, hipStream_t stream) {
    const int parts = (M + kScanTile - 1) / kScanTile;
    const uint32_t spin = spin_limit();
    if (rpg == 2)
        hipLaunchKernelGGL(count_scan_kernel<2>, dim3(parts), dim3(kScanThreads), 0, stream, m2, radii, dbits, M, ts,
                           tw, th, tiles_per_gauss, offsets, rects, pk, total, total_host, status, hist, hplan,
                           spin, err);
    else
        hipLaunchKernelGGL(count_scan_kernel<1>, dim3(parts), dim3(kScanThreads), 0, stream, m2, radii, dbits, M, ts,
                           tw, th, tiles_per_gauss, offsets, rects, pk, total, total_host, status, hist, hplan,
                           spin, err);
    GS_LAUNCH_TRY("count_scan_kernel");
    return ok();
}

// hist (nullable): accumulate the digit histograms of the emitted keys for the passes of hplan, whose digits must
// all lie in the keys' upper words (bits 32..63). clear (nullable, 16-byte aligned): clear_words words (a multiple
// of 4) the emission zeroes.
gs_status launch_emit(int rpg, const float2 *m2, const float *radii, const uint32_t *dbits, int M, int N, float ts,
                      int tw, int th, int tile_bits, const int32_t *perm, const uint32_t *sorted_depth,
                      const void *sorted_rects, RectPacking pk, const int32_t *offsets, int n, uint64_t *keys,
                      int32_t *ids,
                      uint32_t *hist, const PassPlan &hplan, uint32_t *clear, int64_t clear_words,
                      hipStream_t stream) {
    if (hist)
        for (int p = 0; p < hplan.passes; ++p)
            if (hplan.shift[p] < 32 || hplan.shift[p] + hplan.bits[p] > 64)
                return fail(GS_ERR_INVALID_ARG, "emission histogram pass %d over bits [%d, %d) outside the upper word", p,
                            hplan.shift[p], hplan.shift[p] + hplan.bits[p]);
    if (!clear) clear_words = 0;
    if (clear_words % 4 != 0 || clear_words / 4 >= (int64_t(1) << 31) ||
        reinterpret_cast<uintptr_t>(clear) % alignof(uint4) != 0)
        return fail(GS_ERR_INVALID_ARG, "emission: %lld words to clear are not whole aligned 16-byte units",
                    (long long)clear_words);
    uint4 *cq = reinterpret_cast<uint4 *>(clear);
    const int quads = static_cast<int>(clear_words / 4);
    const int chunks = (M + kThreads - 1) / kThreads;
    const int blocks = chunks < kEmitBlocks ? chunks : kEmitBlocks;
    if (rpg == 2)
        hipLaunchKernelGGL(emit_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, dbits, M, N, ts, tw,
                           th, tile_bits, perm, sorted_depth, sorted_rects, pk, offsets, n, keys, ids, hist, hplan, cq,
                           quads);
    else
        hipLaunchKernelGGL(emit_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, m2, radii, dbits, M, N, ts, tw,
                           th, tile_bits, perm, sorted_depth, sorted_rects, pk, offsets, n, keys, ids, hist, hplan, cq,
                           quads);
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
    // rectangles stored for the depth order take one word each when the grid allows it
    const RectPacking pk = rect_packing(tile_width, tile_height);
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
        uint32_t *err = nullptr;
        gs_status st = device_error_word(&err);
        if (st != GS_OK) return st;
        if (depth_plan.passes > 4)
            return fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: the depth sort needs %d passes", depth_plan.passes);
        const uint32_t *dbits = reinterpret_cast<const uint32_t *>(depths);
        int64_t *total = at<int64_t>(workspace, L.total);
        char *depth_scratch = sort ? at<char>(workspace, L.depth_scratch) : nullptr;
        void *rects = sort ? at<void>(workspace, L.rects) : nullptr;
        // Into page-locked memory the count scan writes the total itself and the host waits for that word alone, so
        // the depth-order work queued behind the scan runs while the count travels to the host and the caller
        // prepares phase 2; into pageable memory a copy returns it.
        int64_t *total_host = pinned_device_address(n_isects_out);
        volatile int64_t *host_word = n_isects_out;
        if (total_host) *host_word = -1;
        GS_HIP_TRY(fill_u32(at<uint32_t>(workspace, L.clear_begin), 0, (L.clear_end - L.clear_begin) / sizeof(uint32_t),
                            stream));
        st = launch_count_scan(radii_per_gauss, m2, radii, dbits, M, ts, tile_width, tile_height, tiles_per_gauss,
                               gauss_offsets, rects, pk, total, total_host, at<uint64_t>(workspace, L.count_status),
                               sort ? radix_histograms(depth_scratch, M) : nullptr, depth_plan, err, stream);
        if (st != GS_OK) return st;
        int64_t host_total = 0;
        hipEvent_t copied = nullptr;
        hipError_t e = hipSuccess;
        if (!total_host) {
            GS_HIP_TRY(hipEventCreateWithFlags(&copied, hipEventDisableTiming));
            e = hipMemcpyAsync(&host_total, total, sizeof host_total, hipMemcpyDeviceToHost, stream);
            if (e == hipSuccess) e = hipEventRecord(copied, stream);
        }
        if (e == hipSuccess && sort) {
            // the depth order of the splats (histograms from the count scan), whose last pass also writes the
            // rectangles and first output slots in that order
            int in_b = 0;
            st = depth_order_passes(dbits, at<uint32_t>(workspace, L.dkeys_a), at<int32_t>(workspace, L.dids_a),
                                    at<uint32_t>(workspace, L.dkeys_b), at<int32_t>(workspace, L.dids_b), M,
                                    depth_plan, depth_scratch, rects, at<void>(workspace, L.sorted_rects), pk,
                                    at<int32_t>(workspace, L.sorted_offsets), at<uint64_t>(workspace, L.order_status),
                                    stream, &in_b);
            if (st == GS_OK && (in_b != 0) != depth_in_b)
                st = fail(GS_ERR_INVALID_ARG, "gs_isect_tiles: the depth order landed in the other buffer pair");
        }
        // wait for the total (also after a failed launch, so no write into the caller's memory is left in flight)
        hipError_t w = hipSuccess;
        if (copied) {
            w = hipEventSynchronize(copied);
            (void)hipEventDestroy(copied);
        } else {
            for (uint64_t polls = 1; *host_word < 0; ++polls) {
                if (polls % 1024 != 0) continue;
                const hipError_t q = hipStreamQuery(stream);
                if (q == hipErrorNotReady) continue;
                if (q == hipSuccess && *host_word < 0)  // the stream drained without the scan writing the total
                    return fail(GS_ERR_DEVICE, "gs_isect_tiles: the count scan finished without writing the total");
                w = q;
                break;
            }
            host_total = *host_word;
        }
        if (st != GS_OK) return st;
        if (e != hipSuccess) return fail(GS_ERR_DEVICE, "gs_isect_tiles: %s", hipGetErrorString(e));
        if (w != hipSuccess) return fail(GS_ERR_DEVICE, "gs_isect_tiles: %s", hipGetErrorString(w));
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
                           tile_bits, nullptr, nullptr, nullptr, pk, gauss_offsets, n, keys, flatten_ids, nullptr,
                           PassPlan{}, nullptr, 0, stream);

    // Sorted output. Phase 1 put the splats in stable (depth bits, flat id) order and computed each position's
    // first output slot in that order; emitting each splat's tiles in that order makes the intersections ordered
    // by (depth bits, id) already, so a stable sort of the camera and tile bits [32, end_bit) alone completes the
    // order by the whole key - the unique stable order by key.
    const int32_t *perm = at<int32_t>(workspace, depth_in_b ? L.dids_b : L.dids_a);
    const uint32_t *sorted_depth = at<uint32_t>(workspace, depth_in_b ? L.dkeys_b : L.dkeys_a);
    const int32_t *sorted_offsets = at<int32_t>(workspace, L.sorted_offsets);
    const void *sorted_rects = at<void>(workspace, L.sorted_rects);
    // the tile sort's histogram copies and counters sit in the prefix (zero after phase 1, and again after every
    // tile sort); its look-back arrays and digit starts follow the alternate buffers
    const SortScratch scratch =
        sort_scratch_split(at<char>(workspace, L.tile_head), at<char>(workspace, L.tile_scratch), n);
    const PassPlan tile_plan = make_pass_plan(32, 32 + tile_bits + cam_bits);
    uint64_t *alt_keys = at<uint64_t>(workspace, L.alt_keys);
    int32_t *alt_ids = at<int32_t>(workspace, L.alt_ids);
    // the tile passes alternate buffers; emit where the last pass then lands in the caller's arrays
    const bool odd = (tile_plan.passes % 2) == 1;
    uint64_t *emit_keys = odd ? alt_keys : keys;
    int32_t *emit_ids = odd ? alt_ids : flatten_ids;
    if (tile_plan.passes == 0)
        return launch_emit(radii_per_gauss, m2, radii, dbits, M, static_cast<int>(N), ts, tile_width, tile_height,
                           tile_bits, perm, sorted_depth, sorted_rects, pk, sorted_offsets, n, emit_keys, emit_ids,
                           nullptr, PassPlan{}, nullptr, 0, stream);
    // the emission also accumulates the tile passes' digit histograms, so the keys are not read again for them,
    // and zeroes the first pass's look-back array
    gs_status st = launch_emit(radii_per_gauss, m2, radii, dbits, M, static_cast<int>(N), ts, tile_width, tile_height,
                               tile_bits, perm, sorted_depth, sorted_rects, pk, sorted_offsets, n, emit_keys, emit_ids,
                               scratch.hist, tile_plan, scratch.status0, radix_partitions<uint64_t>(n) * 256, stream);
    if (st != GS_OK) return st;
    int in_b = 0;
    if (odd)
        return radix_passes<uint64_t>(alt_keys, alt_ids, keys, flatten_ids, alt_keys, alt_ids, n, tile_plan, scratch,
                                      stream, &in_b);
    return radix_passes<uint64_t>(keys, flatten_ids, alt_keys, alt_ids, keys, flatten_ids, n, tile_plan, scratch,
                                  stream, &in_b);
}

// Stable LSD radix sort of (64-bit key, int32 id) pairs on gfx950, onesweep style:
//   1. one read of the keys builds every pass's 256-bucket digit histogram in LDS (global atomics at the end);
//   2. one kernel per 8-bit digit pass: a workgroup takes the next partition of 4096 pairs (dynamic index, so
//      every predecessor is already running), ranks its keys stably with wave64 ballot matching, publishes its
//      per-digit counts, resolves its global per-digit offsets by a decoupled look-back over the predecessors'
//      published counts, reorders the pairs through LDS by digit and writes runs of consecutive addresses.
// Only bits [0, end_bit) are sorted; passes over them are ceil(end_bit / 8).
//
// Semantics: gsplat 1.0.0 native extension, intersections.c, gs_radix_sort_without_gvl (a stable LSD radix sort
// of keys with their ids). Stability makes the result unique, so it is compared bit for bit.
#include "gs_internal.hpp"

namespace gs {
namespace {

constexpr int kThreads = 256;                 // 4 waves
constexpr int kWaves = kThreads / kWave;
constexpr int kItems = 16;                    // pairs per thread
constexpr int kTile = kThreads * kItems;      // pairs per partition
constexpr int kWaveSpan = kWave * kItems;     // contiguous pairs owned by one wave
constexpr int kRadix = 256;
constexpr int kMaxPasses = 8;
constexpr uint32_t kFlagAggregate = 1u << 30; // partition's own count published
constexpr uint32_t kFlagInclusive = 2u << 30; // count including every earlier partition published
constexpr uint32_t kValueMask = (1u << 30) - 1;

__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix over the 256 threads of the workgroup (one value each); *total = sum.
__device__ __forceinline__ uint32_t block_exclusive_u32(uint32_t v, uint32_t *s_tmp, uint32_t *total) {
    const int wave = threadIdx.x / kWave, lane = __lane_id();
    const uint32_t inc = wave_inclusive_sum(v);
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t t = s_tmp[w];
        if (w < wave) before += t;
        all += t;
    }
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(kThreads) void histogram_kernel(const uint64_t *__restrict__ keys, int64_t n,
                                                             int passes, int end_bit, uint32_t *__restrict__ hist) {
    __shared__ uint32_t s_hist[kMaxPasses][kRadix];
    for (int p = 0; p < passes; ++p) s_hist[p][threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
#pragma unroll 4
    for (int i = 0; i < kItems; ++i) {
        const int64_t idx = base + i * kThreads + threadIdx.x;
        if (idx < n) {
            const uint64_t k = keys[idx];
            for (int p = 0; p < passes; ++p) {
                const int shift = 8 * p;
                const int bits = end_bit - shift < 8 ? end_bit - shift : 8;
                const uint32_t d = static_cast<uint32_t>(k >> shift) & ((1u << bits) - 1u);
                atomicAdd(&s_hist[p][d], 1u);
            }
        }
    }
    __syncthreads();
    for (int p = 0; p < passes; ++p) {
        const uint32_t c = s_hist[p][threadIdx.x];
        if (c) atomicAdd(&hist[p * kRadix + threadIdx.x], c);
    }
}

// One digit pass. Partition `part` covers pairs [part * kTile, part * kTile + kTile); wave w owns the
// contiguous span [w * kWaveSpan, (w + 1) * kWaveSpan) of it, item i of lane l sitting at w*kWaveSpan + i*64 + l,
// so (wave, item, lane) order is input order and the per-wave running counts give a stable rank.
// status[part][d] holds the look-back words of this pass; status_next[part][d] is cleared for the next pass.
__global__ __launch_bounds__(kThreads) void onesweep_pass_kernel(
    const uint64_t *__restrict__ keys_in, const int32_t *__restrict__ ids_in, uint64_t *__restrict__ keys_out,
    int32_t *__restrict__ ids_out, int64_t n, int shift, int digit_bits, const uint32_t *__restrict__ hist,
    uint32_t *__restrict__ part_counter, uint32_t *status, uint32_t *__restrict__ status_next) {
    __shared__ uint64_t s_keys[kTile];
    __shared__ int32_t s_ids[kTile];
    __shared__ uint32_t s_wave_hist[kWaves][kRadix];
    __shared__ uint32_t s_local_start[kRadix];
    __shared__ uint32_t s_global_base[kRadix];
    __shared__ uint32_t s_tmp[kWaves];
    __shared__ uint32_t s_part;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = __lane_id();
    const uint32_t digit_mask = (1u << digit_bits) - 1u;

    if (tid == 0) s_part = atomicAdd(part_counter, 1u);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_wave_hist[w][tid] = 0;
    __syncthreads();
    const uint32_t part = s_part;
    if (status_next) status_next[static_cast<size_t>(part) * kRadix + tid] = 0;

    // global start of each digit bucket for this pass (exclusive scan of the histogram)
    uint32_t unused_total;
    const uint32_t digit_global_start = block_exclusive_u32(hist[tid], s_tmp, &unused_total);

    // load this wave's span
    const int64_t base = static_cast<int64_t>(part) * kTile + static_cast<int64_t>(wave) * kWaveSpan;
    uint64_t k[kItems];
    int32_t v[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t pos = base + i * kWave + lane;
        if (pos < n) {
            k[i] = keys_in[pos];
            v[i] = ids_in[pos];
        } else {
            k[i] = ~0ull;  // past the end: largest digit, ranked after every real pair of this partition
            v[i] = 0;
        }
    }

    // stable rank within the wave: lanes holding the same digit found by ballots over the digit's bits
    uint32_t rank[kItems];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const uint32_t d = static_cast<uint32_t>(k[i] >> shift) & digit_mask;
        uint64_t same = ~0ull;
        for (int b = 0; b < digit_bits; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t ballot = __ballot(bit);
            same &= bit ? ballot : ~ballot;
        }
        const uint32_t below = static_cast<uint32_t>(__popcll(same & lt_mask));
        const uint32_t run = s_wave_hist[wave][d];
        rank[i] = run + below;
        const int leader = 63 - __clzll(same);
        if (lane == leader) s_wave_hist[wave][d] = run + static_cast<uint32_t>(__popcll(same));
    }
    __syncthreads();

    // per digit (thread d): counts of the 4 waves -> exclusive prefix over waves, and the partition total
    const int d = tid;
    uint32_t running = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t c = s_wave_hist[w][d];
        s_wave_hist[w][d] = running;
        running += c;
    }
    const uint32_t part_count = running;
    uint32_t *my_status = status + static_cast<size_t>(part) * kRadix + d;
    if (part == 0) atomic_store_agent(my_status, kFlagInclusive | part_count);
    else atomic_store_agent(my_status, kFlagAggregate | part_count);

    uint32_t local_total;
    const uint32_t local_start = block_exclusive_u32(part_count, s_tmp, &local_total);
    s_local_start[d] = local_start;

    // decoupled look-back: sum the predecessors' counts for digit d until one publishes an inclusive count
    uint32_t before = 0;
    if (part > 0) {
        int64_t j = static_cast<int64_t>(part) - 1;
        while (true) {
            const uint32_t s = atomic_load_agent(status + static_cast<size_t>(j) * kRadix + d);
            const uint32_t flag = s & ~kValueMask;
            if (flag == 0) {
                __builtin_amdgcn_s_sleep(1);
                continue;
            }
            before += s & kValueMask;
            if (flag == kFlagInclusive) break;
            --j;
        }
        atomic_store_agent(my_status, kFlagInclusive | (before + part_count));
    }
    s_global_base[d] = digit_global_start + before;
    __syncthreads();

    // reorder the partition by digit through LDS
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const uint32_t dd = static_cast<uint32_t>(k[i] >> shift) & digit_mask;
        const uint32_t lp = s_local_start[dd] + s_wave_hist[wave][dd] + rank[i];
        s_keys[lp] = k[i];
        s_ids[lp] = v[i];
    }
    __syncthreads();

    // write: consecutive local positions of one digit go to consecutive global positions
    const int64_t valid64 = n - static_cast<int64_t>(part) * kTile;
    const int valid = valid64 < kTile ? static_cast<int>(valid64) : kTile;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int lp = i * kThreads + tid;
        if (lp < valid) {
            const uint64_t key = s_keys[lp];
            const uint32_t dd = static_cast<uint32_t>(key >> shift) & digit_mask;
            const uint32_t dst = s_global_base[dd] + (static_cast<uint32_t>(lp) - s_local_start[dd]);
            keys_out[dst] = key;
            ids_out[dst] = s_ids[lp];
        }
    }
}

struct SortLayout {
    size_t alt_keys, alt_ids, hist, counters, status0, status1, bytes;
    int passes;
    int64_t parts;
};

SortLayout sort_layout(int64_t n, int end_bit) {
    SortLayout L{};
    L.passes = (end_bit + 7) / 8;
    L.parts = (n + kTile - 1) / kTile;
    Carver c(nullptr);
    const size_t nn = static_cast<size_t>(n > 0 ? n : 1);
    c.take<uint64_t>(nn);
    L.alt_keys = 0;
    L.alt_ids = align_up(c.used, 256);
    c.take<int32_t>(nn);
    L.hist = align_up(c.used, 256);
    c.take<uint32_t>(kMaxPasses * kRadix);
    L.counters = align_up(c.used, 256);
    c.take<uint32_t>(kMaxPasses);
    const size_t status_words = static_cast<size_t>(L.parts > 0 ? L.parts : 1) * kRadix;
    L.status0 = align_up(c.used, 256);
    c.take<uint32_t>(status_words);
    L.status1 = align_up(c.used, 256);
    c.take<uint32_t>(status_words);
    L.bytes = align_up(c.used, 256);
    return L;
}

}  // namespace

size_t sort_workspace_layout(int64_t n, int end_bit) { return sort_layout(n, end_bit).bytes; }

gs_status sort_pairs_u64(uint64_t *keys, int32_t *ids, int64_t n, int end_bit, void *workspace,
                         hipStream_t stream) {
    if (n < 2 || end_bit == 0) return ok();
    const SortLayout L = sort_layout(n, end_bit);
    char *ws = static_cast<char *>(workspace);
    uint64_t *alt_keys = reinterpret_cast<uint64_t *>(ws + L.alt_keys);
    int32_t *alt_ids = reinterpret_cast<int32_t *>(ws + L.alt_ids);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + L.hist);
    uint32_t *counters = reinterpret_cast<uint32_t *>(ws + L.counters);
    uint32_t *status[2] = {reinterpret_cast<uint32_t *>(ws + L.status0), reinterpret_cast<uint32_t *>(ws + L.status1)};
    const size_t status_words = static_cast<size_t>(L.parts) * kRadix;

    GS_HIP_TRY(fill_u32(hist, 0, kMaxPasses * kRadix, stream));
    GS_HIP_TRY(fill_u32(counters, 0, kMaxPasses, stream));
    GS_HIP_TRY(fill_u32(status[0], 0, status_words, stream));
    hipLaunchKernelGGL(histogram_kernel, dim3(static_cast<unsigned>(L.parts)), dim3(kThreads), 0, stream, keys, n,
                       L.passes, end_bit, hist);
    GS_LAUNCH_TRY("histogram_kernel");

    uint64_t *src_k = keys, *dst_k = alt_keys;
    int32_t *src_i = ids, *dst_i = alt_ids;
    for (int p = 0; p < L.passes; ++p) {
        const int shift = 8 * p;
        const int bits = end_bit - shift < 8 ? end_bit - shift : 8;
        uint32_t *st = status[p & 1];
        uint32_t *st_next = (p + 1 < L.passes) ? status[(p + 1) & 1] : nullptr;
        hipLaunchKernelGGL(onesweep_pass_kernel, dim3(static_cast<unsigned>(L.parts)), dim3(kThreads), 0, stream,
                           src_k, src_i, dst_k, dst_i, n, shift, bits, hist + p * kRadix, counters + p, st, st_next);
        GS_LAUNCH_TRY("onesweep_pass_kernel");
        uint64_t *tk = src_k;
        src_k = dst_k;
        dst_k = tk;
        int32_t *ti = src_i;
        src_i = dst_i;
        dst_i = ti;
    }
    if (src_k != keys) {
        GS_HIP_TRY(hipMemcpyAsync(keys, src_k, static_cast<size_t>(n) * sizeof(uint64_t), hipMemcpyDeviceToDevice,
                                  stream));
        GS_HIP_TRY(hipMemcpyAsync(ids, src_i, static_cast<size_t>(n) * sizeof(int32_t), hipMemcpyDeviceToDevice,
                                  stream));
    }
    return ok();
}

}  // namespace gs

using namespace gs;

extern "C" size_t gs_sort_workspace_bytes(int64_t n, int end_bit) {
    if (n < 0 || end_bit < 0 || end_bit > 64) return 0;
    return sort_layout(n, end_bit).bytes;
}

extern "C" gs_status gs_sort_keys(uint64_t *keys, int32_t *flatten_ids, int64_t n, int end_bit, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    if (n < 0 || n >= (int64_t(1) << 30))
        return fail(GS_ERR_INVALID_ARG, "gs_sort_keys: n = %lld outside [0, 2^30)", (long long)n);
    if (end_bit < 0 || end_bit > 64)
        return fail(GS_ERR_INVALID_ARG, "gs_sort_keys: end_bit = %d outside [0, 64]", end_bit);
    if (n > 0 && (!keys || !flatten_ids)) return fail(GS_ERR_INVALID_ARG, "gs_sort_keys: keys and ids are required");
    if (n < 2 || end_bit == 0) return ok();
    const size_t need = sort_layout(n, end_bit).bytes;
    if (!workspace || workspace_bytes < need)
        return fail(GS_ERR_WORKSPACE, "gs_sort_keys: needs %zu workspace bytes (got %zu)", need, workspace_bytes);
    return sort_pairs_u64(keys, flatten_ids, n, end_bit, workspace, static_cast<hipStream_t>(stream));
}

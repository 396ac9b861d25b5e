// Stable LSD radix sort of (key, int32 id) pairs on gfx950, onesweep style:
//   1. one read of the keys builds every pass's digit histogram (lanes holding consecutive keys compare digits
//      with their neighbour and only the first lane of a run of equal digits adds to the LDS histogram, so keys
//      that share digits - e.g. one splat's intersections - cost one LDS atomic per run);
//   2. one kernel per digit pass: a 16-wave workgroup takes a partition (13 or 14 x 1024 pairs for 8-byte keys,
//      taken from a counter so every predecessor is already running; 4096 for 4-byte keys, indexed by block),
//      ranks its keys stably with wave64
//      ballot matching, publishes its per-digit counts, resolves its global per-digit offsets by a decoupled
//      look-back (a window of predecessors per load round) that overlaps the LDS reorder and the id loads,
//      reorders the pairs through LDS by digit (keys first, then ids in the same LDS bytes) and writes runs of
//      consecutive addresses.
// Only bits [begin_bit, end_bit) are sorted, split evenly into passes of at most 8 bits.
//
// Semantics: gsplat 1.0.0 native extension, intersections.c, gs_radix_sort_without_gvl (a stable LSD radix sort
// of keys with their ids). Stability makes the result unique, so it is compared bit for bit.
#include "gs_sort.hpp"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace gs {
namespace {

constexpr int kRadix = 256;
constexpr int kThreads = 1024;                // digit-pass workgroup: 16 waves; threads [0, kRadix) own a digit each
constexpr int kWaves = kThreads / kWave;
constexpr int kHistThreads = kRadix;          // histogram workgroup: one thread per digit
static_assert(kThreads % kRadix == 0 && kThreads / kWave * kWave == kThreads, "digit threads are whole waves");
constexpr uint32_t kFlagAggregate = 1u << 30; // partition's own count published
constexpr uint32_t kFlagInclusive = 2u << 30; // count including every earlier partition published
constexpr uint32_t kValueMask = (1u << 30) - 1;

// Partition shape of a digit pass: Items pairs per thread of a 1024-thread workgroup. Large partitions shorten the
// look-back walks (device-coherent loads, ~1 us each under load) as long as the CU keeps 16 waves: one workgroup per
// CU with 14 pairs per thread (128 VGPRs, 130 KB of LDS) holds 14336 pairs; measured on 13M and 157M random 45/47-bit
// keys it beat 256 threads x 28 pairs (two workgroups per CU) by 12% and 16%, 512 x 14 by 3% and 13%, 768 x 18-20
// by 1-4%, and 1024 x 12 by 5%; more than 14 pairs per thread spill past 128 VGPRs. 8-byte keys take 13 or 14 pairs
// per thread, whichever leaves the fuller last round of partitions over the CUs (pass_items; 13 was 2.5% faster on
// 13M keys, 912 vs 982 partitions on 256 CUs, and 14 was 1.7% faster on 157M). Look-back windows of 2, 3 and 4 were
// within 1% (2 best). 4-byte keys sort the splats' depths (about a million, every partition in flight at once):
// 4, 6 or 8 pairs per thread and windows of 2, 3 or 4 measured the same there, wider windows slower.
template <typename KeyT, int Items>
struct Tiling {
    static constexpr int items = Items;                        // pairs per thread
    static constexpr int tile = kThreads * items;              // pairs per partition
    static constexpr int wave_span = kWave * items;            // contiguous pairs owned by one wave
    static constexpr int window = sizeof(KeyT) == 8 ? 2 : 4;   // predecessors inspected per look-back round
};
constexpr int kItems32 = 4;                  // pairs per thread for 4-byte keys
constexpr int kItems32Big = 16;              // ... from kItems32BigMin pairs on (one workgroup per CU)
constexpr int64_t kItems32BigMin = int64_t(1) << 21;
constexpr int kItems64Min = 13, kItems64Max = 14;
// the smallest partition of any shape sizes the look-back arrays (one status word per digit and partition)
constexpr int kMinTile = kThreads * (kItems32 < kItems64Min ? kItems32 : kItems64Min);
static_assert(kHistCopyWords == kMaxPasses * kRadix, "one histogram copy holds every pass's digits");
// histogram kernel: keys per thread and per workgroup step
constexpr int kHistItems = 16;
constexpr int kHistTile = kHistThreads * kHistItems;

}  // namespace

// Device-wide error word of the library (one per GPU): bit kDeviceErrSortLookBack is set by a digit pass whose
// look-back wait for a predecessor partition ran past the spin limit, bit kDeviceErrScanLookBack by a single-pass
// scan of the intersection counts in the same case. Read and cleared by gs_device_check.
__device__ uint32_t g_device_error = 0;

namespace {

// Spin limit handed to every digit pass launched after it is set (gs_set_spin_limit): look-back rounds a
// partition may wait for its predecessors before it gives up. A round is one device-coherent load of the window
// (about a microsecond under load) plus a short sleep, so the default bounds a wait by about a second, far past
// any legitimate one (a predecessor took its partition index first and is already running).
constexpr uint32_t kDefaultSpinLimit = 1u << 20;
std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};

__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t atomic_load_agent64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent64(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename KeyT>
__device__ __forceinline__ uint32_t digit_of(KeyT k, int shift, uint32_t mask) {
    return static_cast<uint32_t>(k >> shift) & mask;
}

// Exclusive prefix over the threads of the workgroup (one value each); *total = sum.
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

// histogram workgroups: 2048 up to 16384 tiles of keys, then one per 8 tiles up to 4096 (measured with the
// flushes spread over the histogram copies: 2048 read 13M keys 15% faster than 1024, and 4096 read 157M keys 19%
// faster than 1024)
constexpr int64_t kHistBlocksMin = 2048, kHistBlocksMax = 4096, kHistTilesPerBlock = 8;

// Digit histograms of every pass. Each thread holds 16 keys read lane-contiguous (consecutive lanes hold
// consecutive keys), and every pass's digits are counted by runs (wave_add_runs), so keys that share digits - one
// splat's intersections share their depth bits - cost one LDS atomic per run. Every tile but the last is full and
// is counted without the per-key bounds test.
template <typename KeyT, bool kFull>
__device__ __forceinline__ void count_tile_digits(const KeyT (&k)[kHistItems], int valid, const PassPlan &plan,
                                                  uint32_t (&s_hist)[kMaxPasses][kRadix], const RunLanes &rl) {
    for (int p = 0; p < plan.passes; ++p) {
        const int shift = plan.shift[p];
        const uint32_t mask = (1u << plan.bits[p]) - 1u;
#pragma unroll
        for (int i = 0; i < kHistItems; ++i) {
            const bool in = kFull || i * kHistThreads + static_cast<int>(threadIdx.x) < valid;
            const uint32_t d = in ? digit_of(k[i], shift, mask) : 0xffffffffu;
            wave_add_runs(s_hist[p], d, in, rl);
        }
    }
}

template <typename KeyT>
__global__ __launch_bounds__(kHistThreads) void histogram_kernel(const KeyT *__restrict__ keys, int64_t n,
                                                             PassPlan plan, uint32_t *__restrict__ hist) {
    __shared__ uint32_t s_hist[kMaxPasses][kRadix];
    for (int p = 0; p < plan.passes; ++p) s_hist[p][threadIdx.x] = 0;
    const RunLanes rl = run_lanes();
    const int64_t tiles = (n + kHistTile - 1) / kHistTile;
    __syncthreads();
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int64_t base = tile * kHistTile;
        const int valid = n - base < kHistTile ? static_cast<int>(n - base) : kHistTile;
        KeyT k[kHistItems];
#pragma unroll
        for (int i = 0; i < kHistItems; ++i) {
            const int q = i * kHistThreads + threadIdx.x;
            k[i] = q < valid ? keys[base + q] : KeyT(0);
        }
        if (valid == kHistTile)
            count_tile_digits<KeyT, true>(k, valid, plan, s_hist, rl);
        else
            count_tile_digits<KeyT, false>(k, valid, plan, s_hist, rl);
    }
    __syncthreads();
    uint32_t *copy = hist_copy(hist, blockIdx.x);
    for (int p = 0; p < plan.passes; ++p) {
        const uint32_t c = s_hist[p][threadIdx.x];
        if (c) atomicAdd(&copy[p * kRadix + threadIdx.x], c);
    }
}

// Global start of every digit bucket of every pass: for pass p and digit d, the number of keys whose digit p is
// below d, summed over the histogram copies. One workgroup of 256 threads per pass (blockIdx.x = p), one thread per
// digit; computed once per sort, so a digit pass's partitions only load their digit's start (off their critical
// path) instead of each summing the copies and scanning them. With counters non-null the step also readies the
// scratch for the next sort: it zeroes the histogram entries it has read and resets pass p's partition counter.
__global__ __launch_bounds__(kRadix) void digit_starts_kernel(uint32_t *__restrict__ hist,
                                                          uint32_t *__restrict__ starts,
                                                          uint32_t *__restrict__ counters) {
    __shared__ uint32_t s_w[kRadix / kWave];
    const int p = blockIdx.x, d = threadIdx.x, wave = d / kWave, lane = __lane_id();
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kHistCopies; ++k) c += hist[k * kHistCopyWords + p * kRadix + d];
    if (counters) {
#pragma unroll
        for (int k = 0; k < kHistCopies; ++k) hist[k * kHistCopyWords + p * kRadix + d] = 0;
        if (d == 0) counters[p] = 0;
    }
    const uint32_t inc = wave_inclusive_sum(c);
    if (lane == kWave - 1) s_w[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kRadix / kWave; ++w) before += w < wave ? s_w[w] : 0u;
    starts[p * kRadix + d] = before + inc - c;
}

// Stable rank of each of a wave's items among the wave's items of the same digit (digit_bits bits at shift), item
// i of every lane coming after items 0..i-1 of all lanes and after item i of lower lanes; wave_hist (this wave's
// LDS counts per digit, zero before the first call) advances by the wave's count of each digit. The lanes holding
// the same digit come from one ballot per digit bit: a lane's mismatch set gathers, for every bit, the lanes whose
// bit differs from its own (ballot XOR the lane's bit spread over 32 bits, ORed in by one three-input bit operation
// per half of the 64-lane mask); its complement is the set of lanes with the same digit.
template <typename KeyT, int kItems, int kDigitBits>
__device__ __forceinline__ void rank_in_wave(const KeyT (&k)[kItems], int shift, uint32_t *wave_hist,
                                             uint32_t (&rank)[kItems]) {
    const int lane = __lane_id();
    const uint32_t digit_mask = (1u << kDigitBits) - 1u;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const uint32_t d = digit_of(k[i], shift, digit_mask);
        uint32_t miss_lo = 0u, miss_hi = 0u;
#pragma unroll
        for (int b = 0; b < kDigitBits; ++b) {
            const uint32_t spread = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(d), b, 1));
            const uint64_t ballot = __ballot(spread != 0u);
            // truth table 0xF6: first | (second ^ third), the first operand being the table's high index bit
            miss_lo = __builtin_amdgcn_bitop3_b32(miss_lo, static_cast<uint32_t>(ballot), spread, 0xF6);
            miss_hi = __builtin_amdgcn_bitop3_b32(miss_hi, static_cast<uint32_t>(ballot >> 32), spread, 0xF6);
        }
        const uint32_t same_lo = ~miss_lo, same_hi = ~miss_hi;
        const uint64_t same = (static_cast<uint64_t>(same_hi) << 32) | same_lo;
        const uint32_t below = static_cast<uint32_t>(__popcll(same & lt_mask));
        const uint32_t run = wave_hist[d];
        rank[i] = run + below;
        const int leader = 63 - __clzll(same);
        if (lane == leader) wave_hist[d] = run + static_cast<uint32_t>(__popcll(same));
    }
}

// One digit pass. Partition `part` covers pairs [part * kTile, part * kTile + kTile) (kTile from Tiling);
// wave w owns the contiguous span [w * kWaveSpan, (w + 1) * kWaveSpan) of it, item i of lane l sitting at
// w * kWaveSpan + i * 64 + l, so (wave, item, lane) order is input order and the per-wave running counts give a
// stable rank.
// ids_in == nullptr means the identity (id = input position). status[part][d] holds this pass's look-back
// words; status_next[part][d] is cleared for the next pass. kStream: the pass reads its keys and ids with
// non-temporal loads (see stream_loads).
template <typename KeyT, int kDigitBits, int kPassItems, bool kStream>
__global__ __launch_bounds__(kThreads) void onesweep_pass_kernel(
    const KeyT *__restrict__ keys_in, const int32_t *__restrict__ ids_in, KeyT *__restrict__ keys_out,
    int32_t *__restrict__ ids_out, int64_t n, int shift, const uint32_t *__restrict__ digit_starts,
    uint32_t *__restrict__ part_counter, uint32_t *status, uint32_t *__restrict__ status_next,
    uint32_t spin_limit) {
    constexpr int digit_bits = kDigitBits;
    using T = Tiling<KeyT, kPassItems>;
    constexpr int kItems = T::items, kTile = T::tile, kWaveSpan = T::wave_span;
    constexpr int kLookWindow = T::window;
    __shared__ union {
        KeyT keys[kTile];
        int32_t ids[kTile];
    } s_buf;
    __shared__ uint32_t s_wave_hist[kWaves][kRadix];
    __shared__ uint32_t s_local_start[kRadix];
    __shared__ uint32_t s_global_base[kRadix];
    __shared__ uint32_t s_tmp[kWaves];
    __shared__ uint32_t s_part;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = __lane_id();
    const uint32_t digit_mask = (1u << digit_bits) - 1u;

    // The partition index. Passes over 8-byte keys (one workgroup per CU) take the next index from a counter, so the
    // look-back chain follows the order in which workgroups actually start; indexed by block instead, the 45-bit
    // sort of 13M pairs took 0.53 ms against 0.50. Passes over 4-byte keys (several workgroups per CU) index by
    // block and save the counter's round trip: the depth sort of 6M splats ran 5% faster. Workgroups start in
    // block order on each XCD, so every predecessor of a running partition is running or done, and the bounded
    // look-back below turns any violation of that into a reported error rather than a hang.
    constexpr bool kByBlock = sizeof(KeyT) == 4;
    uint32_t part;
    if constexpr (kByBlock) {
        part = blockIdx.x;
    } else {
        if (tid == 0) s_part = atomicAdd(part_counter, 1u);
        for (int i = tid; i < kWaves * kRadix; i += kThreads) (&s_wave_hist[0][0])[i] = 0;
        __syncthreads();
        part = __builtin_amdgcn_readfirstlane(s_part);  // uniform: the load paths below branch on it
    }
    // the host launches exactly one workgroup per partition; a counter left inconsistent by a corrupted workspace
    // must not address past the arrays (the result is then wrong, but every access stays in bounds)
    if (static_cast<int64_t>(part) * kTile >= n) return;
    // threads [0, kRadix) own digit d = tid for the per-digit steps; the other waves only rank and move pairs
    const bool digit_thread = tid < kRadix;
    const int d = digit_thread ? tid : 0;

    // load this wave's span of keys (ids are loaded after the keys are written, to keep registers free)
    const int64_t base = static_cast<int64_t>(part) * kTile + static_cast<int64_t>(wave) * kWaveSpan + lane;
    const bool full = static_cast<int64_t>(part + 1) * kTile <= n;
    // Both kinds of partition issue the same kItems loads in the same order (a partial one clamps its addresses to
    // the last pair, then replaces what lies past the end), so the ranking of each item waits for its own load
    // only, not for the whole span.
    KeyT k[kItems];
    if (full) {
#pragma unroll
        for (int i = 0; i < kItems; ++i)
            k[i] = kStream ? __builtin_nontemporal_load(keys_in + base + i * kWave) : keys_in[base + i * kWave];
    } else {
#pragma unroll
        for (int i = 0; i < kItems; ++i) {
            const int64_t pos = base + i * kWave;
            k[i] = keys_in[pos < n ? pos : n - 1];
        }
    }
    if constexpr (kByBlock) {  // the keys are already requested
        for (int i = tid; i < kWaves * kRadix; i += kThreads) (&s_wave_hist[0][0])[i] = 0;
        __syncthreads();
    }
    if (!full) {
#pragma unroll
        for (int i = 0; i < kItems; ++i)
            if (base + i * kWave >= n) k[i] = ~KeyT(0);  // past the end: largest digit, ranked after every real pair
    }
    // issued after the key loads, so that nothing waits for them before the keys are requested
    if (status_next && digit_thread) status_next[static_cast<size_t>(part) * kRadix + d] = 0;
    // global start of this thread's digit bucket for the pass (precomputed once per sort); used only when the
    // pairs are written, so its load is in flight with the key loads
    const uint32_t digit_global_start = digit_thread ? digit_starts[d] : 0u;


    uint32_t rank[kItems];
    rank_in_wave<KeyT, kItems, digit_bits>(k, shift, s_wave_hist[wave], rank);
    __syncthreads();

    // per digit (thread d): counts of the waves -> exclusive prefix over waves, and the partition total
    uint32_t running = 0;
    if (digit_thread) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = s_wave_hist[w][d];
            s_wave_hist[w][d] = running;
            running += c;
        }
    }
    const uint32_t part_count = running;
    uint32_t *my_status = status + static_cast<size_t>(part) * kRadix + d;
    if (digit_thread) atomic_store_agent(my_status, (part == 0 ? kFlagInclusive : kFlagAggregate) | part_count);

    // issue the first look-back window now; its round trip overlaps the local reorder and the id loads below
    uint32_t s[kLookWindow];
    int64_t j = static_cast<int64_t>(part) - 1;
#pragma unroll
    for (int w = 0; w < kLookWindow; ++w)
        s[w] = (digit_thread && j - w >= 0) ? atomic_load_agent(status + static_cast<size_t>(j - w) * kRadix + d)
                                            : kFlagInclusive;

    uint32_t local_total;
    const uint32_t local_start = block_exclusive_u32(part_count, s_tmp, &local_total);
    if (digit_thread) s_local_start[d] = local_start;
    __syncthreads();

    // reorder the partition's keys by digit through LDS (local positions need no global offsets)
    uint32_t lp[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const uint32_t dd = digit_of(k[i], shift, digit_mask);
        lp[i] = s_local_start[dd] + s_wave_hist[wave][dd] + rank[i];
        s_buf.keys[lp[i]] = k[i];
    }
    // decoupled look-back for digit d: walk back over the predecessors' published counts, a window of kLookWindow
    // at a time, until one carries an inclusive count (partition 0 always does). The wait is bounded: after
    // spin_limit rounds without finding one the partition gives up, flags the device error word and publishes
    // what it has, so that every later partition also finishes (the pass's output is then invalid, and every
    // write still stays inside the arrays).
    // Adds the window's published counts up to the first unpublished word or the inclusive one; `used` = words
    // consumed, the result = whether an inclusive count was among them.
    auto consume = [&](uint32_t &sum, int &used) {
        bool found = false;
        used = 0;
#pragma unroll
        for (int w = 0; w < kLookWindow; ++w) {
            if (found || used < w) continue;
            const uint32_t flag = s[w] & ~kValueMask;
            if (flag == 0) continue;
            sum += s[w] & kValueMask;
            used = w + 1;
            if (flag == kFlagInclusive) found = true;
        }
        return found;
    };
    uint32_t before = 0;
    const bool looks_back = part > 0 && digit_thread;
    int used = 0;
    // The first window (requested before the local scan) is inspected before the ids are requested, so that this
    // inspection waits for the status words only; a wait placed after the id loads would also wait for them.
    bool found = !looks_back || consume(before, used);

    // the ids travel with the keys; load them while the rest of the look-back is in flight
    int32_t v[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t pos = base + i * kWave;
        if (ids_in) v[i] = (full || pos < n) ? (kStream ? __builtin_nontemporal_load(ids_in + pos) : ids_in[pos]) : 0;
        else v[i] = static_cast<int32_t>(pos);
    }

    if (looks_back) {
        uint32_t rounds = 0;
        while (!found) {
            if (rounds++ >= spin_limit) {
                atomicOr(&g_device_error, kDeviceErrSortLookBack);
                break;
            }
            j -= used;
            if (used < kLookWindow) __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int w = 0; w < kLookWindow; ++w)
                s[w] = (j - w >= 0) ? atomic_load_agent(status + static_cast<size_t>(j - w) * kRadix + d)
                                    : kFlagInclusive;
            found = consume(before, used);
        }
        atomic_store_agent(my_status, kFlagInclusive | (before + part_count));
    }
    if (digit_thread) s_global_base[d] = digit_global_start + before;
    __syncthreads();

    // write keys: consecutive local positions of one digit go to consecutive global positions
    const int64_t valid64 = n - static_cast<int64_t>(part) * kTile;
    const int valid = valid64 < kTile ? static_cast<int>(valid64) : kTile;
    uint32_t dst[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int q = i * kThreads + tid;
        const KeyT key = s_buf.keys[q];
        const uint32_t dd = digit_of(key, shift, digit_mask);
        dst[i] = s_global_base[dd] + (static_cast<uint32_t>(q) - s_local_start[dd]);
        // dst < n always holds when the histogram matches the keys; the test keeps a corrupted one in bounds
        if ((full || q < valid) && dst[i] < n) keys_out[dst[i]] = key;
    }
    // the ids follow through the same LDS bytes
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) s_buf.ids[lp[i]] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int q = i * kThreads + tid;
        if ((full || q < valid) && dst[i] < n) ids_out[dst[i]] = s_buf.ids[q];
    }
}

// The last pass of the splats' depth sort (4-byte keys, 8-bit digits, partitions indexed by block), which also
// produces what the emission reads in depth order: besides the sorted (key, id) pairs, for every output position
// the rectangle of its splat (gathered by id from rects, which is in splat order: int4, or one packed word when
// pk.cx is nonzero, which keeps the gathered array small enough to stay mostly in L2) and the splat's first output
// slot, the sum of the tile counts (width x height of the rectangles) of every splat placed before it. That sum has
// three parts: the counts of the splats whose digit is smaller (weight_starts: the exclusive scan over digits of a
// histogram of counts by this pass's digit), of the earlier partitions' splats with the same digit (the look-back,
// whose words carry each partition's count sum beside its key count), and of the partition's own earlier splats
// with that digit (an exclusive scan of the counts in the partition's reordered sequence). A 64-bit status word
// holds 2 flag bits, the count sum in bits [30, 62) and the key count in bits [0, 30); both fields add as one
// integer while the counts stay below 2^30 keys and 2^32 tiles, and the flags are masked off every published sum.
constexpr uint64_t kFlag64Aggregate = 1ull << 62;
constexpr uint64_t kFlag64Inclusive = 2ull << 62;
constexpr uint64_t kValue64Mask = (1ull << 62) - 1;
constexpr int kPackShift = 30;
constexpr uint64_t kPackKeysMask = (1ull << kPackShift) - 1;

__global__ __launch_bounds__(kThreads) void depth_order_pass_kernel(
    const uint32_t *__restrict__ keys_in, const int32_t *__restrict__ ids_in, const void *__restrict__ rects,
    RectPacking pk, uint32_t *__restrict__ keys_out, int32_t *__restrict__ ids_out, void *__restrict__ sorted_rects,
    int32_t *__restrict__ sorted_offsets, int64_t n, int shift, const uint32_t *__restrict__ digit_starts,
    const uint32_t *__restrict__ weight_starts, uint64_t *status, uint32_t spin_limit) {
    constexpr int kItems = kItems32, kTile = kThreads * kItems, kWaveSpan = kWave * kItems;
    constexpr int kLookWindow = 4;
    constexpr uint32_t kMask = kRadix - 1;
    __shared__ union {
        uint32_t keys[kTile];
        int32_t ids[kTile];
    } s_buf;
    // tile counts in the partition's reordered sequence, then their exclusive prefix (entry kTile: the total)
    __shared__ union {
        uint4 quad[kTile / 4 + 1];
        uint32_t word[kTile + 4];
    } s_count;
    __shared__ union {
        int4 full[kTile];
        uint32_t packed[kTile];
    } s_rect;
    __shared__ uint32_t s_wave_hist[kWaves][kRadix];
    __shared__ uint32_t s_local_start[kRadix];
    __shared__ uint32_t s_global_base[kRadix];
    __shared__ uint32_t s_count_base[kRadix];
    __shared__ uint32_t s_tmp[kWaves];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = __lane_id();
    const uint32_t part = blockIdx.x;
    if (static_cast<int64_t>(part) * kTile >= n) return;
    const bool digit_thread = tid < kRadix;
    const int d = digit_thread ? tid : 0;
    const int64_t base = static_cast<int64_t>(part) * kTile + static_cast<int64_t>(wave) * kWaveSpan + lane;
    const bool full = static_cast<int64_t>(part + 1) * kTile <= n;

    // keys and ids at once; the ids address the gather of the rectangles, issued as soon as they arrive
    uint32_t k[kItems];
    int32_t v[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int64_t at = base + i * kWave < n ? base + i * kWave : n - 1;
        k[i] = keys_in[at];
        v[i] = ids_in[at];
    }
    for (int i = tid; i < kWaves * kRadix; i += kThreads) (&s_wave_hist[0][0])[i] = 0;
    // a position past the end, and an id outside [0, n) (only from a corrupted workspace), take an empty rectangle
    // (packed: the zero word)
    int4 r[kItems];
    uint32_t rp[kItems];
    const bool packed = pk.cx != 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const bool real = (full || base + i * kWave < n) && static_cast<uint64_t>(v[i]) < static_cast<uint64_t>(n);
        if (packed) rp[i] = real ? static_cast<const uint32_t *>(rects)[v[i]] : 0u;
        else r[i] = real ? static_cast<const int4 *>(rects)[v[i]] : make_int4(0, 0, 0, 0);
    }
    __syncthreads();
    if (!full) {
#pragma unroll
        for (int i = 0; i < kItems; ++i)
            if (base + i * kWave >= n) k[i] = ~0u;  // past the end: largest digit, ranked after every real pair
    }
    const uint32_t digit_global_start = digit_thread ? digit_starts[d] : 0u;
    const uint32_t digit_count_start = digit_thread ? weight_starts[d] : 0u;

    uint32_t rank[kItems];
    rank_in_wave<uint32_t, kItems, 8>(k, shift, s_wave_hist[wave], rank);
    __syncthreads();
    uint32_t running = 0;
    if (digit_thread) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = s_wave_hist[w][d];
            s_wave_hist[w][d] = running;
            running += c;
        }
    }
    const uint32_t part_keys = running;
    uint32_t local_total;
    const uint32_t local_start = block_exclusive_u32(part_keys, s_tmp, &local_total);
    if (digit_thread) s_local_start[d] = local_start;
    __syncthreads();

    // reorder keys, rectangles and tile counts by digit through LDS
    uint32_t lp[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const uint32_t dd = (k[i] >> shift) & kMask;
        lp[i] = s_local_start[dd] + s_wave_hist[wave][dd] + rank[i];
        s_buf.keys[lp[i]] = k[i];
        if (packed) {
            s_rect.packed[lp[i]] = rp[i];
            const int4 u = unpack_rect(rp[i], pk);
            s_count.word[lp[i]] = static_cast<uint32_t>(u.z) * static_cast<uint32_t>(u.w);
        } else {
            s_rect.full[lp[i]] = r[i];
            // a rectangle from a workspace the count scan did not fill still counts >= 0
            s_count.word[lp[i]] = static_cast<uint32_t>(max(r[i].z, 0)) * static_cast<uint32_t>(max(r[i].w, 0));
        }
    }
    __syncthreads();
    // exclusive prefix of the counts in reordered sequence: thread t takes positions 4t .. 4t + 3
    {
        const uint4 c = s_count.quad[tid];
        uint32_t total;
        const uint32_t before_t = block_exclusive_u32(c.x + c.y + c.z + c.w, s_tmp, &total);
        s_count.quad[tid] = make_uint4(before_t, before_t + c.x, before_t + c.x + c.y, before_t + c.x + c.y + c.z);
        if (tid == 0) s_count.word[kTile] = total;
    }
    __syncthreads();

    // per digit: publish the key count and count sum, then find those of all earlier partitions by a decoupled
    // look-back (a window of predecessors per round, bounded by spin_limit as in the other passes)
    uint64_t mine = 0;
    if (digit_thread) {
        const uint32_t sum = s_count.word[local_start + part_keys] - s_count.word[local_start];
        mine = (static_cast<uint64_t>(sum) << kPackShift) | part_keys;
        atomic_store_agent64(status + static_cast<size_t>(part) * kRadix + d,
                             (part == 0 ? kFlag64Inclusive : kFlag64Aggregate) | mine);
    }
    uint64_t before = 0;
    if (digit_thread && part > 0) {
        int64_t j = static_cast<int64_t>(part) - 1;  // the newest predecessor not yet added
        uint32_t rounds = 0;
        while (true) {
            uint64_t s[kLookWindow];
#pragma unroll
            for (int w = 0; w < kLookWindow; ++w)
                s[w] = j - w >= 0 ? atomic_load_agent64(status + static_cast<size_t>(j - w) * kRadix + d)
                                  : kFlag64Inclusive;
            // add the window's published words up to the first unpublished one, or through the inclusive one
            bool found = false;
            int used = 0;
#pragma unroll
            for (int w = 0; w < kLookWindow; ++w) {
                if (found || used < w) continue;
                const uint64_t flag = s[w] & ~kValue64Mask;
                if (flag == 0) continue;
                before += s[w] & kValue64Mask;
                used = w + 1;
                if (flag == kFlag64Inclusive) found = true;
            }
            if (found) break;
            if (rounds++ >= spin_limit) {
                atomicOr(&g_device_error, kDeviceErrSortLookBack);
                break;
            }
            j -= used;
            if (used < kLookWindow) __builtin_amdgcn_s_sleep(1);
        }
        atomic_store_agent64(status + static_cast<size_t>(part) * kRadix + d,
                             kFlag64Inclusive | ((before + mine) & kValue64Mask));
    }
    if (digit_thread) {
        s_global_base[d] = digit_global_start + static_cast<uint32_t>(before & kPackKeysMask);
        s_count_base[d] = digit_count_start + static_cast<uint32_t>(before >> kPackShift);
    }
    __syncthreads();

    // keys, rectangles and first slots: consecutive local positions of one digit go to consecutive positions
    const int64_t valid64 = n - static_cast<int64_t>(part) * kTile;
    const int valid = valid64 < kTile ? static_cast<int>(valid64) : kTile;
    uint32_t dst[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int q = i * kThreads + tid;
        const uint32_t key = s_buf.keys[q];
        const uint32_t dd = (key >> shift) & kMask;
        const uint32_t ls = s_local_start[dd];
        dst[i] = s_global_base[dd] + (static_cast<uint32_t>(q) - ls);
        // dst < n always holds when the histograms match the keys; the test keeps a corrupted one in bounds
        if ((full || q < valid) && dst[i] < n) {
            keys_out[dst[i]] = key;
            if (packed) static_cast<uint32_t *>(sorted_rects)[dst[i]] = s_rect.packed[q];
            else static_cast<int4 *>(sorted_rects)[dst[i]] = s_rect.full[q];
            sorted_offsets[dst[i]] = static_cast<int32_t>(s_count_base[dd] + (s_count.word[q] - s_count.word[ls]));
        }
    }
    // the ids follow through the keys' LDS bytes
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) s_buf.ids[lp[i]] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int q = i * kThreads + tid;
        if ((full || q < valid) && dst[i] < n) ids_out[dst[i]] = s_buf.ids[q];
    }
}

}  // namespace

PassPlan make_pass_plan(int begin_bit, int end_bit) {
    PassPlan plan{};
    const int total = end_bit - begin_bit;
    if (total <= 0) return plan;
    plan.passes = (total + 7) / 8;
    const int base = total / plan.passes, extra = total % plan.passes;
    int shift = begin_bit;
    for (int p = 0; p < plan.passes; ++p) {
        plan.shift[p] = shift;
        plan.bits[p] = base + (p < extra ? 1 : 0);
        shift += plan.bits[p];
    }
    return plan;
}

SortScratchLayout sort_scratch_layout(int64_t n) {
    SortScratchLayout L{};
    L.parts = (n + kMinTile - 1) / kMinTile;
    Carver c(nullptr);
    L.hist = 0;
    c.take<uint32_t>(static_cast<size_t>(kHistCopies) * kHistCopyWords);
    L.counters = align_up(c.used, 256);
    c.take<uint32_t>(kMaxPasses);
    const size_t status_words = static_cast<size_t>(L.parts > 0 ? L.parts : 1) * kRadix;
    L.status0 = align_up(c.used, 256);
    c.take<uint32_t>(status_words);
    L.status1 = align_up(c.used, 256);
    c.take<uint32_t>(status_words);
    L.starts = align_up(c.used, 256);
    c.take<uint32_t>(static_cast<size_t>(kMaxPasses) * kRadix);
    L.bytes = align_up(c.used, 256);
    return L;
}

gs_status radix_prepare(int64_t n, void *scratch, hipStream_t stream) {
    // histograms, counters and the first look-back array are consecutive: one fill clears all three
    GS_HIP_TRY(fill_u32(static_cast<uint32_t *>(scratch), 0, radix_clear_bytes(n) / sizeof(uint32_t), stream));
    return ok();
}

size_t radix_clear_bytes(int64_t n) {
    const SortScratchLayout L = sort_scratch_layout(n);
    return L.status0 + static_cast<size_t>(L.parts) * kRadix * sizeof(uint32_t);
}

uint32_t *radix_histograms(void *scratch, int64_t n) {
    return reinterpret_cast<uint32_t *>(static_cast<char *>(scratch) + sort_scratch_layout(n).hist);
}

SortScratch sort_scratch(void *scratch, int64_t n) {
    const SortScratchLayout L = sort_scratch_layout(n);
    char *ws = static_cast<char *>(scratch);
    return SortScratch{reinterpret_cast<uint32_t *>(ws + L.hist), reinterpret_cast<uint32_t *>(ws + L.counters),
                       reinterpret_cast<uint32_t *>(ws + L.status0), reinterpret_cast<uint32_t *>(ws + L.status1),
                       reinterpret_cast<uint32_t *>(ws + L.starts), L.parts};
}

size_t sort_scratch_head_bytes() { return sort_scratch_layout(1).status0; }

size_t sort_scratch_tail_bytes(int64_t n) {
    const SortScratchLayout L = sort_scratch_layout(n);
    return L.bytes - L.status0;
}

SortScratch sort_scratch_split(void *head, void *tail, int64_t n) {
    const SortScratchLayout L = sort_scratch_layout(n);
    char *h = static_cast<char *>(head), *t = static_cast<char *>(tail) - L.status0;
    return SortScratch{reinterpret_cast<uint32_t *>(h + L.hist), reinterpret_cast<uint32_t *>(h + L.counters),
                       reinterpret_cast<uint32_t *>(t + L.status0), reinterpret_cast<uint32_t *>(t + L.status1),
                       reinterpret_cast<uint32_t *>(t + L.starts), L.parts};
}

template <typename KeyT>
gs_status radix_sort_pairs(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                           KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan, void *scratch,
                           hipStream_t stream, int *result_in_b) {
    *result_in_b = 0;
    if (plan.passes == 0 || n < 1) return ok();
    gs_status st = radix_prepare(n, scratch, stream);
    if (st != GS_OK) return st;
    // a few workgroups per CU, each striding over several tiles, so that the per-workgroup flushes into the
    // histogram copies stay few (contended device-scope atomics dominate when every tile flushes its own)
    const int64_t hist_tiles = (n + kHistTile - 1) / kHistTile;
    const int64_t want = std::min(kHistBlocksMax, std::max(kHistBlocksMin, hist_tiles / kHistTilesPerBlock));
    const unsigned hist_blocks = static_cast<unsigned>(hist_tiles < want ? hist_tiles : want);
    hipLaunchKernelGGL(histogram_kernel<KeyT>, dim3(hist_blocks), dim3(kHistThreads), 0, stream,
                       keys_in, n, plan, radix_histograms(scratch, n));
    GS_LAUNCH_TRY("histogram_kernel");
    return radix_passes<KeyT>(keys_in, ids_in, buf_a_keys, buf_a_ids, buf_b_keys, buf_b_ids, n, plan, scratch, stream,
                              result_in_b);
}

// Whether the passes over n pairs read them with non-temporal loads: for 8-byte keys up to 2^25 pairs (12 bytes
// each, 402 MB per buffer). A pass's reads then do not displace the pairs the previous pass has just written from
// the caches, so more of them are still there when this pass's successor reads them. Measured on random 45-bit
// keys, whole sort: 6% faster at 13M pairs, 10% at 20M, 3% at 32M, and 1% slower at 38M, 4-6% slower at 44-192M
// (the crossover lies between 32M and 38M); 4-byte keys (1-6M depth keys) within 1% either way, so they stay plain.
template <typename KeyT>
bool stream_loads(int64_t n) {
    return sizeof(KeyT) == 8 && n <= (int64_t(1) << 25);
}

// Launches one digit pass of `bits` bits with Items pairs per thread.
template <typename KeyT, int Items>
gs_status launch_pass(int bits, dim3 grid, hipStream_t stream, const KeyT *src_k, const int32_t *src_i, KeyT *dk,
                      int32_t *di, int64_t n, int shift, const uint32_t *starts, uint32_t *counter, uint32_t *status,
                      uint32_t *status_next, uint32_t spin) {
    const bool nt = stream_loads<KeyT>(n);
    switch (bits) {
#define GS_PASS(B)                                                                                                  \
    case B:                                                                                                         \
        if (nt)                                                                                                     \
            hipLaunchKernelGGL((onesweep_pass_kernel<KeyT, B, Items, sizeof(KeyT) == 8>), grid, dim3(kThreads), 0, \
                               stream, src_k, src_i, dk, di, n, shift, starts, counter, status, status_next, spin); \
        else                                                                                                        \
            hipLaunchKernelGGL((onesweep_pass_kernel<KeyT, B, Items, false>), grid, dim3(kThreads), 0, stream,     \
                               src_k, src_i, dk, di, n, shift, starts, counter, status, status_next, spin);         \
        return ok();
        GS_PASS(1) GS_PASS(2) GS_PASS(3) GS_PASS(4) GS_PASS(5) GS_PASS(6) GS_PASS(7) GS_PASS(8)
#undef GS_PASS
        default: return fail(GS_ERR_INVALID_ARG, "radix pass of %d bits", bits);
    }
}

// Pairs per thread of the digit passes over n pairs: for 4-byte keys 4, or 16 from 2^21 pairs on (fewer, larger
// partitions shorten the look-back once there are several rounds of them); for 8-byte keys the one of 13 and 14
// whose partitions fill the CUs' last round best (cost: rounds of partitions over the CUs times the per-partition
// work, counted as items plus 3 for the fixed steps of a partition; ties go to 14).
template <typename KeyT>
int pass_items(int64_t n) {
    if (sizeof(KeyT) == 4) return n >= kItems32BigMin ? kItems32Big : kItems32;
    static std::atomic<int> cus{0};
    int c = cus.load(std::memory_order_relaxed);
    if (c <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                   hipSuccess || c <= 0) {
            (void)hipGetLastError();
            c = 256;
        }
        cus.store(c, std::memory_order_relaxed);
    }
    int best = kItems64Max;
    int64_t best_cost = -1;
    for (int items = kItems64Max; items >= kItems64Min; --items) {
        const int64_t parts = (n + int64_t(kThreads) * items - 1) / (int64_t(kThreads) * items);
        const int64_t cost = (parts + c - 1) / c * (items + 3);
        if (best_cost < 0 || cost < best_cost) {
            best = items;
            best_cost = cost;
        }
    }
    return best;
}

template <typename KeyT>
int64_t radix_partitions(int64_t n) {
    const int64_t tile = int64_t(kThreads) * pass_items<KeyT>(n);
    return (n + tile - 1) / tile;
}
template int64_t radix_partitions<uint32_t>(int64_t);
template int64_t radix_partitions<uint64_t>(int64_t);

namespace {

// Digit passes [0, count) of plan (count <= plan.passes), after digit_starts_kernel: pass p reads the previous
// pass's output (the input for p = 0) and writes buffer A when p is even, B when odd. Each pass clears the look-back
// array of the next pass it runs; the pass at count - 1 clears none.
template <typename KeyT>
gs_status run_digit_passes(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                           KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan, int count,
                           const SortScratch &S, hipStream_t stream) {
    uint32_t *counters = S.counters;
    uint32_t *status[2] = {S.status0, S.status1};
    const uint32_t *starts = S.starts;
    const KeyT *src_k = keys_in;
    const int32_t *src_i = ids_in;
    const uint32_t spin = spin_limit();
    const int items = pass_items<KeyT>(n);
    for (int p = 0; p < count; ++p) {
        const bool to_a = (p % 2) == 0;
        KeyT *dk = to_a ? buf_a_keys : buf_b_keys;
        int32_t *di = to_a ? buf_a_ids : buf_b_ids;
        uint32_t *st = status[p & 1];
        uint32_t *st_next = (p + 1 < count) ? status[(p + 1) & 1] : nullptr;
        const int64_t tile = int64_t(kThreads) * items;
        const int64_t parts = (n + tile - 1) / tile;
        if (parts > S.parts)  // the look-back arrays hold S.parts partitions of 256 words
            return fail(GS_ERR_INVALID_ARG, "radix pass: %lld partitions exceed the look-back arrays (%lld)",
                        (long long)parts, (long long)S.parts);
        const dim3 grid(static_cast<unsigned>(parts));
        const uint32_t *h = starts + p * kRadix;
        gs_status st_launch;
        if constexpr (sizeof(KeyT) == 4) {
            if (items == kItems32Big)
                st_launch = launch_pass<KeyT, kItems32Big>(plan.bits[p], grid, stream, src_k, src_i, dk, di, n,
                                                           plan.shift[p], h, counters + p, st, st_next, spin);
            else
                st_launch = launch_pass<KeyT, kItems32>(plan.bits[p], grid, stream, src_k, src_i, dk, di, n,
                                                        plan.shift[p], h, counters + p, st, st_next, spin);
        } else if (items == kItems64Min) {
            st_launch = launch_pass<KeyT, kItems64Min>(plan.bits[p], grid, stream, src_k, src_i, dk, di, n,
                                                       plan.shift[p], h, counters + p, st, st_next, spin);
        } else {
            st_launch = launch_pass<KeyT, kItems64Max>(plan.bits[p], grid, stream, src_k, src_i, dk, di, n,
                                                       plan.shift[p], h, counters + p, st, st_next, spin);
        }
        if (st_launch != GS_OK) return st_launch;
        GS_LAUNCH_TRY("onesweep_pass_kernel");
        src_k = dk;
        src_i = di;
    }
    return ok();
}

// The global digit starts of `rows` rows of the histogram copies (one workgroup per row); with recycle, the rows
// read are zeroed and the partition counters of those passes reset.
gs_status launch_digit_starts(const SortScratch &S, int rows, bool recycle, hipStream_t stream) {
    hipLaunchKernelGGL(digit_starts_kernel, dim3(rows), dim3(kRadix), 0, stream, S.hist, S.starts,
                       recycle ? S.counters : nullptr);
    GS_LAUNCH_TRY("digit_starts_kernel");
    return ok();
}

template <typename KeyT>
gs_status passes_after_histograms(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                                  KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan,
                                  const SortScratch &S, bool recycle, hipStream_t stream, int *result_in_b) {
    *result_in_b = 0;
    if (plan.passes == 0 || n < 1) return ok();
    gs_status st = launch_digit_starts(S, plan.passes, recycle, stream);
    if (st != GS_OK) return st;
    st = run_digit_passes<KeyT>(keys_in, ids_in, buf_a_keys, buf_a_ids, buf_b_keys, buf_b_ids, n, plan, plan.passes,
                                S, stream);
    if (st != GS_OK) return st;
    *result_in_b = (plan.passes % 2) == 0;
    return ok();
}

}  // namespace

template <typename KeyT>
gs_status radix_passes(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                       KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan, void *scratch,
                       hipStream_t stream, int *result_in_b) {
    return passes_after_histograms<KeyT>(keys_in, ids_in, buf_a_keys, buf_a_ids, buf_b_keys, buf_b_ids, n, plan,
                                         sort_scratch(scratch, n), false, stream, result_in_b);
}

template <typename KeyT>
gs_status radix_passes(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                       KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan,
                       const SortScratch &scratch, hipStream_t stream, int *result_in_b) {
    return passes_after_histograms<KeyT>(keys_in, ids_in, buf_a_keys, buf_a_ids, buf_b_keys, buf_b_ids, n, plan,
                                         scratch, true, stream, result_in_b);
}

size_t depth_order_status_bytes(int64_t n) {
    const int64_t parts = (n + kThreads * kItems32 - 1) / (kThreads * kItems32);
    return static_cast<size_t>(parts > 0 ? parts : 1) * kRadix * sizeof(uint64_t);
}

gs_status depth_order_passes(const uint32_t *depth_bits, uint32_t *buf_a_keys, int32_t *buf_a_ids,
                             uint32_t *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan,
                             void *scratch, const void *rects, void *sorted_rects, RectPacking pk,
                             int32_t *sorted_offsets, uint64_t *order_status, hipStream_t stream, int *result_in_b) {
    *result_in_b = 0;
    const int last = plan.passes - 1;
    if (last < 1 || last + 1 >= kMaxPasses || plan.bits[last] != 8)
        return fail(GS_ERR_INVALID_ARG, "depth order: %d passes (need 2 to %d, the last of 8 bits)", plan.passes,
                    kMaxPasses - 1);
    if (n < 1) return ok();
    // row plan.passes of the histogram copies holds the tile counts by the last pass's digit
    const SortScratch S = sort_scratch(scratch, n);
    gs_status st = launch_digit_starts(S, plan.passes + 1, false, stream);
    if (st != GS_OK) return st;
    st = run_digit_passes<uint32_t>(depth_bits, nullptr, buf_a_keys, buf_a_ids, buf_b_keys, buf_b_ids, n, plan, last,
                                    S, stream);
    if (st != GS_OK) return st;
    // pass `last` reads what pass last - 1 wrote
    const bool to_a = (last % 2) == 0;
    const uint32_t *starts = S.starts;
    const int64_t parts = (n + kThreads * kItems32 - 1) / (kThreads * kItems32);
    hipLaunchKernelGGL(depth_order_pass_kernel, dim3(static_cast<unsigned>(parts)), dim3(kThreads), 0, stream,
                       to_a ? buf_b_keys : buf_a_keys, to_a ? buf_b_ids : buf_a_ids, rects, pk,
                       to_a ? buf_a_keys : buf_b_keys, to_a ? buf_a_ids : buf_b_ids, sorted_rects, sorted_offsets, n,
                       plan.shift[last], starts + last * kRadix, starts + plan.passes * kRadix, order_status,
                       spin_limit());
    GS_LAUNCH_TRY("depth_order_pass_kernel");
    *result_in_b = to_a ? 0 : 1;
    return ok();
}

template gs_status radix_sort_pairs<uint32_t>(const uint32_t *, const int32_t *, uint32_t *, int32_t *, uint32_t *,
                                              int32_t *, int64_t, const PassPlan &, void *, hipStream_t, int *);
template gs_status radix_sort_pairs<uint64_t>(const uint64_t *, const int32_t *, uint64_t *, int32_t *, uint64_t *,
                                              int32_t *, int64_t, const PassPlan &, void *, hipStream_t, int *);
template gs_status radix_passes<uint32_t>(const uint32_t *, const int32_t *, uint32_t *, int32_t *, uint32_t *,
                                          int32_t *, int64_t, const PassPlan &, void *, hipStream_t, int *);
template gs_status radix_passes<uint64_t>(const uint64_t *, const int32_t *, uint64_t *, int32_t *, uint64_t *,
                                          int32_t *, int64_t, const PassPlan &, void *, hipStream_t, int *);
template gs_status radix_passes<uint64_t>(const uint64_t *, const int32_t *, uint64_t *, int32_t *, uint64_t *,
                                          int32_t *, int64_t, const PassPlan &, const SortScratch &, hipStream_t,
                                          int *);

namespace {

struct SortLayout {
    size_t alt_keys, alt_ids, scratch, bytes;
};

SortLayout sort_layout(int64_t n) {
    SortLayout L{};
    Carver c(nullptr);
    const size_t nn = static_cast<size_t>(n > 0 ? n : 1);
    c.take<uint64_t>(nn);
    L.alt_keys = 0;
    L.alt_ids = align_up(c.used, 256);
    c.take<int32_t>(nn);
    L.scratch = align_up(c.used, 256);
    L.bytes = L.scratch + sort_scratch_layout(n).bytes;
    return L;
}

}  // namespace

size_t sort_workspace_layout(int64_t n, int) { return sort_layout(n).bytes; }

// In-place stable sort of (keys, ids) by bits [0, end_bit): passes alternate between the caller's arrays and the
// workspace copies; an odd pass count starts with a copy into the workspace so the last pass lands in place.
gs_status sort_pairs_u64(uint64_t *keys, int32_t *ids, int64_t n, int end_bit, void *workspace,
                         hipStream_t stream) {
    if (n < 2 || end_bit == 0) return ok();
    const SortLayout L = sort_layout(n);
    char *ws = static_cast<char *>(workspace);
    uint64_t *alt_keys = reinterpret_cast<uint64_t *>(ws + L.alt_keys);
    int32_t *alt_ids = reinterpret_cast<int32_t *>(ws + L.alt_ids);
    const PassPlan plan = make_pass_plan(0, end_bit);
    int in_b = 0;
    if (plan.passes % 2 == 0) {
        // keys -> alt -> keys -> ...: the even last pass writes the caller's arrays
        return radix_sort_pairs<uint64_t>(keys, ids, alt_keys, alt_ids, keys, ids, n, plan, ws + L.scratch, stream,
                                          &in_b);
    }
    GS_HIP_TRY(hipMemcpyAsync(alt_keys, keys, static_cast<size_t>(n) * sizeof(uint64_t), hipMemcpyDeviceToDevice,
                              stream));
    GS_HIP_TRY(hipMemcpyAsync(alt_ids, ids, static_cast<size_t>(n) * sizeof(int32_t), hipMemcpyDeviceToDevice,
                              stream));
    return radix_sort_pairs<uint64_t>(alt_keys, alt_ids, keys, ids, alt_keys, alt_ids, n, plan, ws + L.scratch,
                                      stream, &in_b);
}

}  // namespace gs

using namespace gs;

extern "C" size_t gs_sort_workspace_bytes(int64_t n, int end_bit) {
    if (n < 0 || end_bit < 0 || end_bit > 64) return 0;
    return sort_layout(n).bytes;
}

extern "C" gs_status gs_sort_keys(uint64_t *keys, int32_t *flatten_ids, int64_t n, int end_bit, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    if (n < 0 || n >= (int64_t(1) << 30))
        return fail(GS_ERR_INVALID_ARG, "gs_sort_keys: n = %lld outside [0, 2^30)", (long long)n);
    if (end_bit < 0 || end_bit > 64)
        return fail(GS_ERR_INVALID_ARG, "gs_sort_keys: end_bit = %d outside [0, 64]", end_bit);
    if (n > 0 && (!keys || !flatten_ids)) return fail(GS_ERR_INVALID_ARG, "gs_sort_keys: keys and ids are required");
    if (n < 2 || end_bit == 0) return ok();
    const size_t need = sort_layout(n).bytes;
    if (!workspace || workspace_bytes < need)
        return fail(GS_ERR_WORKSPACE, "gs_sort_keys: needs %zu workspace bytes (got %zu)", need, workspace_bytes);
    return sort_pairs_u64(keys, flatten_ids, n, end_bit, workspace, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------------------------
// The sort without a caller workspace: its alternate buffers, histograms and look-back words live in a file-scope
// device array (one per GPU, held until the process ends), for callers that cannot allocate.
namespace gs {
namespace {

constexpr int64_t kStaticSortMaxPairs = int64_t(1) << 22;
constexpr size_t kStaticScratchBytes = size_t(52) << 20;  // >= sort_layout(kStaticSortMaxPairs).bytes (checked)
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace
}  // namespace gs

__device__ __align__(256) unsigned char scratch[gs::kStaticScratchBytes];

namespace gs {
namespace {

// The device address of this GPU's `scratch` array (the host-side name is only a stand-in for the symbol), looked up
// once per device with that device current.
gs_status static_scratch(void **out) {
    int dev = 0;
    GS_HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(GS_ERR_DEVICE, "gs_sort_keys_static: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        GS_HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) return fail(GS_ERR_DEVICE, "gs_sort_keys_static: no address for the scratch array");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}

}  // namespace
}  // namespace gs

extern "C" gs_status gs_sort_keys_static(uint64_t *keys, int32_t *flatten_ids, int64_t n, int end_bit, void *stream) {
    if (n < 0 || n > gs::kStaticSortMaxPairs)
        return fail(GS_ERR_INVALID_ARG, "gs_sort_keys_static: n = %lld outside [0, 2^22] (the static scratch holds at "
                                        "most 2^22 pairs; use gs_sort_keys with a workspace for more)", (long long)n);
    if (end_bit < 0 || end_bit > 64)
        return fail(GS_ERR_INVALID_ARG, "gs_sort_keys_static: end_bit = %d outside [0, 64]", end_bit);
    if (n > 0 && (!keys || !flatten_ids))
        return fail(GS_ERR_INVALID_ARG, "gs_sort_keys_static: keys and ids are required");
    if (n < 2 || end_bit == 0) return ok();
    if (sort_layout(gs::kStaticSortMaxPairs).bytes > gs::kStaticScratchBytes)
        return fail(GS_ERR_DEVICE, "gs_sort_keys_static: the static scratch is smaller than the sort's layout");
    void *ws = nullptr;
    gs_status st = gs::static_scratch(&ws);
    if (st != GS_OK) return st;
    return sort_pairs_u64(keys, flatten_ids, n, end_bit, ws, static_cast<hipStream_t>(stream));
}

extern "C" uint32_t gs_set_spin_limit(uint32_t limit) { return g_spin_limit.exchange(limit); }

namespace gs {
namespace {
std::mutex g_error_mutex;
uint32_t *g_error_ptr[kMaxDevices] = {};
}  // namespace

uint32_t spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

gs_status device_error_word(uint32_t **out) {
    int dev = 0;
    GS_HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(GS_ERR_DEVICE, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_error_mutex);
    if (!g_error_ptr[dev]) {
        void *ptr = nullptr;
        GS_HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_device_error)));
        if (!ptr) return fail(GS_ERR_DEVICE, "no address for the device error word");
        g_error_ptr[dev] = static_cast<uint32_t *>(ptr);
    }
    *out = g_error_ptr[dev];
    return ok();
}
}  // namespace gs

extern "C" gs_status gs_device_check(void *stream_handle) {
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    uint32_t word = 0;
    const uint32_t zero = 0;
    GS_HIP_TRY(hipMemcpyFromSymbolAsync(&word, HIP_SYMBOL(g_device_error), sizeof word, 0, hipMemcpyDeviceToHost,
                                        stream));
    GS_HIP_TRY(hipStreamSynchronize(stream));
    if (word == 0) return ok();
    GS_HIP_TRY(hipMemcpyToSymbolAsync(HIP_SYMBOL(g_device_error), &zero, sizeof zero, 0, hipMemcpyHostToDevice,
                                      stream));
    GS_HIP_TRY(hipStreamSynchronize(stream));
    const bool sort = word & kDeviceErrSortLookBack, scan = word & kDeviceErrScanLookBack;
    if (sort || scan)
        return fail(GS_ERR_DEVICE, "gs_device_check: a partition of %s stopped waiting for its predecessors (spin limit "
                                   "reached); that call's output is invalid (device error word 0x%x)",
                    sort && scan ? "a radix sort and of an intersection-count scan"
                                 : (sort ? "a radix sort" : "an intersection-count scan"),
                    word);
    return fail(GS_ERR_DEVICE, "gs_device_check: device error word 0x%x", word);
}

// Internal interface of the onesweep radix sort (sort.hip), shared with the intersection step.
#pragma once

#include "gs_rect.hpp"

namespace gs {

constexpr int kMaxPasses = 8;

// The digit histograms (kMaxPasses x 256 counts) are kept in kHistCopies copies: producer workgroup b adds its
// counts into copy b % kHistCopies and the digit passes sum the copies. Device-scope atomics to one word serialize
// at the memory side, so thousands of workgroups flushing into a single copy queue up behind each other.
constexpr int kHistCopies = 16;
constexpr int kHistCopyWords = kMaxPasses * 256;
__device__ __forceinline__ uint32_t *hist_copy(uint32_t *hist, unsigned block) {
    return hist + static_cast<size_t>(block % kHistCopies) * kHistCopyWords;
}

// Digit counting by runs. Lanes holding consecutive keys compare a digit with the previous lane's, and each run
// of equal digits is added to an LDS histogram once, by its first lane, as its length: keys that share a digit
// (one splat's intersections share their depth bits) then cost one LDS atomic per run instead of one per key.
// The two halves of the wave (lanes 0-31 and 32-63) are counted apart, so a run's length is found in one 32-bit
// word: its first lane shifts the 64-bit mask of run starts right by lane + 1, which puts lane (lane + 1 + k) at
// bit k. A lower-half run ends at the latest at lane 32 (always marked a start); an upper-half run ends at the
// latest at the wave's end, which a per-lane sentinel bit at the position of lane 64 marks.
struct RunLanes {
    uint32_t shift;     // lane + 1, and 63 for lane 63 (its own start bit, set whenever it counts, lands at bit 0)
    uint32_t sentinel;  // 1 << (63 - lane) in lanes 32..63, 0 in lanes 0..31
    bool first;         // lanes 0 and 32 start a run whatever their digit
};
__device__ __forceinline__ RunLanes run_lanes() {
    const uint32_t lane = __lane_id();
    return {lane < 63u ? lane + 1u : 63u, lane >= 32u ? 1u << (63u - lane) : 0u, lane == 0u || lane == 32u};
}
// Adds the wave's digits d to the LDS histogram hist. The whole wave must call it together (it reads the previous
// lane's digit); a lane with in == false holds no key, adds nothing and must hold a digit no key can have
// (0xffffffff), so that it never extends a run.
__device__ __forceinline__ void wave_add_runs(uint32_t *hist, uint32_t d, bool in, const RunLanes &rl) {
    // the previous lane's digit (a whole-wave shift right by one lane; lane 0 reads 0 and is a start anyway)
    const uint32_t prev = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(d), 0x138, 0xf, 0xf, true));
    const bool differs = d != prev;
    // the ballot of the comparison alone stays one compare; lanes 0 and 32 are or-ed in as constants
    const uint64_t starts = __builtin_amdgcn_ballot_w64(differs) | 0x0000000100000001ull;
    if ((differs | rl.first) & in) {  // bitwise: a short-circuit turns into branches
        // nonzero: bit 32 of starts (lower half) or the sentinel (upper half) bounds the run
        const uint32_t later = static_cast<uint32_t>(starts >> rl.shift) | rl.sentinel;
        atomicAdd(&hist[d], static_cast<uint32_t>(__builtin_ctz(later)) + 1u);
    }
}

// Digit passes over bits [begin_bit, end_bit): pass p sorts `bits[p]` bits starting at `shift[p]`.
struct PassPlan {
    int passes;
    int shift[kMaxPasses];
    int bits[kMaxPasses];
};

// Splits [begin_bit, end_bit) evenly into ceil(width / 8) passes of at most 8 bits.
PassPlan make_pass_plan(int begin_bit, int end_bit);

// Per-sort scratch: digit histograms, partition counters and two look-back arrays sized for n pairs.
struct SortScratchLayout {
    size_t hist, counters, status0, status1, starts, bytes;
    int64_t parts;
};
SortScratchLayout sort_scratch_layout(int64_t n);

// The scratch of one sort as separate regions (the contiguous layout above, or regions a caller places itself):
// histogram copies (kHistCopies x kHistCopyWords words), partition counters (kMaxPasses words), two look-back arrays
// of parts x 256 words and the digit starts (kMaxPasses x 256 words).
struct SortScratch {
    uint32_t *hist, *counters, *status0, *status1, *starts;
    int64_t parts;
};
SortScratch sort_scratch(void *scratch, int64_t n);
// The contiguous layout in two pieces: the head (histogram copies and counters, the same size for every n) and the
// tail (look-back arrays and digit starts), each at its own address.
size_t sort_scratch_head_bytes();
size_t sort_scratch_tail_bytes(int64_t n);
SortScratch sort_scratch_split(void *head, void *tail, int64_t n);
// Partitions of one digit pass over n pairs of KeyT keys: its look-back array spans that many times 256 words.
template <typename KeyT>
int64_t radix_partitions(int64_t n);

// Clears the scratch's histograms, partition counters and first look-back array for a sort of n pairs.
gs_status radix_prepare(int64_t n, void *scratch, hipStream_t stream);
// Bytes at the start of the scratch that radix_prepare clears (a caller may clear them itself instead).
size_t radix_clear_bytes(int64_t n);
// The scratch's per-pass digit histograms (kHistCopies copies of kMaxPasses x 256 counts) for a sort of n pairs.
uint32_t *radix_histograms(void *scratch, int64_t n);

// The digit passes alone, after radix_prepare and with the histograms already accumulated by the caller.
template <typename KeyT>
gs_status radix_passes(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                       KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan, void *scratch,
                       hipStream_t stream, int *result_in_b);
// The same with the scratch in separate regions. The histogram copies must be zero before the caller accumulates
// the histograms and the first look-back array zero when the passes start; the digit starts step zeroes the
// histogram entries once it has read them and resets the passes' partition counters itself, so after a sort the
// histogram copies are ready for the next one.
template <typename KeyT>
gs_status radix_passes(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                       KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan,
                       const SortScratch &scratch, hipStream_t stream, int *result_in_b);

// The splats' depth order for the emission: the passes of plan (histograms already accumulated by the caller, and
// in row plan.passes of the histogram copies the tile counts by the last pass's digit), the last one (8 bits) also
// writing, for every position of the order, the rectangle of its splat (gathered from rects, in splat order; int4,
// or one packed word when pk.cx is nonzero) and its first output slot (the exclusive prefix of the tile counts in
// that order). Pass p writes buffer A when p is even and B when odd; *result_in_b tells where the order lands.
// order_status holds depth_order_status_bytes(n) bytes, zero before the call.
size_t depth_order_status_bytes(int64_t n);
gs_status depth_order_passes(const uint32_t *depth_bits, uint32_t *buf_a_keys, int32_t *buf_a_ids,
                             uint32_t *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan,
                             void *scratch, const void *rects, void *sorted_rects, RectPacking pk,
                             int32_t *sorted_offsets, uint64_t *order_status, hipStream_t stream, int *result_in_b);

// Stable LSD sort of n (key, id) pairs (prepare + histograms + passes). Pass 0 reads (keys_in, ids_in)
// (ids_in == nullptr: ids are the input positions); pass p writes buffer A when p is even and B when odd, so the
// result is in B after an even number of passes (*result_in_b = 1) and in A after an odd number. keys_in may alias
// B but never A.
template <typename KeyT>
gs_status radix_sort_pairs(const KeyT *keys_in, const int32_t *ids_in, KeyT *buf_a_keys, int32_t *buf_a_ids,
                           KeyT *buf_b_keys, int32_t *buf_b_ids, int64_t n, const PassPlan &plan, void *scratch,
                           hipStream_t stream, int *result_in_b);

// Bits of the library's device error word (one per GPU, read and cleared by gs_device_check): a digit pass, or a
// single-pass scan of the intersection counts, whose look-back wait ran past the spin limit.
constexpr uint32_t kDeviceErrSortLookBack = 1u;
constexpr uint32_t kDeviceErrScanLookBack = 2u;
// The device address of this GPU's error word (looked up once per device with that device current).
gs_status device_error_word(uint32_t **out);
// Look-back rounds a waiting partition may spend before it gives up (gs_set_spin_limit).
uint32_t spin_limit();

}  // namespace gs

// Internal interface of the onesweep radix sort (sort.hip), shared with the intersection step.
#pragma once

#include "gs_internal.hpp"

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

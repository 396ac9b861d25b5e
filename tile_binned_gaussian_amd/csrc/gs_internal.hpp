// Internal helpers shared by the HIP translation units of libgs_raster (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "gs_raster.h"

namespace gs {

constexpr int kWave = 64;  // CDNA wavefront width

// Records a formatted message for gs_last_error() on this thread and returns `status`.
gs_status fail(gs_status status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
gs_status ok();

#define GS_HIP_TRY(expr)                                                                              \
    do {                                                                                              \
        hipError_t gs_e_ = (expr);                                                                    \
        if (gs_e_ != hipSuccess) return ::gs::fail(GS_ERR_DEVICE, "%s failed: %s", #expr,            \
                                                   hipGetErrorString(gs_e_));                         \
    } while (0)

#define GS_LAUNCH_TRY(name)                                                                           \
    do {                                                                                              \
        hipError_t gs_e_ = hipGetLastError();                                                         \
        if (gs_e_ != hipSuccess) return ::gs::fail(GS_ERR_DEVICE, "launch of %s failed: %s", name,   \
                                                   hipGetErrorString(gs_e_));                         \
    } while (0)

// Smallest b >= 0 with 2^b >= count ([gsplat] gs_tile_bits).
inline int bits_for(int64_t count) {
    int bits = 0;
    uint64_t capacity = 1;
    while (capacity < static_cast<uint64_t>(count)) {
        capacity <<= 1;
        ++bits;
    }
    return bits;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Carves consecutive 256-byte-aligned slices out of a caller-provided workspace.
struct Carver {
    char *base;
    size_t used = 0;
    explicit Carver(void *b) : base(static_cast<char *>(b)) {}
    template <typename T>
    T *take(size_t count) {
        used = align_up(used, 256);
        T *p = base ? reinterpret_cast<T *>(base + used) : nullptr;
        used += count * sizeof(T);
        return p;
    }
};

// Fills `count` 32-bit words with `value` (a kernel, not hipMemsetAsync, so the work can sit in a graph).
hipError_t fill_u32(uint32_t *dst, uint32_t value, size_t count, hipStream_t stream);

// Stable LSD radix sort of (key, id) pairs by bits [0, end_bit), result in keys/ids. Workspace laid out by
// sort_workspace_layout. Caller has validated the arguments.
gs_status sort_pairs_u64(uint64_t *keys, int32_t *ids, int64_t n, int end_bit, void *workspace,
                         hipStream_t stream);
size_t sort_workspace_layout(int64_t n, int end_bit);

// ------------------------------------------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum across the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_inclusive_sum(T v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        T o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

}  // namespace gs

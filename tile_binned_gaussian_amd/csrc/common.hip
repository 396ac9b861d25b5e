// Error reporting and small utility kernels of libgs_raster.
#include "gs_internal.hpp"

namespace gs {

static thread_local char g_error[512] = "";

gs_status fail(gs_status status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return status;
}

gs_status ok() {
    g_error[0] = '\0';
    return GS_OK;
}

__global__ void fill_u32_kernel(uint32_t *__restrict__ dst, uint32_t value, size_t count) {
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (; i < count; i += stride) dst[i] = value;
}

hipError_t fill_u32(uint32_t *dst, uint32_t value, size_t count, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, dst, value,
                       count);
    return hipGetLastError();
}

}  // namespace gs

extern "C" const char *gs_last_error(void) { return gs::g_error; }

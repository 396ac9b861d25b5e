// EWA projection of 3D Gaussians into C cameras on gfx950: one thread per (camera, Gaussian), the camera's view and
// intrinsics read once per wavefront (uniform across the workgroup's camera row), every output written coalesced.
// Memory-bound: per (camera, Gaussian) 48 bytes read (mean, covariance) and 36-40 bytes written.
//
// Definition: gsplat 1.0.0 projection.c, gs_project_one (with gs_mat3_product, gs_camera_covar and gs_clip),
// evaluated in float32 in the page's operation order with no contraction, so the results equal a plain C
// evaluation of the same steps bit for bit.
#include "gs_internal.hpp"

#include <cmath>

namespace gs {
namespace {

constexpr int kThreads = 256;

// 3x3 product, each entry summed from 0 over the inner index in order.
__device__ __forceinline__ void mat3_product(const float *l, const float *r, float *out) {
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            float v = 0.0f;
#pragma unroll
            for (int k = 0; k < 3; ++k) v += l[i * 3 + k] * r[k * 3 + j];
            out[i * 3 + j] = v;
        }
}

// ceil as int32 with the float clamped to [0, 2^31 - 1] first (NaN -> 0), defined for every input.
__device__ __forceinline__ int32_t ceil_radius(float v) {
    const float c = ceilf(v);
    if (!(c > 0.0f)) return 0;
    if (c >= 2147483648.0f) return 2147483647;
    return static_cast<int32_t>(c);
}

struct ProjectArgs {
    const float *means, *covars, *views, *Ks;
    int64_t N;
    int width, height, orthographic;
    float eps2d, near_plane, far_plane, radius_clip;
    int32_t *radii;
    float *means2d, *depths, *conics, *comps;
};

// grid: x over Gaussians, y over cameras.
__global__ __launch_bounds__(kThreads) void project_kernel(ProjectArgs a) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int c = static_cast<int>(blockIdx.y);
    if (g >= a.N) return;
    const float *view = a.views + c * 16;
    const float *K = a.Ks + c * 9;
    const float R[9] = {view[0], view[1], view[2], view[4], view[5], view[6], view[8], view[9], view[10]};
    const float Rt[9] = {R[0], R[3], R[6], R[1], R[4], R[7], R[2], R[5], R[8]};
    const float *m = a.means + g * 3;
    const float m0 = m[0], m1 = m[1], m2 = m[2];
    float cov[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) cov[i] = a.covars[g * 9 + i];

    float mc[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) mc[r] = R[r * 3] * m0 + R[r * 3 + 1] * m1 + R[r * 3 + 2] * m2 + view[r * 4 + 3];
    float tmp[9], cc[9];
    mat3_product(R, cov, tmp);
    mat3_product(tmp, Rt, cc);
    const float depth = mc[2];
    const float z = (depth <= a.near_plane || depth >= a.far_plane) ? 1.0f : depth;
    float J[6] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float p0, p1;
    if (a.orthographic) {
        J[0] = K[0];
        J[4] = K[4];
        p0 = mc[0] * K[0] + K[2];
        p1 = mc[1] * K[4] + K[5];
    } else {
        const float w = static_cast<float>(a.width), h = static_cast<float>(a.height);
        const float min_x = -(K[2] / K[0] + 0.15f * w / K[0]);
        const float max_x = (w - K[2]) / K[0] + 0.15f * w / K[0];
        const float min_y = -(K[5] / K[4] + 0.15f * h / K[4]);
        const float max_y = (h - K[5]) / K[4] + 0.15f * h / K[4];
        const float cx = fminf(fmaxf(mc[0] / z, min_x), max_x) * z;
        const float cy = fminf(fmaxf(mc[1] / z, min_y), max_y) * z;
        J[0] = K[0] / z;
        J[2] = -K[0] * cx / (z * z);
        J[4] = K[4] / z;
        J[5] = -K[4] * cy / (z * z);
        p0 = (K[0] * mc[0] + K[1] * mc[1] + K[2] * z) / z;
        p1 = (K[3] * mc[0] + K[4] * mc[1] + K[5] * z) / z;
    }
    float c2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j) c2[r * 2 + q] += J[r * 3 + i] * cc[i * 3 + j] * J[q * 3 + j];
    const float det0 = c2[0] * c2[3] - c2[1] * c2[2];
    c2[0] += a.eps2d;
    c2[3] += a.eps2d;
    const float det = c2[0] * c2[3] - c2[1] * c2[2];
    const float safe = det <= 0.0f ? 1e-10f : det;
    const int32_t rx = ceil_radius(3.33f * sqrtf(fmaxf(c2[0], 0.0f)));
    const int32_t ry = ceil_radius(3.33f * sqrtf(fmaxf(c2[3], 0.0f)));
    const float frx = static_cast<float>(rx), fry = static_cast<float>(ry);
    const bool visible = det > 0.0f && depth > a.near_plane && depth < a.far_plane &&
                         (frx > a.radius_clip || fry > a.radius_clip) && p0 + frx > 0.0f &&
                         p0 - frx < static_cast<float>(a.width) && p1 + fry > 0.0f &&
                         p1 - fry < static_cast<float>(a.height);
    const int64_t i = static_cast<int64_t>(c) * a.N + g;
    reinterpret_cast<int2 *>(a.radii)[i] = visible ? make_int2(rx, ry) : make_int2(0, 0);
    reinterpret_cast<float2 *>(a.means2d)[i] = make_float2(p0, p1);
    a.depths[i] = depth;
    a.conics[i * 3] = c2[3] / safe;
    a.conics[i * 3 + 1] = -(c2[1] + c2[2]) / (2.0f * safe);
    a.conics[i * 3 + 2] = c2[0] / safe;
    if (a.comps) a.comps[i] = sqrtf(fmaxf(det0 / safe, 0.0f));
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" gs_status gs_project_fwd(const float *means, const float *covars, const float *viewmats, const float *Ks,
                                    int64_t C, int64_t N, int width, int height, float eps2d, float near_plane,
                                    float far_plane, float radius_clip, int orthographic, int32_t *radii,
                                    float *means2d, float *depths, float *conics, float *compensations,
                                    void *stream_handle) {
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    if (C < 1 || C > 65535 || N < 0 || C * N >= (int64_t(1) << 31))
        return fail(GS_ERR_INVALID_ARG, "gs_project_fwd: need 1 <= C <= 65535, N >= 0 and C*N < 2^31");
    if (width < 1 || height < 1) return fail(GS_ERR_INVALID_ARG, "gs_project_fwd: width and height must be >= 1");
    if (!viewmats || !Ks) return fail(GS_ERR_INVALID_ARG, "gs_project_fwd: viewmats and Ks are required");
    if (N > 0 && (!means || !covars || !radii || !means2d || !depths || !conics))
        return fail(GS_ERR_INVALID_ARG, "gs_project_fwd: a required pointer is NULL");
    if (N == 0) return ok();
    ProjectArgs args{means, covars, viewmats, Ks, N, width, height, orthographic ? 1 : 0,
                     eps2d, near_plane, far_plane, radius_clip, radii, means2d, depths, conics, compensations};
    const dim3 grid(static_cast<unsigned>((N + kThreads - 1) / kThreads), static_cast<unsigned>(C));
    hipLaunchKernelGGL(project_kernel, grid, dim3(kThreads), 0, stream, args);
    GS_LAUNCH_TRY("project_kernel");
    return ok();
}

// Calibration kernels for the profiler's VALU instruction counter and for the FP32 VALU issue rate on gfx950.
//
// Each kernel runs `iters` rounds of 16 vector instructions written as inline assembly (so the instruction count
// per wave is known exactly: 16 per round, plus a fixed prologue and epilogue that cancels between two launches
// with different round counts), over 8 independent register chains, with every lane active. Per wave it also
// records the shader clock (s_memtime) and the constant-rate clock (s_memrealtime) at the start and the end of
// the rounds, so the clock the SIMDs actually ran at under this load can be read back.
//
// Kinds: 0 v_fmac_f32; 1 v_mul_f32; 2 v_cndmask_b32; 3 v_mov_b32 with a DPP row shift; 4 v_exp_f32;
// 5 v_cmp_gt_f32 into a scalar pair; 6 a mix (per 8: 4 fmac, 2 mul, 1 cndmask, 1 exp); 7 v_add_f32; 8 v_sub_f32;
// 9 v_fma_f32 (three vector sources); 10 v_fmaak_f32 (literal addend); 11 v_mov_b32; 12 v_add_u32;
// 13 v_rndne_f32; 14 v_ldexp_f32; 15 v_cvt_i32_f32; 16 v_max_f32; 17 the forward composite loop's proportions
// without a transcendental (per 16: 5 mul, 2 add, 1 sub, 2 fma, 2 cndmask, 2 cmp, 1 rndne, 1 ldexp).
// Measurement infrastructure only (not part of the rasterizer's ABI).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

#define FMAC(x) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(x) : "v"(a), "v"(b))
#define MUL(x) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(a))
#define CND(x) asm volatile("v_cndmask_b32_e64 %0, %0, %1, %2" : "+v"(x) : "v"(b), "s"(mask))
#define DPP(x) asm volatile("v_mov_b32_dpp %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(x))
#define EXP(x) asm volatile("v_exp_f32 %0, %0" : "+v"(x))
#define CMP(m, x) asm volatile("v_cmp_gt_f32_e64 %0, %1, %2" : "=s"(m) : "v"(x), "v"(a))
#define ADD(x) asm volatile("v_add_f32 %0, %0, %1" : "+v"(x) : "v"(b))
#define SUB(x) asm volatile("v_sub_f32 %0, %0, %1" : "+v"(x) : "v"(b))
#define FMA3(x) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(a), "v"(b))
#define FMAAK(x) asm volatile("v_fmaak_f32 %0, %0, %1, 0x3a83126f" : "+v"(x) : "v"(a))
#define MOV(x) asm volatile("v_mov_b32 %0, %1" : "=v"(x) : "v"(b))
#define ADDU(x) asm volatile("v_add_u32 %0, %0, %1" : "+v"(x) : "v"(b))
#define RND(x) asm volatile("v_rndne_f32 %0, %0" : "+v"(x))
#define LDX(x) asm volatile("v_ldexp_f32 %0, %0, %1" : "+v"(x) : "v"(k))
#define CVT(y, x) asm volatile("v_cvt_i32_f32 %0, %1" : "=v"(y) : "v"(x))
#define MAX(x) asm volatile("v_max_f32 %0, %0, %1" : "+v"(x) : "v"(b))

template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_calib_kernel(float *__restrict__ out,
                                                              unsigned long long *__restrict__ clocks, int iters,
                                                              float a, float b, unsigned long long mask) {
    float x0 = threadIdx.x * 1e-3f, x1 = x0 + 1.0f, x2 = x0 + 2.0f, x3 = x0 + 3.0f, x4 = x0 + 4.0f, x5 = x0 + 5.0f,
          x6 = x0 + 6.0f, x7 = x0 + 7.0f;
    unsigned long long m0 = 0, m1 = 0, m2 = 0, m3 = 0, m4 = 0, m5 = 0, m6 = 0, m7 = 0;
    int k = 0, y0 = 0, y1 = 0, y2 = 0, y3 = 0, y4 = 0, y5 = 0, y6 = 0, y7 = 0;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if constexpr (KIND == 0) {
                FMAC(x0); FMAC(x1); FMAC(x2); FMAC(x3); FMAC(x4); FMAC(x5); FMAC(x6); FMAC(x7);
            } else if constexpr (KIND == 1) {
                MUL(x0); MUL(x1); MUL(x2); MUL(x3); MUL(x4); MUL(x5); MUL(x6); MUL(x7);
            } else if constexpr (KIND == 2) {
                CND(x0); CND(x1); CND(x2); CND(x3); CND(x4); CND(x5); CND(x6); CND(x7);
            } else if constexpr (KIND == 3) {
                DPP(x0); DPP(x1); DPP(x2); DPP(x3); DPP(x4); DPP(x5); DPP(x6); DPP(x7);
            } else if constexpr (KIND == 4) {
                EXP(x0); EXP(x1); EXP(x2); EXP(x3); EXP(x4); EXP(x5); EXP(x6); EXP(x7);
            } else if constexpr (KIND == 5) {
                CMP(m0, x0); CMP(m1, x1); CMP(m2, x2); CMP(m3, x3); CMP(m4, x4); CMP(m5, x5); CMP(m6, x6);
                CMP(m7, x7);
            } else if constexpr (KIND == 6) {
                FMAC(x0); MUL(x1); FMAC(x2); CND(x3); FMAC(x4); MUL(x5); EXP(x6); FMAC(x7);
            } else if constexpr (KIND == 7) {
                ADD(x0); ADD(x1); ADD(x2); ADD(x3); ADD(x4); ADD(x5); ADD(x6); ADD(x7);
            } else if constexpr (KIND == 8) {
                SUB(x0); SUB(x1); SUB(x2); SUB(x3); SUB(x4); SUB(x5); SUB(x6); SUB(x7);
            } else if constexpr (KIND == 9) {
                FMA3(x0); FMA3(x1); FMA3(x2); FMA3(x3); FMA3(x4); FMA3(x5); FMA3(x6); FMA3(x7);
            } else if constexpr (KIND == 10) {
                FMAAK(x0); FMAAK(x1); FMAAK(x2); FMAAK(x3); FMAAK(x4); FMAAK(x5); FMAAK(x6); FMAAK(x7);
            } else if constexpr (KIND == 11) {
                MOV(x0); MOV(x1); MOV(x2); MOV(x3); MOV(x4); MOV(x5); MOV(x6); MOV(x7);
            } else if constexpr (KIND == 12) {
                ADDU(x0); ADDU(x1); ADDU(x2); ADDU(x3); ADDU(x4); ADDU(x5); ADDU(x6); ADDU(x7);
            } else if constexpr (KIND == 13) {
                RND(x0); RND(x1); RND(x2); RND(x3); RND(x4); RND(x5); RND(x6); RND(x7);
            } else if constexpr (KIND == 14) {
                LDX(x0); LDX(x1); LDX(x2); LDX(x3); LDX(x4); LDX(x5); LDX(x6); LDX(x7);
            } else if constexpr (KIND == 15) {
                CVT(y0, x0); CVT(y1, x1); CVT(y2, x2); CVT(y3, x3); CVT(y4, x4); CVT(y5, x5); CVT(y6, x6);
                CVT(y7, x7);
            } else if constexpr (KIND == 16) {
                MAX(x0); MAX(x1); MAX(x2); MAX(x3); MAX(x4); MAX(x5); MAX(x6); MAX(x7);
            } else {
                if (u == 0) {
                    MUL(x0); FMA3(x1); MUL(x2); CND(x3); ADD(x4); CMP(m5, x5); MUL(x6); RND(x7);
                } else {
                    MUL(x0); FMA3(x1); SUB(x2); CND(x3); ADD(x4); CMP(m5, x5); MUL(x6); LDX(x7);
                }
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    const float m = static_cast<float>((m0 ^ m1 ^ m2 ^ m3 ^ m4 ^ m5 ^ m6 ^ m7) & 1ull) +
                    static_cast<float>(y0 ^ y1 ^ y2 ^ y3 ^ y4 ^ y5 ^ y6 ^ y7 ^ k);
    out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7 + m;
    if ((threadIdx.x & 63) == 0) {
        const size_t w = (static_cast<size_t>(blockIdx.x) * (kThreads / 64) + threadIdx.x / 64) * 4;
        clocks[w + 0] = t0;
        clocks[w + 1] = t1;
        clocks[w + 2] = r0;
        clocks[w + 3] = r1;
    }
}

#undef FMAC
#undef MUL
#undef CND
#undef DPP
#undef EXP
#undef CMP
#undef ADD
#undef SUB
#undef FMA3
#undef FMAAK
#undef MOV
#undef ADDU
#undef RND
#undef LDX
#undef CVT
#undef MAX

}  // namespace

// Vector instructions per round of each kind (the rounds' part of a wave's count).
extern "C" int gs_calib_valu_per_round(int kind) { return (kind >= 0 && kind <= 17) ? 16 : -1; }

// Launches `blocks` workgroups of 256 threads of kernel `kind` for `iters` rounds. out: [blocks * 256] floats;
// clocks: [blocks * 4 waves * 4] (shader clock start, end, constant clock start, end per wave). Returns 0 or
// the HIP error code.
extern "C" int gs_calib_valu_launch(int kind, int blocks, int iters, float *out, unsigned long long *clocks,
                                    void *stream) {
    if (blocks < 1 || iters < 0 || !out || !clocks) return static_cast<int>(hipErrorInvalidValue);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const float a = 0.999f, b = 1e-3f;
    const unsigned long long mask = 0xaaaaaaaaaaaaaaaaull;
    switch (kind) {
#define GS_CAL(K)                                                                                                  \
    case K:                                                                                                        \
        hipLaunchKernelGGL(valu_calib_kernel<K>, dim3(blocks), dim3(kThreads), 0, s, out, clocks, iters, a, b,  \
                           mask);                                                                                  \
        break;
        GS_CAL(0) GS_CAL(1) GS_CAL(2) GS_CAL(3) GS_CAL(4) GS_CAL(5) GS_CAL(6) GS_CAL(7) GS_CAL(8) GS_CAL(9)
        GS_CAL(10) GS_CAL(11) GS_CAL(12) GS_CAL(13) GS_CAL(14) GS_CAL(15) GS_CAL(16) GS_CAL(17)
#undef GS_CAL
        default: return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
}

// The constant-rate clock's frequency in kHz on the current device (what s_memrealtime counts), or 0.
extern "C" int gs_calib_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

// Device-side scalar helpers for the gfx950 selective-scan kernels: bf16 <-> fp32,
// exp2 / log2 / reciprocal on the hardware transcendental unit, softplus and SiLU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// v_exp_f32 / v_log_f32 / v_rcp_f32: about 1 ulp, half issue rate on gfx950.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element access for the two I/O types.
template <typename IO> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float ld(const float *p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void st(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct io<uint16_t> {
    __device__ __forceinline__ static float ld(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void st(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|).
// log1p(e), e in (0, 1]: for e < 1/16 the alternating series to e^5 (relative error
// below e^5/6 < 2e-7); otherwise log2(1 + e) ln 2, whose only extra error is the
// rounding of 1 + e (below 2^-24 absolute, i.e. < 1e-6 relative for e >= 1/16).
__device__ __forceinline__ float softplus_f32(float x) {
    float e = hw_exp2(-fabsf(x) * kLog2e);
    float poly = e * (1.0f + e * (-0.5f + e * (0.33333334f + e * (-0.25f + e * 0.2f))));
    float lg = hw_log2(1.0f + e) * kLn2;
    float l1p = e < 0.0625f ? poly : lg;
    return fmaxf(x, 0.0f) + l1p;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).  For z << 0, e^-z = inf and the result is -0.
__device__ __forceinline__ float silu_f32(float z) {
    float e = hw_exp2(-z * kLog2e);
    return z * hw_rcp(1.0f + e);
}

}  // namespace ssm

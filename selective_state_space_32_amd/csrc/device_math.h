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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// V consecutive I/O elements moved as raw 32-bit words (W = V * sizeof(IO) / 4 words; bf16
// pairs share a word, low half first).  Requires V * sizeof(IO) to be 4, 8 or a multiple of
// 16 bytes and the address to be aligned to min(16, V * sizeof(IO)) bytes.
// These are the streaming tensors of the scan (u, delta and z read once, y written once), so
// the accesses are non-temporal: they then do not push out of L2 the B / C rows and the
// per-channel parameters that every workgroup of a sequence reads again.
template <int V, typename IO> struct vec {
    static constexpr int W = V * (int)sizeof(IO) / 4;
    static_assert(W >= 1 && (W <= 2 || W % 4 == 0), "unsupported vector width");

    __device__ __forceinline__ static void load(const IO *p, int64_t idx, uint32_t (&w)[W]) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(p + idx);
        if constexpr (W % 4 == 0) {
#pragma unroll
            for (int i = 0; i < W / 4; ++i) {
                const u32x4_t r = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(q) + i);
                w[4 * i] = r.x; w[4 * i + 1] = r.y; w[4 * i + 2] = r.z; w[4 * i + 3] = r.w;
            }
        } else if constexpr (W == 2) {
            const u32x2_t r = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(q));
            w[0] = r.x; w[1] = r.y;
        } else {
            w[0] = __builtin_nontemporal_load(q);
        }
    }
    __device__ __forceinline__ static float get(const uint32_t (&w)[W], int v) {
        if constexpr (sizeof(IO) == 2)
            return __uint_as_float((v & 1) ? (w[v >> 1] & 0xffff0000u) : (w[v >> 1] << 16));
        else
            return __uint_as_float(w[v]);
    }
    __device__ __forceinline__ static void store(IO *p, int64_t idx, const float (&y)[V]) {
        uint32_t w[W];
        if constexpr (sizeof(IO) == 2) {
#pragma unroll
            for (int i = 0; i < W; ++i) w[i] = f32x2_to_bf16x2(y[2 * i], y[2 * i + 1]);
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) w[i] = __float_as_uint(y[i]);
        }
        uint32_t *q = reinterpret_cast<uint32_t *>(p + idx);
        if constexpr (W % 4 == 0) {
#pragma unroll
            for (int i = 0; i < W / 4; ++i) {
                const u32x4_t r = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
                __builtin_nontemporal_store(r, reinterpret_cast<u32x4_t *>(q) + i);
            }
        } else if constexpr (W == 2) {
            const u32x2_t r = {w[0], w[1]};
            __builtin_nontemporal_store(r, reinterpret_cast<u32x2_t *>(q));
        } else {
            __builtin_nontemporal_store(w[0], q);
        }
    }
};

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e), e = e^-|x| in (0, 1].
// log1p(e): w = 1 + e is rounded; the rounding error r = e - (w - 1) is exact, and
// log1p(e) = log(w) + r/w.  r/w is taken as r: |r| <= 2^-24 and r only matters when w is
// close to 1 (for e < 2^-24, w = 1 and the result is e itself).
// max(x, 0) + f is formed as max(x + f, f), the same value for f >= 0 (for x <= 0 the
// rounded x + f cannot exceed f), in two instructions: both operands are arithmetic results,
// so the maximum needs no NaN-quieting step.  A NaN x makes f NaN and the result NaN.
// The derivative sigmoid(x) = e^x / (1 + e^x) comes from the same e: 1 / w for x >= 0 and
// e / w for x < 0.
__device__ __forceinline__ float softplus_f32(float x, float &sig) {
    const float e = hw_exp2(-fabsf(x) * kLog2e);
    const float w = 1.0f + e;
    const float r = e - (w - 1.0f);
    const float f = fmaf(hw_log2(w), kLn2, r);
    sig = (x >= 0.0f ? 1.0f : e) * hw_rcp(w);
    return fmaxf(x + f, f);
}
__device__ __forceinline__ float softplus_f32(float x) {
    float sig;
    return softplus_f32(x, sig);
}

// softplus for bf16 I/O: max(x, 0) + log(1 + e) with e = e^-|x|, without the rounding
// correction of log1p above.  log(1 + e) is then off by the rounding of 1 + e, at most 2^-24
// in absolute terms (so a step size of 1e-3 carries a relative error of 6e-5, far inside what
// bf16 inputs and outputs resolve), and the result is 0 where e < 2^-24 (softplus < 6e-8).
// Three issue slots fewer per element than softplus_f32.  A NaN x gives NaN (through e).
__device__ __forceinline__ float softplus_short_f32(float x) {
    const float e = hw_exp2(-fabsf(x) * kLog2e);
    return fmaf(hw_log2(1.0f + e), kLn2, fmaxf(x, 0.0f));
}
// The same value, and the derivative sigmoid(x) from the same e (as for softplus_f32).
__device__ __forceinline__ float softplus_short_f32(float x, float &sig) {
    const float e = hw_exp2(-fabsf(x) * kLog2e);
    const float w = 1.0f + e;
    sig = (x >= 0.0f ? 1.0f : e) * hw_rcp(w);
    return fmaf(hw_log2(w), kLn2, fmaxf(x, 0.0f));
}

// Exact zero-order hold of the input term: B_bar u = (exp(delta A) - 1) / A * B * u =
// delta * phi(delta A) * B * u with phi(x) = (e^x - 1) / x.  zoh_weight returns the factor m
// with B_bar u = m * u * B, from y = x log2(e) and e = exp2(y) (both already formed for the
// decay), delta and 1 / A: (e - 1) / A where |x| >= 1/32, else delta (1 + x/2 + x^2/6).  Below
// the threshold the dropped terms are under x^3/24 < 1.3e-6 of phi; above it e - 1 loses at
// most 2^-24 / |x| <= 1.9e-6 of its value to the rounding of e.  (For A = 0, x = 0 selects
// the series, so 1 / A never reaches the result.)
__device__ __forceinline__ float zoh_weight(float y, float e, float delta, float inv_a) {
    const float t = fmaf(y, kLn2 * kLn2 * (1.0f / 6.0f), kLn2 * 0.5f);   // (1/2 + x/6) with x = y ln 2, over ln 2
    const float p = fmaf(delta * y, t, delta);                            // delta (1 + x/2 + x^2/6)
    const float q = (e - 1.0f) * inv_a;
    return fabsf(y) < (1.0f / 32.0f) * kLog2e ? p : q;
}

// d m / dA of the exact-ZOH factor m = (e^x - 1) / A, x = delta A (the input term's
// coefficient): (delta e^x - m) / A, which tends to delta^2 / 2 at A = 0.  From y = x log2(e),
// e = exp2(y), m (zoh_weight of the same y and e), delta and 1 / A.  Where |x| < 1/4 the
// power series delta^2 (1/2 + x/3 + x^2/8 + x^3/30 + x^4/144) is used (the next term is below
// 1.3e-6 of the value); elsewhere the closed form, whose cancellation costs at most ~3e-6 of it.
__device__ __forceinline__ float zoh_weight_da(float y, float e, float m, float delta, float inv_a) {
    const float x = y * kLn2;
    float s = fmaf(x, 1.0f / 144.0f, 1.0f / 30.0f);
    s = fmaf(x, s, 1.0f / 8.0f);
    s = fmaf(x, s, 1.0f / 3.0f);
    s = fmaf(x, s, 0.5f);
    const float series = (delta * delta) * s;
    const float closed = fmaf(delta, e, -m) * inv_a;
    return fabsf(x) < 0.25f ? series : closed;
}

// sigmoid(x) = 1 / (1 + e^-x) (0 for x << 0, where e^-x = inf).
__device__ __forceinline__ float sigmoid_f32(float x) { return hw_rcp(1.0f + hw_exp2(-x * kLog2e)); }

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).  For z << 0, e^-z = inf and the result is -0.
__device__ __forceinline__ float silu_f32(float z) {
    float e = hw_exp2(-z * kLog2e);
    return z * hw_rcp(1.0f + e);
}

}  // namespace ssm

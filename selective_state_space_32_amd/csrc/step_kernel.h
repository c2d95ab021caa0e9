// The single-token recurrent step (the constant-memory inference form:
// shakilmahmud.com section 3; urworte.de "Methodische Grundlagen").
//
// Per (sequence s, channel d) the fp32 state row state[s][d][0..N) is read, updated in
// place and y[s][d] written.  The step is bound by the state traffic (2 * 4N bytes per
// (s, d)), so the mapping is chosen for streaming:
//  * G = N / NS lanes share one (s, d), each holding NS = min(N, 4) states, so for N >= 4 a
//    lane moves 16 contiguous bytes of its state row and a wave streams 1 KiB of contiguous
//    state; the partial readouts of the G lanes are added with DPP quad permutes.
//  * A thread handles SP consecutive sequences of one channel: its slice of A is loaded
//    once for all of them, and every load of the SP sequences is issued before the first
//    update, so each lane has SP state rows in flight.
//  * The state is read once and written once per step, so both accesses are non-temporal.
#pragma once

#include "device_math.h"

namespace ssm {

constexpr int kStepSeqPerThread = 2;

// VP: the A, B and C slices of a lane are read as one vector each (needs 16-byte aligned A
// and B / C aligned to NS elements); otherwise element by element.
// ACT: 0 -- delta is the step size itself (already activated);
//      1 -- delta is the raw step-size input, as the scan takes it: the step size is
//           softplus(delta + bias) (softplus != 0) or delta + bias (bias nullable), formed with
//           the scan kernel's own functions (the short softplus for bf16 I/O), so that a
//           prefilled sequence continues with the step sizes the scan would have used;
//      2 -- as 1, with the exact zero-order-hold input term (exp(delta A) - 1) / A * B * u of
//           the scan's SSM_SCAN_EXACT_ZOH path (zoh_weight, from the same exponent and decay).
template <int N, typename IO, bool VP, int ACT = 0>
__global__ void __launch_bounds__(256)
step_kernel(float *__restrict__ state, const IO *__restrict__ u, const IO *__restrict__ delta,
            const float *__restrict__ A, const IO *__restrict__ B, const IO *__restrict__ C,
            const float *__restrict__ Dv, const IO *__restrict__ z, IO *__restrict__ y,
            int64_t S, int64_t D, const float *__restrict__ bias = nullptr, int softplus = 0) {
    constexpr int NS = N < 4 ? N : 4;      // states per lane
    constexpr int G = N / NS;              // lanes per (s, d)
    constexpr int SP = kStepSeqPerThread;  // sequences per thread
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t cols = D * G;
    const int64_t sblk = gid / cols;
    const int64_t q = gid - sblk * cols;
    const int64_t d = q / G;                // < D for every thread
    const int part = (int)(q - d * G);
    const int64_t s0 = sblk * SP;           // the G lanes of one (s, d) share s0

    float a2[NS];
    if constexpr (VP && NS == 4) {
        const float4 a = *reinterpret_cast<const float4 *>(A + d * N + part * NS);
        a2[0] = a.x * kLog2e; a2[1] = a.y * kLog2e; a2[2] = a.z * kLog2e; a2[3] = a.w * kLog2e;
    } else {
#pragma unroll
        for (int i = 0; i < NS; ++i) a2[i] = A[d * N + part * NS + i] * kLog2e;
    }
    const float Dd = Dv ? Dv[d] : 0.0f;
    const float bd = (ACT > 0 && bias) ? bias[d] : 0.0f;
    float inv_a[ACT == 2 ? NS : 1];   // 1 / A for the exact zero-order hold
    if constexpr (ACT == 2) {
#pragma unroll
        for (int i = 0; i < NS; ++i) inv_a[i] = 1.0f / A[d * N + part * NS + i];
    }

    // loads of all SP sequences first (indices clamped in bounds; rows past S are not used)
    float h[SP][NS];
    float dt[SP], uu[SP], zz[SP], Bv[SP][NS], Cv[SP][NS];
#pragma unroll
    for (int j = 0; j < SP; ++j) {
        const int64_t s = s0 + j < S ? s0 + j : S - 1;
        const int64_t pair = s * D + d;
        const float *row = state + pair * N + part * NS;
        if constexpr (NS == 4) {  // 16-byte aligned: the state pointer is checked for it
            const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(row));
            h[j][0] = v.x; h[j][1] = v.y; h[j][2] = v.z; h[j][3] = v.w;
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) h[j][i] = __builtin_nontemporal_load(row + i);
        }
        dt[j] = io<IO>::ld(delta, pair);
        uu[j] = io<IO>::ld(u, pair);
        zz[j] = z ? io<IO>::ld(z, pair) : 0.0f;
        const int64_t bo = s * N + part * NS;
        if constexpr (VP && sizeof(IO) == 2 && NS == 4) {
            const uint2 bw = *reinterpret_cast<const uint2 *>(B + bo);
            const uint2 cw = *reinterpret_cast<const uint2 *>(C + bo);
            Bv[j][0] = __uint_as_float(bw.x << 16); Bv[j][1] = __uint_as_float(bw.x & 0xffff0000u);
            Bv[j][2] = __uint_as_float(bw.y << 16); Bv[j][3] = __uint_as_float(bw.y & 0xffff0000u);
            Cv[j][0] = __uint_as_float(cw.x << 16); Cv[j][1] = __uint_as_float(cw.x & 0xffff0000u);
            Cv[j][2] = __uint_as_float(cw.y << 16); Cv[j][3] = __uint_as_float(cw.y & 0xffff0000u);
        } else if constexpr (VP && sizeof(IO) == 4 && NS == 4) {
            const float4 bw = *reinterpret_cast<const float4 *>(B + bo);
            const float4 cw = *reinterpret_cast<const float4 *>(C + bo);
            Bv[j][0] = bw.x; Bv[j][1] = bw.y; Bv[j][2] = bw.z; Bv[j][3] = bw.w;
            Cv[j][0] = cw.x; Cv[j][1] = cw.y; Cv[j][2] = cw.z; Cv[j][3] = cw.w;
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                Bv[j][i] = io<IO>::ld(B, bo + i);
                Cv[j][i] = io<IO>::ld(C, bo + i);
            }
        }
    }

#pragma unroll
    for (int j = 0; j < SP; ++j) {
        const bool act = s0 + j < S;        // the same for the G lanes of a group
        if constexpr (ACT > 0) {
            const float x = dt[j] + bd;
            dt[j] = softplus ? (sizeof(IO) == 2 ? softplus_short_f32(x) : softplus_f32(x)) : x;
        }
        const float k = ACT == 2 ? uu[j] : dt[j] * uu[j];
        float acc = 0.0f;
        float hn[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const float ya = dt[j] * a2[i];
            const float e = hw_exp2(ya);
            float bu = k * Bv[j][i];
            if constexpr (ACT == 2) bu *= zoh_weight(ya, e, dt[j], inv_a[i]);
            hn[i] = fmaf(e, h[j][i], bu);
            acc = fmaf(Cv[j][i], hn[i], acc);
        }
        const int64_t pair = (s0 + j) * D + d;
        if (act) {
            float *row = state + pair * N + part * NS;
            if constexpr (NS == 4) {
                const f32x4_t v = {hn[0], hn[1], hn[2], hn[3]};
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t *>(row));
            } else {
#pragma unroll
                for (int i = 0; i < NS; ++i) __builtin_nontemporal_store(hn[i], row + i);
            }
        }
        // add the G partial readouts of one (s, d): lanes of a group are adjacent within a quad
        if constexpr (G >= 2)
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xf, 0xf, true));  // quad_perm [1,0,3,2]
        if constexpr (G >= 4)
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xf, 0xf, true));  // quad_perm [2,3,0,1]
        if (act && part == 0) {
            float yv = Dv ? fmaf(Dd, uu[j], acc) : acc;
            if (z) yv *= silu_f32(zz[j]);
            io<IO>::st(y, pair, yv);
        }
    }
}

}  // namespace ssm

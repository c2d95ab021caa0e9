// The single-token recurrent step (the constant-memory inference form:
// shakilmahmud.com section 3; urworte.de "Methodische Grundlagen").
//
// Per (sequence s, channel d) the fp32 state row state[s][d][0..N) is read, updated in
// place and y[s][d] written.  The step is bound by the state traffic (2 * 4N bytes per
// (s, d)), so the mapping is chosen for coalescing: G = N/4 lanes share one (s, d), each
// moving 16 contiguous bytes of its state row, so a wave streams 1 KiB of contiguous
// state.  The partial readouts of the G lanes are added with DPP quad permutes.
#pragma once

#include "device_math.h"

namespace ssm {

template <int N, typename IO>
__global__ void __launch_bounds__(256)
step_kernel(float *__restrict__ state, const IO *__restrict__ u, const IO *__restrict__ delta,
            const float *__restrict__ A, const IO *__restrict__ B, const IO *__restrict__ C,
            const float *__restrict__ Dv, const IO *__restrict__ z, IO *__restrict__ y,
            int64_t S, int64_t D) {
    constexpr int G = N >= 4 ? N / 4 : 1;  // lanes per (s, d)
    constexpr int NS = N / G;              // states per lane
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t pair = gid / G;
    const int part = (int)(gid - pair * G);
    const bool act = pair < S * D;
    const int64_t s = act ? pair / D : 0;
    const int64_t d = act ? pair - s * D : 0;

    float h[NS];
    float acc = 0.0f;
    float uu = 0.0f;
    if (act) {
        float *row = state + pair * N + part * NS;
        if constexpr (NS == 4) {
            const float4 v = *reinterpret_cast<const float4 *>(row);
            h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) h[i] = row[i];
        }
        const float dt = io<IO>::ld(delta, pair);
        uu = io<IO>::ld(u, pair);
        const float k = dt * uu;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int n = part * NS + i;
            const float e = hw_exp2(dt * (A[d * N + n] * kLog2e));
            h[i] = fmaf(e, h[i], k * io<IO>::ld(B, s * N + n));
            acc = fmaf(io<IO>::ld(C, s * N + n), h[i], acc);
        }
        if constexpr (NS == 4) {
            *reinterpret_cast<float4 *>(row) = make_float4(h[0], h[1], h[2], h[3]);
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) row[i] = h[i];
        }
    }
    // add the G partial readouts of one (s, d): lanes of a group are adjacent within a quad
    if constexpr (G >= 2)
        acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xf, 0xf, true));  // quad_perm [1,0,3,2]
    if constexpr (G >= 4)
        acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xf, 0xf, true));  // quad_perm [2,3,0,1]
    if (act && part == 0) {
        float yv = acc;
        if (Dv) yv += Dv[d] * uu;
        if (z) yv *= silu_f32(io<IO>::ld(z, pair));
        io<IO>::st(y, pair, yv);
    }
}

}  // namespace ssm

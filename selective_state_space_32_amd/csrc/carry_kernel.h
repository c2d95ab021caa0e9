// Pass 2 of the chunked scan: the prefix over chunks.
//
// The recurrence h_t = a_t h_{t-1} + b_t is associative under
//     (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2)
// (azimuth.plus/paper/mamba, hardware-aware algorithm section, parallel-scan bullet), so a
// chunk c of the sequence acts on the state as the pair (P_c, hc_c): P_c[n] = exp(A[n] *
// sum of the chunk's step sizes) and hc_c = the chunk's final state when started from 0.
// The state after chunk c is the inclusive prefix H_c = (P_0,hc_0) o ... o (P_c,hc_c)
// applied to the initial state (zero unless one is given).  Here one wave64 computes that
// prefix for 64 chunks at once, lane =
// chunk, with a DPP scan: row_shr 1, 2, 4, 8 inside rows of 16 lanes, then row_bcast 15
// and row_bcast 31 across rows (6 steps).  Lanes with no predecessor at a step combine
// with the identity (1, 0).  Longer chunk lists are processed 64 at a time, carrying the
// running state across blocks.
#pragma once

#include "device_math.h"

namespace ssm {

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or(float v, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xf, false));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_step(float &a, float &b) {
    const float ap = dpp_or<CTRL, ROW_MASK>(a, 1.0f);
    const float bp = dpp_or<CTRL, ROW_MASK>(b, 0.0f);
    b = fmaf(a, bp, b);
    a = a * ap;
}

// Inclusive wave64 scan of (a, b) pairs under the operator above (lane order = sequence order).
__device__ __forceinline__ void wave_scan_pairs(float &a, float &b) {
    scan_step<0x111, 0xf>(a, b);  // row_shr:1
    scan_step<0x112, 0xf>(a, b);  // row_shr:2
    scan_step<0x114, 0xf>(a, b);  // row_shr:4
    scan_step<0x118, 0xf>(a, b);  // row_shr:8
    scan_step<0x142, 0xa>(a, b);  // row_bcast:15 -> rows 1 and 3
    scan_step<0x143, 0xc>(a, b);  // row_bcast:31 -> rows 2 and 3
}

// cstate: [bsz][nchunk][D*N] -- in: local final states of chunks 0..nchunk-2;
//         out: the state after each of those chunks (the carry into the next chunk),
//         starting from h0; slot nchunk-1 receives a copy of h0 (when h0 is given) for
//         the first chunk of the last pass.
// cdsum:  [bsz][nchunk][D] sums of step sizes per chunk.
// h0:     [bsz][D*N] initial state, or null for zero.
// One workgroup = one sequence x 64 consecutive (d, n) columns; 4 waves x 16 columns.
template <int N>
__global__ void __launch_bounds__(256)
carry_scan_kernel(float *__restrict__ cstate, const float *__restrict__ cdsum,
                  const float *__restrict__ A, const float *__restrict__ h0, int64_t D, int nchunk,
                  int col_tiles) {
    __shared__ float s_a[64][65];
    __shared__ float s_b[64][65];
    const int64_t DN = D * N;
    const int b = blockIdx.x / col_tiles;
    const int64_t dn0 = (int64_t)(blockIdx.x - b * col_tiles) * 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int nc = nchunk - 1;  // chunks whose summary carries into a later chunk

    const int64_t dn = dn0 + lane;  // column this thread loads / stores
    const bool ok = dn < DN;
    const int64_t dcol = dn / N;
    const float a2 = ok ? A[dn] * kLog2e : 0.0f;

    // the running state of column w*16+k (the same in every lane), from the initial state
    float carry[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t col = dn0 + w * 16 + k;
        carry[k] = (h0 && col < DN) ? h0[(int64_t)b * DN + col] : 0.0f;
    }
    if (h0 && ok) cstate[((int64_t)b * nchunk + nchunk - 1) * DN + dn] = h0[(int64_t)b * DN + dn];

    for (int c0 = 0; c0 < nc; c0 += 64) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = w + 4 * i;
            const int c = c0 + r;
            float av = 1.0f, bv = 0.0f;
            if (ok && c < nc) {
                const int64_t row = (int64_t)b * nchunk + c;
                av = hw_exp2(a2 * cdsum[row * D + dcol]);
                bv = cstate[row * DN + dn];
            }
            s_a[r][lane] = av;
            s_b[r][lane] = bv;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int col = w * 16 + k;
            float av = s_a[lane][col];
            float bv = s_b[lane][col];
            wave_scan_pairs(av, bv);
            const float H = fmaf(av, carry[k], bv);
            s_b[lane][col] = H;
            carry[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(H), 63));
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = w + 4 * i;
            const int c = c0 + r;
            if (ok && c < nc) cstate[((int64_t)b * nchunk + c) * DN + dn] = s_b[r][lane];
        }
        __syncthreads();
    }
}

}  // namespace ssm

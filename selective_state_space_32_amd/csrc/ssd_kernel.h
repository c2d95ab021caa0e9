// Mamba-2's state space dual layer (SSD) in its chunked matrix form on the matrix cores.
//
// With a scalar state matrix a_h per head the sequence map of the selective scan is a
// 1-semiseparable matrix, so a chunk of Q tokens can be computed with matrix products
// (mugbit.ir, the Mamba-2 / structured state space duality section).  Per head h (P
// channels, its group's B and C) and chunk, with dt the step sizes and
// c_t = a_h * (dt_0 + ... + dt_t) the running log-decay inside the chunk:
//   G      = C B^T                                  (Q x Q, contraction over the N states)
//   M[t,s] = G[t,s] exp(c_t - c_s) dt_s for s <= t, 0 above the diagonal
//   Y      = M X + diag(exp(c_t)) C H               (H: the P x N state entering the chunk,
//                                                    used here as H^T, N x P)
//   H^T    <- exp(c_{Q-1}) H^T + X^T Bw,  Bw[s,n] = B[s,n] exp(c_{Q-1} - c_s) dt_s
//   y      = (Y + D x) * silu(z)
// Each of the four products is 64 x 64 x 64 here (Q = P = N = 64): one workgroup per
// (sequence, head), four waves, each owning one 32 x 32 quadrant of every product, computed
// with v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulation).  x, B and C are bf16
// inputs, exact as operands; the operands formed here (M, Bw and the state's copy) are split
// into a bf16 high part and a bf16 low part (v - hi), each multiplied, so that they keep
// about 16 bits of their fp32 value.  Operands are staged in LDS with the contraction index
// contiguous (X and B transposed while staging), so each operand fetch is one 16-byte LDS
// read per lane.  The state stays in fp32 accumulators across chunks.  The next chunk's
// inputs are fetched into registers while the current chunk is computed.
#pragma once

#include "device_math.h"

namespace ssm {

constexpr int kSsdQ = 64;          // tokens per chunk
constexpr int kSsdP = 64;          // channels per head
constexpr int kSsdN = 64;          // states
// LDS tiles are 64 x 64 bf16 in rows of 72 (144 bytes: 16-byte aligned, and 16-byte reads of
// eight consecutive rows fall in distinct banks); element (row, k) is at sw(row, k).
constexpr int kSsdLd = 72;
__device__ __forceinline__ int sw(int row, int k) { return row * kSsdLd + k; }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// One 32 x 32 block of A B over a contraction of 16 * KS: A rows from tile `a` starting at
// row a0, B columns from tile `b` ([col][k]) starting at row b0 (multiples of 8); the lane
// fetches its 8 consecutive k of row / column (lane % 32) at offset 8 * (lane / 32) of each
// 16-wide step.
template <int KS>
__device__ __forceinline__ f32x16_t mma_block(const __bf16 *a, int a0, const __bf16 *b, int b0, int lane,
                                              f32x16_t acc) {
    const int r = lane & 31, ko = (lane >> 5) * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(a + sw(a0 + r, 16 * k + ko));
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(b + sw(b0 + r, 16 * k + ko));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
    return acc;
}

// Row (within the 32 x 32 block) of accumulator element e of this lane; the column is lane % 32.
__device__ __forceinline__ int acc_row(int e, int lane) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

// Inclusive sum over the 64 lanes of a wave (DPP: row_shr 1, 2, 4, 8, row_bcast 15, 31).
__device__ __forceinline__ float wave_incl_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return v;
}

// x, z, y: [bsz][L][H][P] bf16;  dt: [bsz][L][H] bf16;  A, Dv, dt_bias: [H] fp32;
// B, C: [bsz][L][G][N] bf16;  last_state: [bsz][H][P][N] fp32 (or null).
// LDS: eight padded 64 x 72 tiles and an unpadded 64 x 64 one (80 KB, two workgroups per CU);
// the chunk's per-token values live in the padding of the C tile.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
ssd_chunk_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ dt, const float *__restrict__ A,
                 const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dv,
                 const uint16_t *__restrict__ z, const float *__restrict__ dt_bias, uint16_t *__restrict__ y,
                 float *__restrict__ last_state, int64_t L, int H, int G, int softplus) {
    constexpr int Q = kSsdQ, P = kSsdP, N = kSsdN, LD = kSsdLd;
    __shared__ __attribute__((aligned(16))) __bf16 sC[Q * LD];     // C   [t][n]; padding: c_t, dt_t
    __shared__ __attribute__((aligned(16))) __bf16 sBM[Q * LD];    // B   [s][n], then M (high part) [t][s]
    __shared__ __attribute__((aligned(16))) __bf16 sMl[Q * LD];    // M low part [t][s]
    __shared__ __attribute__((aligned(16))) __bf16 sXt[P * LD];    // X^T [p][s]
    __shared__ __attribute__((aligned(16))) __bf16 sBwh[N * LD];   // Bw^T [n][s], high and low parts
    __shared__ __attribute__((aligned(16))) __bf16 sBwl[N * LD];
    __shared__ __attribute__((aligned(16))) __bf16 sHth[P * LD];   // H^T [p][n], high and low parts
    __shared__ __attribute__((aligned(16))) __bf16 sHtl[P * LD];
    __shared__ __attribute__((aligned(16))) __bf16 sZ[Q * 64];     // z [t][p], then y [t][p] (unpadded)
    // c_t (the running log2-decay of token t) and dt_t, in the padding of row t of the C tile
    auto cum2 = [&](int t) -> float & { return *reinterpret_cast<float *>(&sC[t * LD + 64]); };
    auto dts = [&](int t) -> float & { return *reinterpret_cast<float *>(&sC[t * LD + 66]); };
    auto split = [](float v, __bf16 &hi, __bf16 &lo) {
        hi = (__bf16)v;
        lo = (__bf16)(v - (float)hi);
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qi = w >> 1, qj = w & 1;               // this wave's quadrant: rows 32 qi, columns 32 qj
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int g = h / (H / G);
    const float a2 = A[h] * kLog2e;                   // decays as exp2(a2 * sum of dt)
    const float bias_h = dt_bias ? dt_bias[h] : 0.0f;
    const float d_h = Dv ? Dv[h] : 0.0f;
    const int64_t xrow = (int64_t)H * P;              // elements between tokens in x, z, y
    const int64_t brow = (int64_t)G * N;              // ... in B, C

    // staging maps: C, z and y rows coalesced (token tid / 8 + 32 i, 8 elements at 8 (tid % 8));
    // X and B by token = lane (8 channels / states at group w + 4 i), so that the transposed
    // LDS writes of one instruction fall in distinct banks.  Each thread stores the y rows of
    // exactly the z slots it fills with the next chunk's z.
    struct Raw { u32x4_t c[2], xv[2], bv[2], zv[2]; uint32_t dt; };
    auto fetch = [&](int64_t t0, Raw &r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t tc = min(t0 + tid / 8 + 32 * i, L - 1);
            r.c[i] = *reinterpret_cast<const u32x4_t *>(Cm + ((int64_t)b * L + tc) * brow + (int64_t)g * N + (tid % 8) * 8);
            if (z) r.zv[i] = *reinterpret_cast<const u32x4_t *>(z + ((int64_t)b * L + tc) * xrow + (int64_t)h * P + (tid % 8) * 8);
            const int64_t ts = min(t0 + lane, L - 1);
            const int grp = w + 4 * i;
            r.xv[i] = *reinterpret_cast<const u32x4_t *>(x + ((int64_t)b * L + ts) * xrow + (int64_t)h * P + grp * 8);
            r.bv[i] = *reinterpret_cast<const u32x4_t *>(Bm + ((int64_t)b * L + ts) * brow + (int64_t)g * N + grp * 8);
        }
        r.dt = dt[((int64_t)b * L + min(t0 + lane, L - 1)) * H + h];
    };
    auto lo16 = [](uint32_t v) { return __builtin_bit_cast(__bf16, (uint16_t)(v & 0xffffu)); };
    auto hi16 = [](uint32_t v) { return __builtin_bit_cast(__bf16, (uint16_t)(v >> 16)); };

    f32x16_t Hacc = {};                                // this wave's 32 x 32 block of H^T [p][n], fp32
    for (int i = tid; i < P * LD; i += 256) sHth[i] = sHtl[i] = __builtin_bit_cast(__bf16, (uint16_t)0);   // (any order)

    Raw r;
    fetch(0, r);
    const int64_t nchunks = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * Q;
        const int nt = (int)min((int64_t)Q, L - t0);
        // --- stage the chunk (C, B, z natural; X^T transposed), then fetch the next one
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<u32x4_t *>(&sC[sw(tid / 8 + 32 * i, (tid % 8) * 8)]) = r.c[i];
            if (z) *reinterpret_cast<u32x4_t *>(&sZ[(tid / 8 + 32 * i) * 64 + (tid % 8) * 8]) = r.zv[i];
            const int grp = w + 4 * i;
            *reinterpret_cast<u32x4_t *>(&sBM[sw(lane, grp * 8)]) = r.bv[i];
            const uint32_t xw[4] = {r.xv[i].x, r.xv[i].y, r.xv[i].z, r.xv[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sXt[sw(grp * 8 + 2 * k, lane)] = lo16(xw[k]);
                sXt[sw(grp * 8 + 2 * k + 1, lane)] = hi16(xw[k]);
            }
        }
        if (w == 0) {   // step sizes and their running sum (padded tokens: identity steps)
            const float v = bf16_to_f32((uint16_t)r.dt) + bias_h;
            const float d = lane < nt ? (softplus ? softplus_f32(v) : v) : 0.0f;
            dts(lane) = d;
            cum2(lane) = a2 * wave_incl_sum(d);
        }
        if (c + 1 < nchunks) fetch(t0 + Q, r);
        __syncthreads();
        const float ctot = cum2(Q - 1);
        // --- Bw^T [n][s] = B[s][n] exp2(c_last - c_s) dt_s, B read back from the tile (token = lane)
        {
            const float ws = hw_exp2(ctot - cum2(lane)) * dts(lane);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int grp = w + 4 * i;
                const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(&sBM[sw(lane, grp * 8)]);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int o = sw(grp * 8 + k, lane);
                    split((float)bv[k] * ws, sBwh[o], sBwl[o]);
                }
            }
        }
        // --- M = (C B^T) o decay o dt, this wave's quadrant (rows t = 32 qi.., columns s = 32 qj..)
        {
            f32x16_t Gacc = {};
            if (qj <= qi) Gacc = mma_block<N / 16>(sC, 32 * qi, sBM, 32 * qj, lane, Gacc);
            __syncthreads();   // every wave is done with B: M takes its place
            const int s = 32 * qj + (lane & 31);
            const float cs = cum2(s), ds = dts(s);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = 32 * qi + acc_row(e, lane);
                float m = Gacc[e] * hw_exp2(cum2(t) - cs) * ds;
                if (qi == qj) m = s <= t ? m : 0.0f;   // the quadrant above the diagonal is all zero
                split(m, sBM[sw(t, s)], sMl[sw(t, s)]);
            }
        }
        __syncthreads();
        // --- Y = M X + diag(exp2(c_t)) C H   (rows t = 32 qi.., columns p = 32 qj..)
        f32x16_t Y = {}, Y3 = {};
        if (qi == 0) {   // M is zero for s > t
            Y = mma_block<2>(sBM, 0, sXt, 32 * qj, lane, Y);
            Y = mma_block<2>(sMl, 0, sXt, 32 * qj, lane, Y);
        } else {
            Y = mma_block<Q / 16>(sBM, 32, sXt, 32 * qj, lane, Y);
            Y = mma_block<Q / 16>(sMl, 32, sXt, 32 * qj, lane, Y);
        }
        Y3 = mma_block<N / 16>(sC, 32 * qi, sHth, 32 * qj, lane, Y3);
        Y3 = mma_block<N / 16>(sC, 32 * qi, sHtl, 32 * qj, lane, Y3);
        // --- output: y = (Y + exp2(c_t) Y3 + D x) * silu(z), into the z slot it replaces
        {
            const int p = 32 * qj + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = 32 * qi + acc_row(e, lane);
                float v = fmaf(hw_exp2(cum2(t)), Y3[e], Y[e]);
                v = fmaf(d_h, (float)sXt[sw(p, t)], v);
                if (z) v *= silu_f32((float)sZ[t * 64 + p]);
                sZ[t * 64 + p] = (__bf16)v;
            }
        }
        // --- H^T <- exp2(c_last) H^T + X^T Bw   (rows p = 32 qi.., columns n = 32 qj..)
        {
            const float dec = hw_exp2(ctot);
#pragma unroll
            for (int e = 0; e < 16; ++e) Hacc[e] *= dec;
            Hacc = mma_block<Q / 16>(sXt, 32 * qi, sBwh, 32 * qj, lane, Hacc);
            Hacc = mma_block<Q / 16>(sXt, 32 * qi, sBwl, 32 * qj, lane, Hacc);
        }
        __syncthreads();   // every read of this chunk's LDS is done, y is complete in sZ
        {
            const int n = 32 * qj + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int o = sw(32 * qi + acc_row(e, lane), n);
                split(Hacc[e], sHth[o], sHtl[o]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {   // y rows, 16 bytes per thread
                const int t = tid / 8 + 32 * i;
                if (t < nt)
                    *reinterpret_cast<u32x4_t *>(y + ((int64_t)b * L + t0 + t) * xrow + (int64_t)h * P + (tid % 8) * 8) =
                        *reinterpret_cast<const u32x4_t *>(&sZ[t * 64 + (tid % 8) * 8]);
            }
        }
    }
    if (last_state) {
        const int n = 32 * qj + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int p = 32 * qi + acc_row(e, lane);
            last_state[(((int64_t)b * H + h) * P + p) * N + n] = Hacc[e];
        }
    }
}

}  // namespace ssm

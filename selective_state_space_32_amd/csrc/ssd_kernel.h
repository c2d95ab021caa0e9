// Mamba-2's state space dual layer (SSD) in its chunked matrix form on the matrix cores.
//
// With a scalar state matrix a_h per head the sequence map of the selective scan is a
// 1-semiseparable matrix, so a chunk of Q tokens can be computed with matrix products
// (mugbit.ir, the Mamba-2 / structured state space duality section).  Per head h (P
// channels, its group's B and C) and chunk, with dt the step sizes and
// c_t = a_h * (dt_0 + ... + dt_t) the running log-decay inside the chunk:
//   G      = C B^T                                  (Q x Q, contraction over the N states)
//   M[t,s] = G[t,s] exp(c_t - c_s) dt_s for s <= t, 0 above the diagonal
//   Y      = M X + diag(exp(c_t)) C H^T             (H: the N x P state entering the chunk)
//   H      <- exp(c_{Q-1}) H + Bw^T X,  Bw[s,n] = B[s,n] exp(c_{Q-1} - c_s) dt_s
//   y      = (Y + D x) * silu(z)
// Each product is 64 x 64 x 64 here (Q = P = N = 64): one workgroup per (sequence, head),
// four waves, each owning one 32 x 32 quadrant of every product, computed with
// v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulation).  The products are taken
// transposed (G^T = B C^T, Y^T = X^T M^T, and the state as H[n][p]), so that the four
// consecutive accumulator rows a lane holds are four consecutive elements of the operand
// tile they are written to (one 8-byte LDS write) and each lane's output column is one
// token.  D x is folded into M as D on its diagonal.  x, B and C are bf16 inputs, exact as
// operands; the operands formed here (M, Bw and the state's copy) are split into a bf16 high
// part and a bf16 low part (v - hi), each multiplied, so that they keep about 16 bits of
// their fp32 value.  Operands are staged in LDS with the contraction index contiguous (X and
// B transposed while staging), so each operand fetch is one 16-byte LDS read per lane.  The
// state stays in fp32 accumulators across chunks.  The next chunk's inputs are fetched into
// registers while the current chunk is computed (unconditionally -- the last chunk fetches
// itself again -- so that the loads land in the loop's own registers and are waited for only
// when the next chunk is staged).  Five operand tiles and a z / y tile (52 KB of LDS) serve
// every phase of a chunk.
#pragma once

#include "device_math.h"

namespace ssm {

constexpr int kSsdQ = 64;          // tokens per chunk
constexpr int kSsdP = 64;          // channels per head
constexpr int kSsdN = 64;          // states
// Operand tiles are 64 x 64 bf16, element (row, k) at sw(row, k): rows of 72 (144 bytes:
// 16-byte aligned, and 16-byte reads of eight consecutive rows fall in distinct banks), or,
// for the C tile, swz(row, k): unpadded rows whose 16-byte unit k / 8 is stored at unit
// (k / 8) ^ (row % 8), which spreads the same reads over all banks.
constexpr int kSsdLd = 72;
__device__ __forceinline__ int sw(int row, int k) { return row * kSsdLd + k; }
__device__ __forceinline__ int swz(int row, int k) { return row * 64 + ((((k >> 3) ^ row) & 7) << 3) + (k & 7); }
template <bool Z> __device__ __forceinline__ int tix(int row, int k) { return Z ? swz(row, k) : sw(row, k); }
// The z / y tile [t][p] has unpadded rows of 64; its 8-byte unit u (p / 4) of row t is stored
// at unit u ^ (t % 16), so that the output layout's 8-byte accesses (32 rows, one unit) and
// the 16-byte row accesses both spread over all banks.
__device__ __forceinline__ int zsw8(int t, int u) { return t * 64 + ((u ^ (t & 15)) << 2); }
// 16-byte unit v of row t: units 2v, 2v+1 land in unit v ^ (t % 16 / 2), halves swapped for odd t
__device__ __forceinline__ int zsw16(int t, int v) { return t * 64 + ((v ^ ((t & 15) >> 1)) << 3); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One 32 x 32 block of A B over a contraction of 16 * KS: A rows from tile `a` starting at
// row a0, B columns from tile `b` ([col][k]) starting at row b0 (multiples of 8; ZA / ZB:
// the tile is swizzled); the lane fetches its 8 consecutive k of row / column (lane % 32) at
// offset 8 * (lane / 32) of each 16-wide step.
template <int KS, bool ZA = false, bool ZB = false>
__device__ __forceinline__ f32x16_t mma_block(const __bf16 *a, int a0, const __bf16 *b, int b0, int lane,
                                              f32x16_t acc) {
    const int r = lane & 31, ko = (lane >> 5) * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(a + tix<ZA>(a0 + r, 16 * k + ko));
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(b + tix<ZB>(b0 + r, 16 * k + ko));
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
//
// Tiles and their phases within a chunk (barriers 1-4):
//   tC : C [t][n] (swizzled)          -> (2) M low part [t][s]
//   tB : B [s][n]                     -> (2) M high part [t][s]
//   tX : X^T [p][s]; its row padding holds per-token values
//   tH1: the state's copy H^T [p][n], high part  -> (2) Bw^T [n][s] high part -> (4) H^T high
//   tH2: the same, low parts
//   tZ : z [t][p]                     -> (3) y, in place
// Between 1 and 2: Y3^T = H^T C^T and G^T = B C^T; between 2 and 3: M and Bw written; between
// 3 and 4: the state update, Y^T = X^T M^T and the output; after 4: the new H^T, y out to
// HBM, and the next chunk's C, B, X^T, z.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
ssd_chunk_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ dt, const float *__restrict__ A,
                 const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dv,
                 const uint16_t *__restrict__ z, const float *__restrict__ dt_bias, uint16_t *__restrict__ y,
                 float *__restrict__ last_state, int64_t L, int H, int G, int softplus) {
    constexpr int Q = kSsdQ, P = kSsdP, N = kSsdN, LD = kSsdLd;
    static_assert(Q == 64 && P == 64 && N == 64, "one 32 x 32 quadrant per wave of four");
    constexpr bool ZC = true;                         // tC is swizzled
    __shared__ __attribute__((aligned(16))) __bf16 tC[Q * 64];
    __shared__ __attribute__((aligned(16))) __bf16 tB[Q * LD];
    __shared__ __attribute__((aligned(16))) __bf16 tX[P * LD];
    __shared__ __attribute__((aligned(16))) __bf16 tH1[P * LD];
    __shared__ __attribute__((aligned(16))) __bf16 tH2[P * LD];
    __shared__ __attribute__((aligned(16))) __bf16 tZ[Q * 64];
    // per-token values, four tokens per row padding of tX (tokens 4r..4r+3 in row r): c_t (in
    // log2 units) and f_s = exp2(c_r - c_s) dt_s with r the first token of s's half-chunk
    // (dt_s = 0 for tokens past the end)
    float *const s_pad = reinterpret_cast<float *>(tX + 64);   // row r at s_pad + r * LD / 2
    auto s_c4 = [&](int t) -> float * { return s_pad + (t >> 2) * (LD / 2) + (t & 3); };
    auto s_f4 = [&](int t) -> float * { return s_pad + (16 + (t >> 2)) * (LD / 2) + (t & 3); };
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qi = w >> 1, qj = w & 1;                // this wave's quadrant: rows 32 qi, columns 32 qj
    const int col = 32 * qj + (lane & 31);            // the lane's accumulator column
    const int rq = (lane >> 5) * 4;                   // its rows: 32 qi + 8 gq + rq + (0..3), gq < 4
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int g = h / (H / G);
    const float a2 = A[h] * kLog2e;                   // decays as exp2(a2 * sum of dt)
    const float bias_h = dt_bias ? dt_bias[h] : 0.0f;
    const float d_h = Dv ? Dv[h] : 0.0f;
    const int64_t xrow = (int64_t)H * P;              // elements between tokens in x, z, y
    const int64_t brow = (int64_t)G * N;              // ... in B, C
    const uint16_t *xh = x + (int64_t)b * L * xrow + (int64_t)h * P;
    const uint16_t *zh = z ? z + (int64_t)b * L * xrow + (int64_t)h * P : nullptr;
    uint16_t *yh = y + (int64_t)b * L * xrow + (int64_t)h * P;
    const uint16_t *Bg = Bm + (int64_t)b * L * brow + (int64_t)g * N;
    const uint16_t *Cg = Cm + (int64_t)b * L * brow + (int64_t)g * N;

    // staging maps: C and z rows coalesced (token tid / 8 + 32 i, 8 elements at 8 (tid % 8));
    // X and B by token = lane (8 channels / states at group w + 4 i), so that the transposed
    // LDS writes of one instruction fall in distinct banks.  Addresses: the chunk's base
    // (uniform) plus a 32-bit offset per lane (64 rows of H P elements fit 32 bits).  z is read
    // and y written once: streaming (non-temporal) accesses; x and B rows are read by eight
    // instructions in 16-byte pieces and stay cached.
    struct Raw { u32x4_t c[2], xv[2], bv[2], zv[2]; uint32_t dt; };
    const uint32_t xr32 = (uint32_t)xrow, br32 = (uint32_t)brow;
    auto fetch = [&](int64_t t0, Raw &r) {
        const uint32_t lim = (uint32_t)min((int64_t)(Q - 1), L - 1 - t0);   // last token present
        const uint16_t *xc = xh + t0 * xrow, *bc = Bg + t0 * brow, *cc = Cg + t0 * brow;
        const uint32_t ts = min((uint32_t)lane, lim);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t tc = min((uint32_t)(tid / 8 + 32 * i), lim);
            r.c[i] = *reinterpret_cast<const u32x4_t *>(cc + (tc * br32 + (uint32_t)(tid % 8) * 8));
            if (zh)
                r.zv[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t *>(zh + t0 * xrow + (tc * xr32 + (uint32_t)(tid % 8) * 8)));
            const uint32_t grp = (uint32_t)(w + 4 * i);
            r.xv[i] = *reinterpret_cast<const u32x4_t *>(xc + (ts * xr32 + grp * 8));
            r.bv[i] = *reinterpret_cast<const u32x4_t *>(bc + (ts * br32 + grp * 8));
        }
        r.dt = dt[((int64_t)b * L + t0) * H + h + ts * (uint32_t)H];
    };
    auto lo16 = [](uint32_t v) { return __builtin_bit_cast(__bf16, (uint16_t)(v & 0xffffu)); };
    auto hi16 = [](uint32_t v) { return __builtin_bit_cast(__bf16, (uint16_t)(v >> 16)); };
    auto split = [](float v, __bf16 &hi, __bf16 &lo) {
        hi = (__bf16)v;
        lo = (__bf16)(v - (float)hi);
    };

    f32x16_t S = {};                                   // this wave's 32 x 32 block of H [n][p], fp32
    Raw r;
    fetch(0, r);
    const int64_t nchunks = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * Q;
        const int nt = (int)min((int64_t)Q, L - t0);
        // --- stage C, z, B (natural) and X^T (transposed); the step sizes and their running
        //     sum, token = lane, in every wave
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tr = tid / 8 + 32 * i;
            *reinterpret_cast<u32x4_t *>(&tC[tix<ZC>(tr, (tid % 8) * 8)]) = r.c[i];
            if (zh) {
                const u32x4_t zv = (tr & 1) ? u32x4_t{r.zv[i].z, r.zv[i].w, r.zv[i].x, r.zv[i].y} : r.zv[i];
                *reinterpret_cast<u32x4_t *>(&tZ[zsw16(tr, tid % 8)]) = zv;
            }
            const int grp = w + 4 * i;
            *reinterpret_cast<u32x4_t *>(&tB[sw(lane, grp * 8)]) = r.bv[i];
            const uint32_t xw[4] = {r.xv[i].x, r.xv[i].y, r.xv[i].z, r.xv[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                tX[sw(grp * 8 + 2 * k, lane)] = lo16(xw[k]);
                tX[sw(grp * 8 + 2 * k + 1, lane)] = hi16(xw[k]);
            }
        }
        const float v = bf16_to_f32((uint16_t)r.dt) + bias_h;
        const float dl = lane < nt ? (softplus ? softplus_f32(v) : v) : 0.0f;   // padded tokens: identity steps
        const float cl = a2 * wave_incl_sum(dl);
        const float ctot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 63));
        const float c32 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 32));
        const float cref = qi ? c32 : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 0));
        if (w == 0) {
            const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 0));
            *s_c4(lane) = cl;
            *s_f4(lane) = hw_exp2((lane < 32 ? c0 : c32) - cl) * dl;
        }
        const float wsl = hw_exp2(ctot - cl) * dl;    // Bw weight of token lane
        const u32x4_t bcur[2] = {r.bv[0], r.bv[1]};
        fetch(min(t0 + Q, (nchunks - 1) * Q), r);   // (the last chunk fetches itself again, unused)
        __syncthreads();                                // (1)
        // --- Y3^T = H^T C^T (the state entering the chunk) and G^T = B C^T
        f32x16_t Y = {};
        if (c > 0) {
            Y = mma_block<N / 16, false, ZC>(tH1, 32 * qi, tC, 32 * qj, lane, Y);
            Y = mma_block<N / 16, false, ZC>(tH2, 32 * qi, tC, 32 * qj, lane, Y);
        }
        f32x16_t Gt = {};
        if (qi <= qj) Gt = mma_block<N / 16, false, ZC>(tB, 32 * qi, tC, 32 * qj, lane, Gt);   // zero for s > t
        __syncthreads();                                // (2)
        // --- M [t][s] = G^T[s][t] exp2(c_t - c_s) dt_s (s <= t) + D (s = t): rows s of this
        //     wave's quadrant, column t; four consecutive s per 8-byte write.  The decay is
        //     exp2(c_t - c_r) f_s with r = 32 qi <= s <= t: both factors are at most 1 (times
        //     dt_s), as c does not increase along the chunk (a <= 0, dt >= 0).
        if (qi <= qj) {
            const float et = hw_exp2(*s_c4(col) - cref);
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int s0 = 32 * qi + 8 * gq + rq;
                const f32x4_t fs = *reinterpret_cast<const f32x4_t *>(s_f4(s0));
                const float fsv[4] = {fs.x, fs.y, fs.z, fs.w};
                bf16x4_t mh, ml;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float m = Gt[4 * gq + j] * et * fsv[j];
                    if (qi == qj) {
                        m = s0 + j <= col ? m : 0.0f;
                        if (s0 + j == col) m += d_h;
                    }
                    __bf16 hi, lo;
                    split(m, hi, lo);
                    mh[j] = hi;
                    ml[j] = lo;
                }
                *reinterpret_cast<bf16x4_t *>(&tB[sw(col, s0)]) = mh;
                *reinterpret_cast<bf16x4_t *>(&tC[tix<ZC>(col, s0)]) = ml;
            }
        }
        // --- Bw^T [n][s] = B[s][n] exp2(c_last - c_s) dt_s, token s = lane
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int grp = w + 4 * i;
            const uint32_t bw[4] = {bcur[i].x, bcur[i].y, bcur[i].z, bcur[i].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int o = sw(grp * 8 + 2 * k, lane);
                split(bf16_to_f32((uint16_t)(bw[k] & 0xffffu)) * wsl, tH1[o], tH2[o]);
                split(bf16_to_f32((uint16_t)(bw[k] >> 16)) * wsl, tH1[o + LD], tH2[o + LD]);
            }
        }
        __syncthreads();                                // (3)
        // --- H [n][p] <- exp2(c_last) H + Bw^T X   (rows n = 32 qi.., columns p = 32 qj..)
        {
            const float dec = hw_exp2(ctot);
#pragma unroll
            for (int e = 0; e < 16; ++e) S[e] *= dec;
            S = mma_block<Q / 16>(tH1, 32 * qi, tX, 32 * qj, lane, S);
            S = mma_block<Q / 16>(tH2, 32 * qi, tX, 32 * qj, lane, S);
        }
        // --- Y^T = X^T M^T + exp2(c_t) Y3^T   (rows p = 32 qi.., columns t = 32 qj..)
        {
            const float et = hw_exp2(*s_c4(col));
#pragma unroll
            for (int e = 0; e < 16; ++e) Y[e] *= et;
            if (qj == 0) {   // M is zero for s > t
                Y = mma_block<2>(tX, 32 * qi, tB, 0, lane, Y);
                Y = mma_block<2, false, ZC>(tX, 32 * qi, tC, 0, lane, Y);
            } else {
                Y = mma_block<Q / 16>(tX, 32 * qi, tB, 32, lane, Y);
                Y = mma_block<Q / 16, false, ZC>(tX, 32 * qi, tC, 32, lane, Y);
            }
        }
        // --- y = Y * silu(z), token col, channels 32 qi + 8 gq + rq .. +3: into the z slot
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int o8 = zsw8(col, 8 * qi + 2 * gq + (rq >> 2));
            float o[4] = {Y[4 * gq], Y[4 * gq + 1], Y[4 * gq + 2], Y[4 * gq + 3]};
            if (zh) {
                const u32x2_t zv = *reinterpret_cast<const u32x2_t *>(&tZ[o8]);
                o[0] *= silu_f32(bf16_to_f32((uint16_t)(zv.x & 0xffffu)));
                o[1] *= silu_f32(bf16_to_f32((uint16_t)(zv.x >> 16)));
                o[2] *= silu_f32(bf16_to_f32((uint16_t)(zv.y & 0xffffu)));
                o[3] *= silu_f32(bf16_to_f32((uint16_t)(zv.y >> 16)));
            }
            const bf16x4_t ov = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
            *reinterpret_cast<bf16x4_t *>(&tZ[o8]) = ov;
        }
        __syncthreads();                                // (4)
        // --- y rows out (16 bytes per thread, the slots this thread fills with the next z)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tr = tid / 8 + 32 * i;
            if (tr < nt) {
                const u32x4_t yv = *reinterpret_cast<const u32x4_t *>(&tZ[zsw16(tr, tid % 8)]);
                __builtin_nontemporal_store((tr & 1) ? u32x4_t{yv.z, yv.w, yv.x, yv.y} : yv,
                    reinterpret_cast<u32x4_t *>(yh + t0 * xrow + (uint32_t)tr * xr32 + (uint32_t)(tid % 8) * 8));
            }
        }
        // --- H^T [p][n] <- H (high and low parts): column p, four consecutive n per write
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int n0 = 32 * qi + 8 * gq + rq;
            bf16x4_t hh, hl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                __bf16 hi, lo;
                split(S[4 * gq + j], hi, lo);
                hh[j] = hi;
                hl[j] = lo;
            }
            *reinterpret_cast<bf16x4_t *>(&tH1[sw(col, n0)]) = hh;
            *reinterpret_cast<bf16x4_t *>(&tH2[sw(col, n0)]) = hl;
        }
    }
    if (last_state) {
        float *ls = last_state + ((int64_t)b * H + h) * P * N + (int64_t)col * N;
#pragma unroll
        for (int e = 0; e < 16; ++e) ls[32 * qi + acc_row(e, lane)] = S[e];
    }
}

}  // namespace ssm

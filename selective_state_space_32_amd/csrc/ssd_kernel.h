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
// four waves, each owning a 16-row band (all four 16 x 16 blocks) of every product, computed
// with v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation; each operand fetched once
// per step for all four blocks and both high / low parts).  The products are taken
// transposed (G^T = B C^T, Y^T = X^T M^T, and the state as H[n][p]), so that the four
// consecutive accumulator rows a lane holds are four consecutive elements of the operand
// tile they are written to (one 8-byte LDS write) and each lane's output column is one
// token.  D x is folded into M as D on its diagonal.  x, B and C are bf16 inputs, exact as
// operands; the operands formed here (M, Bw and the state's copy) are split into a bf16 high
// part and a bf16 low part (v - hi), each multiplied, so that they keep about 16 bits of
// their fp32 value.  Every input row is loaded coalesced and staged by token; C, B, the M
// tiles and the state's copy have the contraction index contiguous (one 16-byte LDS read per
// operand fetch), X and Bw are stored by token and fetched with gfx950's transposing LDS
// read (two 8-byte reads per operand).  The
// state stays in fp32 accumulators across chunks.  The next chunk's inputs are fetched into
// registers while the current chunk is computed (unconditionally -- the last chunk fetches
// itself again -- so that the loads land in the loop's own registers and are waited for only
// when the next chunk is staged).  Five operand tiles and a z / y tile (52 KB of LDS) serve
// every phase of a chunk; with at most 168 registers three workgroups fit on a CU, so the
// whole grid of a layer with up to 768 (sequence, head) pairs is resident at once.
#pragma once

#include <type_traits>

#include "device_math.h"

namespace ssm {

constexpr int kSsdQ = 64;          // tokens per chunk
constexpr int kSsdP = 64;          // channels per tile (a head's 64 channels, or fewer padded)
constexpr int kSsdN = 64;          // states per tile (64, or fewer padded)
constexpr int kSsdThreads = 256;   // four waves per (sequence, head)
// Operand tiles are 64 x 64 bf16, element (row, k) at sw(row, k): rows of 72 (144 bytes:
// 16-byte aligned, and 16-byte reads of eight consecutive rows fall in distinct banks), or,
// for the C tile, swz(row, k): unpadded rows whose 16-byte unit k / 8 is stored at unit
// (k / 8) ^ (row % 8), which spreads the same reads over all banks.
// With dstate 128 the C, B and state tiles are 128 wide: the same layouts with rows of 136
// (padded) or 128 (swizzled, the unit index XOR row % 8 within the row's 16 units).  Tiles of
// width W: swp<W> (padded), swzw<W> (swizzled); sw / swz are the 64-wide ones.
constexpr int kSsdLd = 72;
template <int W> __device__ __forceinline__ int swp(int row, int k) { return row * (W + 8) + k; }
template <int W> __device__ __forceinline__ int swzw(int row, int k) {
    return row * W + ((((k >> 3) ^ (row & 7)) & (W / 8 - 1)) << 3) + (k & 7);
}
__device__ __forceinline__ int sw(int row, int k) { return swp<64>(row, k); }
__device__ __forceinline__ int swz(int row, int k) { return swzw<64>(row, k); }
template <bool Z, int W = 64> __device__ __forceinline__ int tix(int row, int k) {
    return Z ? swzw<W>(row, k) : swp<W>(row, k);
}
// The z / y tile [t][p] has unpadded rows of 64; its 8-byte unit u (p / 4) of row t is stored
// at unit u ^ (t % 16), so that the output layout's 8-byte accesses (32 rows, one unit) and
// the 16-byte row accesses both spread over all banks.
__device__ __forceinline__ int zsw8(int t, int u) { return t * 64 + ((u ^ (t & 15)) << 2); }
// 16-byte unit v of row t: units 2v, 2v+1 land in unit v ^ (t % 16 / 2), halves swapped for odd t
__device__ __forceinline__ int zsw16(int t, int v) { return t * 64 + ((v ^ ((t & 15) >> 1)) << 3); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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

// Operand and accumulator layout of v_mfma_f32_16x16x32_bf16: a lane fetches the 8
// consecutive k at offset 8 (lane / 16) of each 32-wide step, for A row / B column
// lane % 16; accumulator element e of a lane is row 4 (lane / 16) + e, column lane % 16.
// NB 16 x 16 blocks side by side (B columns from rows bs, bs + 16, ... of tile `b`) over a
// contraction of 32 * KS, each operand fetched once per step:
//   mma16_hl_a: A = ah + al (high and low parts, rows a0): acc_i += (ah + al) B_i
//   mma16_hl_b: B = bh + bl (high and low parts): acc_i += A (bh_i + bl_i)
//   mma16_xn  : acc_i += A B_i where enabled
// (WA, WB: widths of the A and B tiles)
// With fp32 inputs (F3) the input operand is split too (b + bl: high and low bf16 parts), and
// the products take the three terms that carry about 16 bits: ah b + al b + ah bl.
template <int KS, int NB, bool ZB, int WA = 64, int WB = 64, bool F3 = false>
__device__ __forceinline__ void mma16_hl_a(const __bf16 *ah, const __bf16 *al, int a0, const __bf16 *b, int bs,
                                           int lane, f32x4_t (&acc)[NB], const __bf16 *bl = nullptr) {
    const int r = lane & 15, ko = (lane >> 4) * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int kk = 32 * k + ko;
        const bf16x8_t hv = *reinterpret_cast<const bf16x8_t *>(ah + swp<WA>(a0 + r, kk));
        const bf16x8_t lv = *reinterpret_cast<const bf16x8_t *>(al + swp<WA>(a0 + r, kk));
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(b + tix<ZB, WB>(bs + 16 * i + r, kk));
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv, bv, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lv, bv, acc[i], 0, 0, 0);
            if constexpr (F3) {
                const bf16x8_t blv = *reinterpret_cast<const bf16x8_t *>(bl + tix<ZB, WB>(bs + 16 * i + r, kk));
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv, blv, acc[i], 0, 0, 0);
            }
        }
    }
}
// Operand fetch from a padded tile stored [k][m] (rows k): the 8 consecutive k from
// k0 + 8 (lane / 16) of m = m0 + lane % 16, by two transposing LDS reads.  Within a group of
// 16 lanes the read returns to lane j, slot q, slot j % 4 of lane 4 q + j / 4's 8-byte
// address; so lane i addresses the 4 elements m0 + 4 (i % 4) .. +3 of row k + i / 4, and
// lane j receives rows k .. k+3 of column m0 + j.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
template <int W = 64>
__device__ __forceinline__ bf16x8_t ld_tr(const __bf16 *t, int k0, int m0, int lane) {
    const int i = lane & 15, kb = k0 + 8 * (lane >> 4) + (i >> 2), m = m0 + 4 * (i & 3);
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t + swp<W>(kb, m)));
    const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(t + swp<W>(kb + 4, m)));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}
// mma16_hl_a with both operands stored [k][m] (A: ah / al [k][row], B: b [k][col])
template <int KS, int NB, int WA = 64, int WB = 64, bool F3 = false>
__device__ __forceinline__ void mma16_hl_a_tr(const __bf16 *ah, const __bf16 *al, int a0, const __bf16 *b, int bs,
                                              int lane, f32x4_t (&acc)[NB], const __bf16 *bl = nullptr) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const bf16x8_t hv = ld_tr<WA>(ah, 32 * k, a0, lane);
        const bf16x8_t lv = ld_tr<WA>(al, 32 * k, a0, lane);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const bf16x8_t bv = ld_tr<WB>(b, 32 * k, bs + 16 * i, lane);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv, bv, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lv, bv, acc[i], 0, 0, 0);
            if constexpr (F3) {
                const bf16x8_t blv = ld_tr<WB>(bl, 32 * k, bs + 16 * i, lane);
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv, blv, acc[i], 0, 0, 0);
            }
        }
    }
}
// (A stored [k][row]; bh padded, bl swizzled; F3: A's low part al too, times bh)
template <int KS, int NB, int WB = 64, bool F3 = false>
__device__ __forceinline__ void mma16_hl_b(const __bf16 *a, int a0, const __bf16 *bh, const __bf16 *bl, int bs,
                                           int lane, f32x4_t *acc, const __bf16 *al = nullptr) {
    const int r = lane & 15, ko = (lane >> 4) * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int kk = 32 * k + ko;
        const bf16x8_t av = ld_tr(a, 32 * k, a0, lane);
        bf16x8_t alv;
        if constexpr (F3) alv = ld_tr(al, 32 * k, a0, lane);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const bf16x8_t hv = *reinterpret_cast<const bf16x8_t *>(bh + swp<WB>(bs + 16 * i + r, kk));
            const bf16x8_t lv = *reinterpret_cast<const bf16x8_t *>(bl + swzw<WB>(bs + 16 * i + r, kk));
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hv, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, lv, acc[i], 0, 0, 0);
            if constexpr (F3) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alv, hv, acc[i], 0, 0, 0);
        }
    }
}
// (F3: both operands split, a + al and b + bl: a b + al b + a bl)
template <int KS, int NB, bool ZB, int WA = 64, int WB = 64, bool F3 = false>
__device__ __forceinline__ void mma16_xn(const __bf16 *a, int a0, const __bf16 *b, int bs, int first, int lane,
                                         f32x4_t (&acc)[NB], const __bf16 *al = nullptr,
                                         const __bf16 *bl = nullptr) {   // blocks i >= first only
    const int r = lane & 15, ko = (lane >> 4) * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int kk = 32 * k + ko;
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(a + swp<WA>(a0 + r, kk));
        bf16x8_t alv;
        if constexpr (F3) alv = *reinterpret_cast<const bf16x8_t *>(al + swp<WA>(a0 + r, kk));
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i >= first) {
                const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(b + tix<ZB, WB>(bs + 16 * i + r, kk));
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i], 0, 0, 0);
                if constexpr (F3) {
                    const bf16x8_t blv = *reinterpret_cast<const bf16x8_t *>(bl + tix<ZB, WB>(bs + 16 * i + r, kk));
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alv, bv, acc[i], 0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, blv, acc[i], 0, 0, 0);
                }
            }
        }
    }
}

// x, z, y: [bsz][L][H][hp] bf16;  dt: [bsz][L][H] bf16;  A, Dv, dt_bias: [H] fp32;
// B, C: [bsz][L][G][ns] bf16;  h0, last_state: [bsz][H][hp][ns] fp32 (or null; h0 may be
// last_state: each thread reads its own state elements before it writes them).
// Head and state sizes: the tiles are 64 wide.  A head of hp = 64 v channels is v virtual
// heads of 64 (its channels are independent given the head's dt, A, B and C), one
// workgroup each (grid bsz * H * v).  hp = 32 and ns = 32 are padded to 64 with zeros:
// zero x channels give zero outputs and state columns (not stored), zero B / C states add
// nothing to C B^T or to the readout and keep zero state rows (not stored).
//
// Four waves; wave w owns, in every product, the 16-row band w and the four 16 x 16 column
// blocks j = 0..3.
// Tiles and their phases within a chunk (barriers 1-4):
//   tC : C [t][n] (swizzled)          -> (2) M low part [t][s]
//   tB : B [s][n]                     -> (2) M high part [t][s]
//   tX : X [s][p]
//   tH1: the state's copy H^T [p][n], high part  -> (2) Bw [s][n] high part -> (4) H^T high
//   tH2: the same, low parts
//   tZ : z [t][p]                     -> (3) y, in place
// (at most 168 registers: three workgroups of four waves per CU)
// PAD: hp or ns is 32 (the masked loads and stores of padded channels and states).
// NT: states per tile, 64 or 128 (dstate 128: C, B, the state's copy and Bw are 128 wide, and
// each wave holds two 16-row bands of the 128 x 64 state; 86 KB of LDS, one workgroup per CU).
// F32: fp32 x, dt, B, C, z and y (NT = 64).  x, B and C are staged as bf16 high and low parts
// (tX / tXl, tB / tBl, tC / tCl) and every product takes the three terms of about 16 bits
// (hi hi + lo hi + hi lo); z is read and y written from the output layout directly (no z / y
// tile).  70 KB of LDS and up to 256 registers: two workgroups per CU.
template <bool F32> using ssd_io_t = std::conditional_t<F32, float, uint16_t>;   // element type of x, dt, B, C, z, y
template <bool PAD, int NT = 64, bool F32 = false>
__global__ void __launch_bounds__(kSsdThreads)
__attribute__((amdgpu_waves_per_eu(NT == 64 ? (F32 ? 2 : 3) : 1)))
ssd_chunk_kernel(const ssd_io_t<F32> *__restrict__ x, const ssd_io_t<F32> *__restrict__ dt,
                 const float *__restrict__ A, const ssd_io_t<F32> *__restrict__ Bm,
                 const ssd_io_t<F32> *__restrict__ Cm, const float *__restrict__ Dv,
                 const ssd_io_t<F32> *__restrict__ z, const float *__restrict__ dt_bias,
                 ssd_io_t<F32> *__restrict__ y, float *last_state, int64_t L, int H, int G, int softplus,
                 const float *h0, int hp, int ns_in) {
    using TIO = ssd_io_t<F32>;
    const int ns = PAD ? ns_in : NT;   // (without padding the state size is the tile's)
    constexpr int Q = kSsdQ, P = kSsdP, N = kSsdN, LD = kSsdLd;
    static_assert(Q == 64 && P == 64 && N == 64, "a 16-row band and four 16 x 16 blocks per wave of four");
    static_assert(NT == 64 || (NT == 128 && !PAD && !F32), "64 or 128 states per tile (64 with fp32 I/O)");
    constexpr int NBS = NT / 64;                      // 16-row bands of the state per wave
    constexpr int LDN = NT + 8;                       // row stride of the padded NT-wide tiles
    // B / C staging: TPR threads per row of NT elements (8 each), RPB rows per pass, NPB passes
    constexpr int TPR = NT / 8, RPB = kSsdThreads / TPR, NPB = Q / RPB;
    constexpr bool ZC = true;                         // tC is swizzled
    __shared__ __attribute__((aligned(16))) __bf16 tC[Q * NT];
    __shared__ __attribute__((aligned(16))) __bf16 tB[Q * LDN];
    __shared__ __attribute__((aligned(16))) __bf16 tX[P * LD];
    __shared__ __attribute__((aligned(16))) __bf16 tH1[P * LDN];
    __shared__ __attribute__((aligned(16))) __bf16 tH2[P * LDN];
    __shared__ __attribute__((aligned(16))) __bf16 tZ[F32 ? 1 : Q * 64];
    // (fp32 I/O: the low parts of C, B and X, laid out as their high parts)
    __shared__ __attribute__((aligned(16))) __bf16 tCl[F32 ? Q * NT : 1];
    __shared__ __attribute__((aligned(16))) __bf16 tBl[F32 ? Q * LDN : 1];
    __shared__ __attribute__((aligned(16))) __bf16 tXl[F32 ? P * LD : 1];
    // per-token values (formed by wave 0), four tokens per row padding of tX (tokens 4r..4r+3
    // in row r): c_t (in log2 units), f_s = exp2(c_r - c_s) dt_s with r the first token of s's
    // half-chunk, and the Bw weight w_s = exp2(c_last - c_s) dt_s (dt_s = 0 past the end)
    float *const s_pad = reinterpret_cast<float *>(tX + 64);   // row r at s_pad + r * LD / 2
    auto s_c4 = [&](int t) -> float * { return s_pad + (t >> 2) * (LD / 2) + (t & 3); };
    auto s_f4 = [&](int t) -> float * { return s_pad + (16 + (t >> 2)) * (LD / 2) + (t & 3); };
    auto s_w4 = [&](int t) -> float * { return s_pad + (32 + (t >> 2)) * (LD / 2) + (t & 3); };
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qi = w;                                 // row band 16 qi; column blocks 0..3
    const int c16 = lane & 15;                        // the lane's column within a block
    const int rq = (lane >> 4) * 4;                   // its rows: 16 qi + rq + (0..3)
    const int vh = hp > 64 ? hp / 64 : 1;            // virtual heads of 64 channels per head
    const int Hv = H * vh;
    const int bh = blockIdx.x;
    const int b = bh / Hv, hv = bh - b * Hv;          // hv: the virtual head
    const int h = hv / vh, p0 = (hv - h * vh) * 64;   // the head and its first channel here
    const int pw = hp < 64 ? hp : 64;                 // channels present in the 64-wide tile
    const int g = h / (H / G);
    const float a2 = A[h] * kLog2e;                   // decays as exp2(a2 * sum of dt)
    const float bias_h = dt_bias ? dt_bias[h] : 0.0f;
    const float d_h = Dv ? Dv[h] : 0.0f;
    // elements between tokens in x, z, y, and this workgroup's first channel (without
    // padding, virtual head hv's channels start at 64 hv)
    const int64_t xrow = PAD ? (int64_t)H * hp : (int64_t)Hv * P;
    const int64_t xoff = PAD ? (int64_t)h * hp + p0 : (int64_t)hv * P;
    const int64_t brow = (int64_t)G * ns;             // ... in B, C
    const TIO *xh = x + (int64_t)b * L * xrow + xoff;
    const TIO *zh = z ? z + (int64_t)b * L * xrow + xoff : nullptr;
    TIO *yh = y + (int64_t)b * L * xrow + xoff;
    const TIO *Bg = Bm + (int64_t)b * L * brow + (int64_t)g * ns;
    const TIO *Cg = Cm + (int64_t)b * L * brow + (int64_t)g * ns;
    // state element (channel p, state n) of this workgroup in h0 / last_state
    const int64_t st0 = (((int64_t)b * H + h) * hp + p0) * ns;
    auto st_index = [st0, ns](int p, int n) -> int64_t { return st0 + (int64_t)p * ns + n; };

    // staging map: every row coalesced (tokens tid / 8 + 32 i, 8 elements at 8 (tid % 8)); X
    // and Bw are stored by token and read transposed where they are operands.  Addresses: the
    // chunk's base (uniform) plus a 32-bit offset per lane (64 rows of H P elements fit 32
    // bits).  z is read and y written once: streaming (non-temporal) accesses.
    // (EW 16-byte units per thread and row: one for 8 bf16, two for 8 fp32; with fp32 I/O z is
    // not staged)
    constexpr int EW = F32 ? 2 : 1;
    struct Raw { u32x4_t c[NPB][EW], xv[2][EW], bv[NPB][EW], zv[F32 ? 1 : 2]; uint32_t dt; };   // rows tr0 + 32 i (x, z), trb + RPB i (B, C)
    const uint32_t xr32 = (uint32_t)xrow, br32 = (uint32_t)brow;
    const int tr0 = tid / 8, tu = tid % 8;
    const int trb = tid / TPR, tub = tid % TPR;
    const bool xin = !PAD || tu * 8 < pw, bin = !PAD || tub * 8 < ns;   // this thread's 8 channels / states exist
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};
    auto fetch = [&](int64_t t0, Raw &r) {
        const uint32_t lim = (uint32_t)min((int64_t)(Q - 1), L - 1 - t0);   // last token present
        const uint32_t ts = min((uint32_t)lane, lim);
#pragma unroll
        for (int i = 0; i < (NPB > 2 ? NPB : 2); ++i) {
            const uint32_t tcb = min((uint32_t)(trb + RPB * i), lim);
#pragma unroll
            for (int e = 0; e < EW; ++e) {
                if (i < NPB)
                    r.c[i][e] = bin ? *reinterpret_cast<const u32x4_t *>(Cg + t0 * brow + (tcb * br32 + (uint32_t)tub * 8) + 4 * e)
                                    : zero4;
                if (i < 2) {
                    const uint32_t tc = min((uint32_t)(tr0 + 32 * i), lim);
                    if (!F32 && zh)
                        r.zv[F32 ? 0 : i] = xin ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(
                                                      zh + t0 * xrow + (tc * xr32 + (uint32_t)tu * 8)))
                                                : zero4;
                    r.xv[i][e] = xin ? *reinterpret_cast<const u32x4_t *>(xh + t0 * xrow + (tc * xr32 + (uint32_t)tu * 8) + 4 * e)
                                     : zero4;
                }
                if (i < NPB)
                    r.bv[i][e] = bin ? *reinterpret_cast<const u32x4_t *>(Bg + t0 * brow + (tcb * br32 + (uint32_t)tub * 8) + 4 * e)
                                     : zero4;
            }
        }
        const TIO dtv = dt[((int64_t)b * L + t0) * H + h + (w == 0 ? ts : 0u) * (uint32_t)H];   // (used by wave 0)
        if constexpr (F32) r.dt = __float_as_uint(dtv);
        else r.dt = dtv;
    };
    auto split = [](float v, __bf16 &hi, __bf16 &lo) {
        hi = (__bf16)v;
        lo = (__bf16)(v - (float)hi);
    };

    // the state H [n][p]: band q, rows n = 64 q + 16 qi.., columns p 16 j..
    f32x4_t S[NBS][4] = {};
    // the H^T [p][n] copy (high and low parts) that the next chunk's Y3 product reads:
    // column p, four consecutive n per write
    auto state_copy = [&]() {
#pragma unroll
        for (int q = 0; q < NBS; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = 16 * j + c16, n0 = 64 * q + 16 * qi + rq;
                bf16x4_t hh, hl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    __bf16 hi, lo;
                    split(S[q][j][e], hi, lo);
                    hh[e] = hi;
                    hl[e] = lo;
                }
                *reinterpret_cast<bf16x4_t *>(&tH1[swp<NT>(p, n0)]) = hh;
                *reinterpret_cast<bf16x4_t *>(&tH2[swp<NT>(p, n0)]) = hl;
            }
    };
    if (h0) {
        // the initial state into the accumulators (the layout last_state is written in)
#pragma unroll
        for (int q = 0; q < NBS; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = 16 * j + c16, n0 = 64 * q + 16 * qi + rq;
                const float *hs = h0 + st_index(p, n0);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[q][j][e] = (!PAD || (p < pw && n0 + e < ns)) ? hs[e] : 0.0f;
            }
        state_copy();   // (read after barrier (1) of the first chunk)
    }
    Raw r;
    fetch(0, r);
    const int64_t nchunks = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * Q;
        const int nt = (int)min((int64_t)Q, L - t0);
        // --- stage C, z, B and X (rows by token); wave 0: the step sizes and their running sum
#pragma unroll
        for (int i = 0; i < (NPB > 2 ? NPB : 2); ++i) {
            const int tr = tr0 + 32 * i, trs = trb + RPB * i;
            if constexpr (F32) {
                // 8 fp32 values as bf16 high and low parts
                auto split8 = [](const u32x4_t (&v)[EW], bf16x8_t &hi, bf16x8_t &lo) {
                    const uint32_t e8[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[EW - 1].x, v[EW - 1].y, v[EW - 1].z, v[EW - 1].w};
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const float f = __uint_as_float(e8[k]);
                        hi[k] = (__bf16)f;
                        lo[k] = (__bf16)(f - (float)hi[k]);
                    }
                };
                bf16x8_t hv, lv;
                if (i < NPB) {
                    split8(r.c[i], hv, lv);
                    *reinterpret_cast<bf16x8_t *>(&tC[swzw<NT>(trs, tub * 8)]) = hv;
                    *reinterpret_cast<bf16x8_t *>(&tCl[swzw<NT>(trs, tub * 8)]) = lv;
                    split8(r.bv[i], hv, lv);
                    *reinterpret_cast<bf16x8_t *>(&tB[swp<NT>(trs, tub * 8)]) = hv;
                    *reinterpret_cast<bf16x8_t *>(&tBl[swp<NT>(trs, tub * 8)]) = lv;
                }
                if (i < 2) {
                    split8(r.xv[i], hv, lv);
                    *reinterpret_cast<bf16x8_t *>(&tX[sw(tr, tu * 8)]) = hv;
                    *reinterpret_cast<bf16x8_t *>(&tXl[sw(tr, tu * 8)]) = lv;
                }
            } else {
                if (i < NPB) *reinterpret_cast<u32x4_t *>(&tC[swzw<NT>(trs, tub * 8)]) = r.c[i][0];
                if (i < 2 && zh) {
                    const u32x4_t zv = (tr & 1) ? u32x4_t{r.zv[i].z, r.zv[i].w, r.zv[i].x, r.zv[i].y} : r.zv[i];
                    *reinterpret_cast<u32x4_t *>(&tZ[zsw16(tr, tu)]) = zv;
                }
                if (i < NPB) *reinterpret_cast<u32x4_t *>(&tB[swp<NT>(trs, tub * 8)]) = r.bv[i][0];
                if (i < 2) *reinterpret_cast<u32x4_t *>(&tX[sw(tr, tu * 8)]) = r.xv[i][0];
            }
        }
        if (w == 0) {   // token = lane
            const float v = (F32 ? __uint_as_float(r.dt) : bf16_to_f32((uint16_t)r.dt)) + bias_h;
            const float dl = lane < nt ? (softplus ? softplus_f32(v) : v) : 0.0f;   // padded tokens: identity steps
            const float cl = a2 * wave_incl_sum(dl);
            const float ctot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 63));
            const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 0));
            const float c32 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 32));
            *s_c4(lane) = cl;
            *s_f4(lane) = hw_exp2((lane < 32 ? c0 : c32) - cl) * dl;
            *s_w4(lane) = hw_exp2(ctot - cl) * dl;
        }
        u32x4_t bcur[NPB][EW];
#pragma unroll
        for (int i = 0; i < NPB; ++i)
#pragma unroll
            for (int e = 0; e < EW; ++e) bcur[i][e] = r.bv[i][e];
        fetch(min(t0 + Q, (nchunks - 1) * Q), r);   // (the last chunk fetches itself again, unused)
        __syncthreads();                                // (1)
        const float ctot = *s_c4(Q - 1);                // c_last
        const float cref = *s_c4(qi >= 2 ? 32 : 0);     // c at the first token of this band's half-chunk
        // (fp32 I/O: this lane's z values in the output layout -- token 16 j + c16, channels
        // 16 qi + rq .. +3 -- read now, used at the end of the chunk)
        const int och = 16 * qi + rq;                   // the output layout's first channel
        const bool och_in = !PAD || och < pw;
        f32x4_t zq[F32 ? 4 : 1];
        if constexpr (F32) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = min(16 * j + c16, nt - 1);
                zq[j] = (zh && och_in) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(
                                             zh + t0 * xrow + ((uint32_t)t * xr32 + (uint32_t)och)))
                                       : f32x4_t{1.0f, 1.0f, 1.0f, 1.0f};
            }
        }
        // --- Y3^T = H^T C^T (the state entering the chunk) and G^T = B C^T
        f32x4_t Y[4] = {}, Gt[4] = {};
        if (c > 0 || h0) mma16_hl_a<NT / 32, 4, ZC, NT, NT, F32>(tH1, tH2, 16 * qi, tC, 0, lane, Y, tCl);
        mma16_xn<NT / 32, 4, ZC, NT, NT, F32>(tB, 16 * qi, tC, 0, qi, lane, Gt, tBl, tCl);   // blocks j >= qi (zero for s > t)
        __syncthreads();                                // (2)
        // --- M [t][s] = G^T[s][t] exp2(c_t - c_s) dt_s (s <= t) + D (s = t): rows s of this
        //     wave's band, column t; four consecutive s per 8-byte write.  The decay is
        //     exp2(c_t - c_r) f_s with r the first token of s's half-chunk (r <= s <= t): both
        //     factors are at most 1 (times dt_s), as c does not increase along the chunk
        //     (a <= 0, dt >= 0).  Blocks above the diagonal are written as zeros (some are read).
        {
            const int s0 = 16 * qi + rq;
            const f32x4_t fs = *reinterpret_cast<const f32x4_t *>(s_f4(s0));
            const float fsv[4] = {fs.x, fs.y, fs.z, fs.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * j + c16;
                bf16x4_t mh = {}, ml = {};
                if (qi <= j) {
                    const float et = hw_exp2(*s_c4(t) - cref);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float m = Gt[j][e] * et * fsv[e];
                        if (qi == j) {
                            m = s0 + e <= t ? m : 0.0f;
                            if (s0 + e == t) m += d_h;
                        }
                        __bf16 hi, lo;
                        split(m, hi, lo);
                        mh[e] = hi;
                        ml[e] = lo;
                    }
                }
                *reinterpret_cast<bf16x4_t *>(&tB[swp<NT>(t, s0)]) = mh;
                *reinterpret_cast<bf16x4_t *>(&tC[swzw<NT>(t, s0)]) = ml;
            }
        }
        // --- Bw [s][n] = B[s][n] exp2(c_last - c_s) dt_s: tokens tr, states 8 tub .. +7
#pragma unroll
        for (int i = 0; i < NPB; ++i) {
            const int tr = trb + RPB * i;
            const float wsl = *s_w4(tr);
            bf16x8_t bhv, blv;
            if constexpr (F32) {
                const uint32_t bw[8] = {bcur[i][0].x, bcur[i][0].y, bcur[i][0].z, bcur[i][0].w,
                                        bcur[i][EW - 1].x, bcur[i][EW - 1].y, bcur[i][EW - 1].z, bcur[i][EW - 1].w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    __bf16 hh, ll;
                    split(__uint_as_float(bw[k]) * wsl, hh, ll);
                    bhv[k] = hh;
                    blv[k] = ll;
                }
            } else {
                const uint32_t bw[4] = {bcur[i][0].x, bcur[i][0].y, bcur[i][0].z, bcur[i][0].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    __bf16 h0, l0, h1, l1;
                    split(bf16_to_f32((uint16_t)(bw[k] & 0xffffu)) * wsl, h0, l0);
                    split(bf16_to_f32((uint16_t)(bw[k] >> 16)) * wsl, h1, l1);
                    bhv[2 * k] = h0; bhv[2 * k + 1] = h1;
                    blv[2 * k] = l0; blv[2 * k + 1] = l1;
                }
            }
            *reinterpret_cast<bf16x8_t *>(&tH1[swp<NT>(tr, tub * 8)]) = bhv;
            *reinterpret_cast<bf16x8_t *>(&tH2[swp<NT>(tr, tub * 8)]) = blv;
        }
        __syncthreads();                                // (3)
        // --- H [n][p] <- exp2(c_last) H + Bw^T X   (rows n 64 q + 16 qi.., columns p 16 j..)
        const float dec = hw_exp2(ctot);
#pragma unroll
        for (int q = 0; q < NBS; ++q) {
#pragma unroll
            for (int j = 0; j < 4; ++j) S[q][j] *= dec;
            mma16_hl_a_tr<Q / 32, 4, NT, 64, F32>(tH1, tH2, 64 * q + 16 * qi, tX, 0, lane, S[q], tXl);
        }
        // --- Y^T = X^T M^T + exp2(c_t) Y3^T   (rows p 16 qi.., columns t 16 j..), then
        //     y = Y * silu(z): token t, channels 16 qi + rq .. +3, into the z slot
#pragma unroll
        for (int j = 0; j < 4; ++j) Y[j] *= hw_exp2(*s_c4(16 * j + c16));
        mma16_hl_b<1, 2, NT, F32>(tX, 16 * qi, tB, tC, 0, lane, Y, tXl);        // t < 32: s < 32 suffices
        mma16_hl_b<2, 2, NT, F32>(tX, 16 * qi, tB, tC, 32, lane, Y + 2, tXl);
#pragma unroll
        for (int j = 0; j < 4 && F32; ++j) {
            // fp32 I/O: y straight from the accumulators (16 bytes: four channels of token t)
            const int t = 16 * j + c16;
            float o[4] = {Y[j][0], Y[j][1], Y[j][2], Y[j][3]};
            if (zh) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] *= silu_f32(zq[F32 ? j : 0][e]);
            }
            if (t < nt && och_in)
                __builtin_nontemporal_store(f32x4_t{o[0], o[1], o[2], o[3]},
                    reinterpret_cast<f32x4_t *>(yh + t0 * xrow + ((uint32_t)t * xr32 + (uint32_t)och)));
        }
#pragma unroll
        for (int j = 0; j < 4 && !F32; ++j) {
            const int t = 16 * j + c16;
            const int o8 = zsw8(t, 4 * qi + (lane >> 4));
            float o[4] = {Y[j][0], Y[j][1], Y[j][2], Y[j][3]};
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
        // --- y rows out (16 bytes per thread and row, the slots this thread fills with the next z)
#pragma unroll
        for (int i = 0; i < 2 && !F32; ++i) {
            const int tr = tr0 + 32 * i;
            if (tr < nt && xin) {
                const u32x4_t yv = *reinterpret_cast<const u32x4_t *>(&tZ[zsw16(tr, tu)]);
                __builtin_nontemporal_store((tr & 1) ? u32x4_t{yv.z, yv.w, yv.x, yv.y} : yv,
                    reinterpret_cast<u32x4_t *>(yh + t0 * xrow + (uint32_t)tr * xr32 + (uint32_t)tu * 8));
            }
        }
        // --- H^T [p][n] <- H (high and low parts)
        state_copy();
    }
    if (last_state) {
#pragma unroll
        for (int q = 0; q < NBS; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = 16 * j + c16, n0 = 64 * q + 16 * qi + rq;
                float *ls = last_state + st_index(p, n0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!PAD || (p < pw && n0 + e < ns)) ls[e] = S[q][j][e];
            }
    }
}

}  // namespace ssm

// Selective-scan kernels for gfx950.
//
// Work decomposition (one workgroup = one sequence b x a tile of 64 channels x one chunk of
// tokens; K = N / S waves):
//  * wave w owns states n in [w*S, (w+1)*S) of all 64 channels, lane = channel.  The
//    fp32 state h and A*log2(e) for those states live in VGPRs for the whole chunk.
//  * B_t and C_t are the same for every channel of a sequence, so for a wave they are
//    uniform: each wave reads its S-wide slice of them with scalar loads into SGPRs from a
//    small fp32 staging copy (stage_bc_kernel), and every per-(token, state) instruction
//    takes them as its scalar operand.
//  * Per-token, per-channel work (the step-size activation, delta*u, the skip term, the
//    SiLU gate, the output rounding) is done once per element, spread over all K waves:
//    a "prep" pass writes (delta, delta*u) for a tile of T tokens into LDS, the waves run
//    the recurrence over the tile writing partial readouts sum_{n in slice} C h into LDS,
//    and an "epilogue" pass adds the K partials, the skip term and the gate and stores y.
//  * Global loads and stores of u, delta, z and y are along channels (lane = channel), so a
//    wave touches 64 consecutive elements of one token row.
// Per (token, channel, state) the recurrence costs one multiply (delta*A), one exp2, one
// multiply (delta*u*B), one FMA (state) and one FMA (readout) -- no more.
#pragma once

#include "device_math.h"

namespace ssm {

constexpr int kTileT = 32;       // tokens per LDS tile
constexpr int kChanTile = 64;    // channels per workgroup (one per lane)

enum ScanMode { kFull = 0, kSummary = 1 };

// fp32 staging copy of B and C, laid out per (sequence, wave slice):
//   bc[b][w][t][0..S)  = B[b][t][w*S + s],   bc[b][w][t][S..2S) = C[b][t][w*S + s]
// so that one wave's operands for one token are 2S consecutive floats.
template <int N, int S, typename IO>
__global__ void __launch_bounds__(256)
stage_bc_kernel(const IO *__restrict__ B, const IO *__restrict__ C, float *__restrict__ bc,
                int64_t total /* bsz*L*N */, int64_t L) {
    constexpr int K = N / S;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int n = (int)(i % N);
    const int64_t bt = i / N;
    const int64_t b = bt / L, t = bt - b * L;
    const int w = n / S, s = n - w * S;
    const int64_t o = ((b * K + w) * L + t) * (2 * S);
    bc[o + s] = io<IO>::ld(B, i);
    bc[o + S + s] = io<IO>::ld(C, i);
}

// One chunk of the scan for one (sequence, 64-channel tile).
//   kFull:    start from h = 0 (chunk 0) or from the carried state cstate[b][c-1]
//             (the state after chunk c-1), run the recurrence with readout, write y; the
//             last chunk writes last_state.
//   kSummary: start from h = 0, no readout; write the chunk's local final state to
//             cstate[b][c] and the chunk's sum of step sizes to cdsum[b][c].
template <int N, int S, typename IO, int MODE>
__global__ void __launch_bounds__(64 * (N / S))
scan_chunk_kernel(const IO *__restrict__ u, const IO *__restrict__ delta,
                  const IO *__restrict__ z, IO *__restrict__ y,
                  const float *__restrict__ A, const float *__restrict__ Dv,
                  const float *__restrict__ bias, const float *__restrict__ bc,
                  float *__restrict__ last_state, float *__restrict__ cstate,
                  float *__restrict__ cdsum, int64_t L, int64_t D, int tiles_per_b,
                  int64_t chunk_len, int nchunk, int softplus) {
    constexpr int K = N / S;
    constexpr int T = kTileT;
    constexpr int J = T / K;  // prep / epilogue elements per thread per tile
    static_assert(T % K == 0, "tile must split evenly over the waves");
    __shared__ f32x2_t s_dk[T][kChanTile];
    __shared__ float s_yp[MODE == kFull ? K : 1][T][kChanTile];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = blockIdx.x / tiles_per_b;
    const int64_t d = (int64_t)(blockIdx.x - b * tiles_per_b) * kChanTile + lane;
    const bool act = d < D;
    const int c = blockIdx.y;
    const int64_t t_begin = (int64_t)c * chunk_len;
    const int64_t t_end = min(L, t_begin + chunk_len);

    float a2[S], h[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = w * S + s;
        a2[s] = act ? A[d * N + n] * kLog2e : 0.0f;
        h[s] = 0.0f;
        if (MODE == kFull && c > 0 && act) h[s] = cstate[(((int64_t)b * nchunk + c - 1) * D + d) * N + n];
    }
    const float Dd = (act && Dv) ? Dv[d] : 0.0f;
    const float bd = (act && bias) ? bias[d] : 0.0f;
    float dsum = 0.0f;
    const int64_t row0 = (int64_t)b * L;
    const float *__restrict__ bcw = bc + ((int64_t)(b * K + w) * L) * (2 * S);

    for (int64_t t0 = t_begin; t0 < t_end; t0 += T) {
        const int nt = (int)min((int64_t)T, t_end - t0);
        float Du[J], g[J];
        // prep: (delta, delta*u) into LDS; skip and gate factors kept in registers
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int tt = w + j * K;
            float dl = 0.0f, kk = 0.0f;
            Du[j] = 0.0f;
            g[j] = 1.0f;
            if (tt < nt && act) {
                const int64_t idx = (row0 + t0 + tt) * D + d;
                const float uu = io<IO>::ld(u, idx);
                const float x = io<IO>::ld(delta, idx) + bd;
                dl = softplus ? softplus_f32(x) : x;
                kk = dl * uu;
                if (MODE == kFull) {
                    Du[j] = Dd * uu;
                    if (z) g[j] = silu_f32(io<IO>::ld(z, idx));
                }
            }
            s_dk[tt][lane] = f32x2_t{dl, kk};
        }
        __syncthreads();
        // recurrence over the tile
        const float *__restrict__ bct = bcw + t0 * (2 * S);
#pragma unroll 4
        for (int tt = 0; tt < nt; ++tt) {
            const f32x2_t v = s_dk[tt][lane];
            float acc = 0.0f;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float e = hw_exp2(v.x * a2[s]);
                h[s] = fmaf(e, h[s], v.y * bct[tt * (2 * S) + s]);
                if (MODE == kFull) acc = fmaf(bct[tt * (2 * S) + S + s], h[s], acc);
            }
            if (MODE == kFull)
                s_yp[w][tt][lane] = acc;
            else
                dsum += v.x;
        }
        __syncthreads();
        if (MODE == kFull) {
            // epilogue: y = (sum of the K partial readouts + D u) * silu(z)
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int tt = w + j * K;
                if (tt < nt && act) {
                    float yv = Du[j];
#pragma unroll
                    for (int k = 0; k < K; ++k) yv += s_yp[k][tt][lane];
                    yv *= g[j];
                    io<IO>::st(y, (row0 + t0 + tt) * D + d, yv);
                }
            }
        }
    }

    if (!act) return;
    if (MODE == kFull) {
        if (last_state && c == nchunk - 1) {
#pragma unroll
            for (int s = 0; s < S; ++s) last_state[((int64_t)b * D + d) * N + w * S + s] = h[s];
        }
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) cstate[(((int64_t)b * nchunk + c) * D + d) * N + w * S + s] = h[s];
        if (w == 0) cdsum[((int64_t)b * nchunk + c) * D + d] = dsum;
    }
}

// Writes zeros (a scan of zero tokens leaves the zero initial state).
__global__ void __launch_bounds__(256) fill_zero_kernel(float *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

}  // namespace ssm

// Backward pass of the selective scan: gradients with respect to every input, by reverse
// mode of the recurrence with recomputation (the hardware-aware algorithm section of
// azimuth.plus/paper/mamba: intermediate states are recomputed in the backward pass instead
// of being stored).
//
// Per channel, with lambda_t = dLoss/dh_t and G the adjoint carried from token t+1
// (lambda_t = C_t dp_t + G, then G <- dA_t lambda_t for token t-1), dp_t = dy_t silu(z_t):
//   du_t       = D dp_t + sum_n lambda_t[n] delta_t B_t[n]
//   d delta_t  = sum_n lambda_t[n] (A[n] dA_t[n] h_{t-1}[n] + B_t[n] u_t), times
//                softplus'(x_t) = sigmoid(x_t) for the delta input when softplus is on
//   dA[n]     += lambda_t[n] delta_t dA_t[n] h_{t-1}[n]
//   dB_t[n]   += lambda_t[n] delta_t u_t,   dC_t[n] += dp_t h_t[n]   (over channels)
//   dD        += dp_t u_t,   d delta_bias += d x_t,   dz_t = dy_t p_t silu'(z_t)
//   d h0       = the adjoint left after token 0.
//
// Layout: one workgroup per (sequence, 64-channel tile), K waves of S states, lane =
// channel (as in the forward kernel).  A forward pass in checkpoint mode first stores the
// state before every kBwdTile-th token.  This kernel then walks the tiles of kBwdTile
// tokens from the last to the first; per tile it
//   1. prepares (delta, delta*u, u, dp) per (token, channel) and the tile's B and C rows
//      (fp32) in LDS (all threads),
//   2. recomputes the tile's states and exp(delta A) from its checkpoint into registers
//      (the wave's S states x kBwdTile tokens) and the partial readouts p,
//   3. walks the tile backwards, accumulating dA in registers, writing per-wave partial du
//      and d delta to LDS, and summing the dB / dC contributions of the tile's 64 channels
//      through a wave-private LDS transposition, added to global memory atomically (the
//      transposition of one token overlaps the arithmetic of the next),
//   4. finishes du, d delta, dz and the dD / d delta_bias sums per element (all threads).
// dA, dB, dC, dD and d delta_bias are sums over workgroups and are accumulated with atomic
// adds into buffers the host has zeroed; their summation order is not fixed.
#pragma once

#include "scan_kernels.h"

namespace ssm {

constexpr int kBwdTile = kCkptEvery;   // tokens per backward tile: one checkpoint each

template <int N> struct BwdShape {
    static constexpr int S = N < 4 ? N : 4;   // states per wave
    static constexpr int K = N / S;           // waves per workgroup
};

// Inclusive sum over groups of LPV consecutive lanes (LPV = 8, 16 or 32); the last lane of
// each group ends with the group total.
template <int LPV>
__device__ __forceinline__ float group_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));  // row_shr:1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));  // row_shr:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));  // row_shr:4
    if constexpr (LPV >= 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));  // row_shr:8
    if constexpr (LPV >= 32)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
    return v;
}

// Orders this wave's LDS accesses around an exchange between its lanes.  A wavefront's
// own LDS operations are performed in the order it issues them, so no wait is needed:
// the fences only keep the compiler from moving memory accesses across this point.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Register budget: with 4 waves per workgroup three workgroups share a CU (LDS allows it),
// which needs at most 168 VGPRs per lane.
template <int N, typename IO, bool VEC>
__global__ void __launch_bounds__(64 * BwdShape<N>::K)
__attribute__((amdgpu_waves_per_eu(BwdShape<N>::K == 4 ? 3 : 1)))
scan_bwd_kernel(const IO *__restrict__ u, const IO *__restrict__ delta, const IO *__restrict__ z,
                const IO *__restrict__ dy, const float *__restrict__ A, const float *__restrict__ Dv,
                const float *__restrict__ bias, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
                const float *__restrict__ ckpt, const float *__restrict__ dlast, IO *__restrict__ du,
                IO *__restrict__ ddelta, IO *__restrict__ dz, float *__restrict__ dA, float *__restrict__ dB,
                float *__restrict__ dC, float *__restrict__ dD, float *__restrict__ dbias,
                float *__restrict__ dh0, int64_t L, int64_t D, int tiles_per_b, int softplus) {
    constexpr int S = BwdShape<N>::S;
    constexpr int K = BwdShape<N>::K;
    constexpr int T = kBwdTile;
    constexpr int J = T / K;                       // prep / epilogue elements per thread per tile
    constexpr int V = VEC ? (J < 8 ? J : 8) : 1;  // consecutive channels per thread access
    constexpr int P = J / V;
    constexpr int GPR = kChanTile / V;             // threads per token row
    constexpr int RPP = 64 * K / GPR;              // token rows per access round
    static_assert(T % K == 0 && J % V == 0 && RPP * P == T, "tile must split evenly over the threads");
    constexpr int NV = 2 * S;                      // dB and dC of the wave's states, per token
    constexpr int LPV = 64 / NV;                   // lanes that reduce one of them
    using VIO = vec<V, IO>;
    constexpr int W = VEC ? V * (int)sizeof(IO) / 4 : 1;

    __shared__ f32x2_t s_dk[T][kChanTile];         // (delta, delta*u) per (token, channel)
    __shared__ f32x2_t s_ud[T][kChanTile];         // (u, dp)
    __shared__ float s_p[K][T][kChanTile];         // partial readouts, per wave
    __shared__ float s_du[K][T][kChanTile];        // partial du, per wave
    __shared__ float s_dd[K][T][kChanTile];        // partial d delta, per wave
    // per-wave transposition for dB / dC.  Lane (rk, rgrp) sums row rk at columns rgrp +
    // LPV i; rows are 72 words apart, so each group of 32 lanes reads 32 distinct banks.
    __shared__ float s_red[K][NV][64 + 8];
    __shared__ float s_bc[T][2][N];                // the tile's B and C rows, widened to fp32
    __shared__ float s_dbc[T][2][N];               // the tile's dB / dC sums over its 64 channels
    static_assert(T * 2 * N <= 64 * K, "one B / C element per thread");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rsub = tid / GPR;
    const int cq = (tid % GPR) * V;
    const int tile = blockIdx.x;
    const int b = tile / tiles_per_b;
    const int64_t d0 = (int64_t)(tile - b * tiles_per_b) * kChanTile;
    const int64_t d = d0 + lane;
    const bool act = d < D;
    const bool qact = d0 + cq < D;
    const int64_t dq = qact ? d0 + cq : (D - V) / V * V;
    const int64_t row0 = (int64_t)b * L;
    const bool gated = z != nullptr;
    const int64_t n_ckpt = (L + kCkptEvery - 1) / kCkptEvery;

    float a2[S], G[S], dA_acc[S];   // a2 = A log2(e)
#pragma unroll
    for (int s = 0; s < S; ++s) {
        a2[s] = act ? A[d * N + w * S + s] * kLog2e : 0.0f;
        G[s] = (act && dlast) ? dlast[((int64_t)b * D + d) * N + w * S + s] : 0.0f;
        dA_acc[s] = 0.0f;
    }
    float Dq[V], bq[V], dD_acc[V], db_acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const bool ok = qact && (VEC || d0 + cq + v < D);
        Dq[v] = (ok && Dv) ? Dv[dq + v] : 0.0f;
        bq[v] = (ok && bias) ? bias[dq + v] : 0.0f;
        dD_acc[v] = 0.0f;
        db_acc[v] = 0.0f;
    }
    // The next tile's inputs are fetched into registers as raw I/O words while the current
    // tile is processed, and widened to fp32 only when they are used.
    struct Raw { uint32_t w[W]; };
    auto fetch_raw = [&](const IO *p, int64_t idx, Raw &r) {
        if constexpr (VEC) VIO::load(p, idx, r.w);
        else if constexpr (sizeof(IO) == 2) r.w[0] = p[idx];
        else r.w[0] = __float_as_uint(p[idx]);
    };
    auto widen = [&](const Raw &r, int v) -> float {
        if constexpr (VEC) return VIO::get(r.w, v);
        else if constexpr (sizeof(IO) == 2) return bf16_to_f32((uint16_t)r.w[0]);
        else return __uint_as_float(r.w[0]);
    };
    auto st = [&](IO *p, int64_t idx, const float (&val)[V]) {
        if constexpr (VEC) VIO::store(p, idx, val);
        else io<IO>::st(p, idx, val[0]);
    };

    const int n_tiles = (int)((L + T - 1) / T);
    const int rk = lane / LPV, rgrp = lane % LPV;   // the dB / dC entry this lane sums
    Raw ru[P], rx[P], ry[P], rz[P];
    uint32_t rbc = 0;
    float hn[S];
    auto fetch = [&](int jj) {   // tile jj's inputs, its B / C rows and its checkpoint
        const int64_t tb = (int64_t)jj * T;
        const int ntj = (int)min((int64_t)T, L - tb);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int64_t idx = (row0 + tb + min(p * RPP + rsub, ntj - 1)) * D + dq;   // clamped in bounds
            fetch_raw(u, idx, ru[p]);
            fetch_raw(delta, idx, rx[p]);
            fetch_raw(dy, idx, ry[p]);
            if (gated) fetch_raw(z, idx, rz[p]);
        }
        if (tid < T * 2 * N) {
            const int tt = tid / (2 * N), which = (tid / N) % 2, n = tid % N;
            const IO *src = which ? Cm : Bm;
            const int64_t o = (row0 + tb + min(tt, ntj - 1)) * N + n;
            if constexpr (sizeof(IO) == 2) rbc = src[o];
            else rbc = __float_as_uint(src[o]);
        }
#pragma unroll
        for (int s = 0; s < S; ++s)
            hn[s] = act ? ckpt[(((int64_t)b * n_ckpt + jj) * D + d) * N + w * S + s] : 0.0f;
    };
    fetch(n_tiles - 1);
    for (int j = n_tiles - 1; j >= 0; --j) {
        const int64_t t0 = (int64_t)j * T;
        const int nt = (int)min((int64_t)T, L - t0);

        // 1. per-element preparation.  Tokens past the end and channels past D get zeros: a
        // step with delta = 0, delta*u = 0 and dp = 0 leaves the state and the adjoint
        // unchanged and contributes nothing to any sum, so the tile is processed whole.
        // Kept in registers for the epilogue: kgz = dy silu'(z) (so dz = kgz p) and
        // ksg = softplus'(x); u and dp are read back from LDS.
        float kgz[P][V], ksg[P][V];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tt = p * RPP + rsub;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float uu = widen(ru[p], v), yy = widen(ry[p], v);
                const bool live = tt < nt && qact && (VEC || d0 + cq + v < D);
                const float x = widen(rx[p], v) + bq[v];
                float sg = 1.0f;
                const float sp = softplus ? softplus_f32(x, sg) : x;
                const float dl = live ? sp : 0.0f;
                float g = 1.0f, gz = 0.0f;
                if (gated) {   // silu(z) = z sigmoid(z), silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
                    const float zz = widen(rz[p], v);
                    const float sz = sigmoid_f32(zz);
                    g = zz * sz;
                    gz = yy * (sz * fmaf(zz, 1.0f - sz, 1.0f));
                }
                const float dp = live ? yy * g : 0.0f;
                s_dk[tt][cq + v] = f32x2_t{dl, dl * uu};
                s_ud[tt][cq + v] = f32x2_t{uu, dp};
                kgz[p][v] = gz;
                ksg[p][v] = sg;
            }
        }
        // the tile's B and C rows (shared by every channel) into LDS as fp32
        if (tid < T * 2 * N) {
            const float bcv = sizeof(IO) == 2 ? bf16_to_f32((uint16_t)rbc) : __uint_as_float(rbc);
            s_bc[tid / (2 * N)][(tid / N) % 2][tid % N] = bcv;
        }
        float hs[S];
#pragma unroll
        for (int s = 0; s < S; ++s) hs[s] = hn[s];
        if (j > 0) fetch(j - 1);
        __syncthreads();

        // 2. recompute the tile's states from its checkpoint, keeping h_t and exp(delta_t A)
        float hist[T][S], ex[T][S];
        {
            float h[S];
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = hs[s];
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
                const f32x2_t v = s_dk[tt][lane];
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    ex[tt][s] = hw_exp2(v.x * a2[s]);
                    h[s] = fmaf(ex[tt][s], h[s], v.y * s_bc[tt][0][w * S + s]);
                    hist[tt][s] = h[s];
                    acc = fmaf(s_bc[tt][1][w * S + s], h[s], acc);
                }
                s_p[w][tt][lane] = acc;
            }
        }

        // 3. walk the tile backwards.  With lambda = C dp + G and r = exp(delta A) lambda
        // h_{t-1} (= the new G times h_{t-1}):
        //   dA += delta r,   d delta = sum_n A r + u q,   du = delta q,   q = sum_n lambda B,
        //   dB = lambda delta u,   dC = dp h_t.
        // The dB / dC sums over the wave's 64 channels go through LDS: a token's values are
        // transposed at the start of the next (earlier) token's step, after that token's
        // inputs are requested, and summed at its end.
        float pr[NV], rvp[NV];
        auto transpose = [&]() {   // rvp -> pr: lane (rk, rgrp) gets row rk at columns rgrp + LPV i
#pragma unroll
            for (int k = 0; k < NV; ++k) s_red[w][k][lane] = rvp[k];
            wave_lds_fence();
#pragma unroll
            for (int i = 0; i < NV; ++i) pr[i] = s_red[w][rk][rgrp + LPV * i];
            wave_lds_fence();
        };
        auto finish = [&](int tt) {   // complete the channel sums of token tt
#pragma unroll
            for (int m = 1; m < NV; m *= 2)
#pragma unroll
                for (int i = 0; i + m < NV; i += 2 * m) pr[i] += pr[i + m];
            const float part = group_sum<LPV>(pr[0]);
            if (rgrp == LPV - 1) s_dbc[tt][rk < S ? 0 : 1][w * S + rk % S] = part;
        };
#pragma unroll
        for (int tt = T - 1; tt >= 0; --tt) {
            const f32x2_t dk = s_dk[tt][lane];   // (delta, delta*u)
            const f32x2_t ud = s_ud[tt][lane];   // (u, dp)
            float Bs[S], Cs[S];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                Bs[s] = s_bc[tt][0][w * S + s];
                Cs[s] = s_bc[tt][1][w * S + s];
            }
            if (tt < T - 1) transpose();
            float q = 0.0f, ddA = 0.0f;   // ddA = sum_n A r / ln 2
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float lam = fmaf(Cs[s], ud.y, G[s]);
                G[s] = ex[tt][s] * lam;
                const float r = G[s] * (tt > 0 ? hist[tt > 0 ? tt - 1 : 0][s] : hs[s]);
                dA_acc[s] = fmaf(dk.x, r, dA_acc[s]);
                ddA = fmaf(a2[s], r, ddA);
                q = fmaf(lam, Bs[s], q);
                rvp[s] = lam * dk.y;                 // dB contribution
                rvp[S + s] = ud.y * hist[tt][s];     // dC contribution
            }
            s_du[w][tt][lane] = dk.x * q;
            s_dd[w][tt][lane] = fmaf(ud.x, q, ddA * kLn2);
            if (tt < T - 1) finish(tt + 1);
        }
        transpose();
        finish(0);
        __syncthreads();

        // 4. add the tile's dB / dC sums out (one element per thread), finish the
        // per-element gradients
        if (tid < T * 2 * N) {
            const int tt = tid / (2 * N), which = (tid / N) % 2, n = tid % N;
            if (tt < nt) unsafeAtomicAdd((which ? dC : dB) + (row0 + t0 + tt) * N + n, s_dbc[tt][which][n]);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tt = p * RPP + rsub;
            if (tt < nt && qact) {
                float o_du[V], o_dd[V], o_dz[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const int c = cq + v;
                    const f32x2_t ud = s_ud[tt][c];   // (u, dp)
                    float pp = fmaf(Dq[v], ud.x, s_p[0][tt][c]);
                    float gu = fmaf(Dq[v], ud.y, s_du[0][tt][c]);
                    float gd = s_dd[0][tt][c];
#pragma unroll
                    for (int kk = 1; kk < K; ++kk) {
                        pp += s_p[kk][tt][c];
                        gu += s_du[kk][tt][c];
                        gd += s_dd[kk][tt][c];
                    }
                    const float gx = gd * ksg[p][v];
                    o_du[v] = gu;
                    o_dd[v] = gx;
                    if (gated) o_dz[v] = pp * kgz[p][v];
                    const bool ok = VEC || d0 + c < D;
                    if (ok) {
                        dD_acc[v] = fmaf(ud.y, ud.x, dD_acc[v]);
                        db_acc[v] += gx;
                    }
                }
                const int64_t idx = (row0 + t0 + tt) * D + d0 + cq;
                st(du, idx, o_du);
                st(ddelta, idx, o_dd);
                if (gated) st(dz, idx, o_dz);
            }
        }
    }

    // per-channel sums over this workgroup's tokens (and, through the atomics, the batch)
    if (act) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            unsafeAtomicAdd(dA + d * N + w * S + s, dA_acc[s]);
            if (dh0) dh0[((int64_t)b * D + d) * N + w * S + s] = G[s];
        }
    }
    if (qact) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (VEC || d0 + cq + v < D) {
                if (dD) unsafeAtomicAdd(dD + dq + v, dD_acc[v]);
                if (dbias) unsafeAtomicAdd(dbias + dq + v, db_acc[v]);
            }
        }
    }
}

}  // namespace ssm

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
//   2. recomputes the tile's states from its checkpoint into registers (the wave's S states
//      x kBwdTile tokens) and the partial readouts p,
//   3. walks the tile backwards, accumulating dA in registers, writing per-wave partial du
//      and d delta to LDS, and summing the dB / dC contributions of the tile's 64 channels
//      through a wave-private LDS transposition, added to global memory atomically,
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

__device__ __forceinline__ float sigmoid_f32(float x) { return hw_rcp(1.0f + hw_exp2(-x * kLog2e)); }

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

// Orders this wave's LDS accesses around an exchange between its lanes: the compiler may
// not move memory accesses across it, and it waits until earlier LDS operations are done.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
}

template <int N, typename IO, bool VEC>
__global__ void __launch_bounds__(64 * BwdShape<N>::K)
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

    __shared__ f32x4_t s_in[T][kChanTile];         // (delta, delta*u, u, dp) per (token, channel)
    __shared__ float s_p[K][T][kChanTile];         // partial readouts, per wave
    __shared__ float s_du[K][T][kChanTile];        // partial du, per wave
    __shared__ float s_dd[K][T][kChanTile];        // partial d delta, per wave
    __shared__ float s_red[K][NV][64];             // per-wave transposition for dB / dC
    __shared__ float s_bc[T][2][N];                // the tile's B and C rows, widened to fp32

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

    float a2[S], Aw[S], G[S], dA_acc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        Aw[s] = act ? A[d * N + w * S + s] : 0.0f;
        a2[s] = Aw[s] * kLog2e;
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
    auto ld = [&](const IO *p, int64_t idx, float (&out)[V]) {
        if constexpr (VEC) {
            uint32_t wd[W];
            VIO::load(p, idx, wd);
#pragma unroll
            for (int v = 0; v < V; ++v) out[v] = VIO::get(wd, v);
        } else {
            out[0] = io<IO>::ld(p, idx);
        }
    };
    auto st = [&](IO *p, int64_t idx, const float (&val)[V]) {
        if constexpr (VEC) VIO::store(p, idx, val);
        else io<IO>::st(p, idx, val[0]);
    };

    const int n_tiles = (int)((L + T - 1) / T);
    for (int j = n_tiles - 1; j >= 0; --j) {
        const int64_t t0 = (int64_t)j * T;
        const int nt = (int)min((int64_t)T, L - t0);

        // 1. per-element preparation; the values the epilogue needs stay in registers
        float ku[P][V], kdp[P][V], kdy[P][V], kz[P][V], ksg[P][V];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tt = p * RPP + rsub;
            const int64_t idx = (row0 + t0 + min(tt, nt - 1)) * D + dq;   // clamped in bounds
            float uu[V], xx[V], yy[V], zz[V];
            ld(u, idx, uu);
            ld(delta, idx, xx);
            ld(dy, idx, yy);
            if (gated) ld(z, idx, zz);
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float x = xx[v] + bq[v];
                const float dl = softplus ? softplus_f32(x) : x;
                const float g = gated ? silu_f32(zz[v]) : 1.0f;
                const float dp = yy[v] * g;
                s_in[tt][cq + v] = f32x4_t{dl, dl * uu[v], uu[v], dp};
                ku[p][v] = uu[v];
                kdp[p][v] = dp;
                kdy[p][v] = yy[v];
                kz[p][v] = gated ? zz[v] : 0.0f;
                ksg[p][v] = softplus ? sigmoid_f32(x) : 1.0f;
            }
        }
        // the tile's B and C rows (shared by every channel) into LDS as fp32
        for (int i = tid; i < T * 2 * N; i += 64 * K) {
            const int tt = i / (2 * N), which = (i / N) % 2, n = i % N;
            const int64_t o = (row0 + t0 + min(tt, nt - 1)) * N + n;
            s_bc[tt][which][n] = io<IO>::ld(which ? Cm : Bm, o);
        }
        __syncthreads();

        // 2. recompute the tile's states from its checkpoint
        float hs[S], hist[T][S];
#pragma unroll
        for (int s = 0; s < S; ++s)
            hs[s] = act ? ckpt[(((int64_t)b * n_ckpt + j) * D + d) * N + w * S + s] : 0.0f;
        {
            float h[S];
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = hs[s];
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
                if (tt < nt) {
                    const f32x4_t v = s_in[tt][lane];
                    float Bs[S], Cs[S];
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        Bs[s] = s_bc[tt][0][w * S + s];
                        Cs[s] = s_bc[tt][1][w * S + s];
                    }
                    float acc = 0.0f;
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        h[s] = fmaf(hw_exp2(v.x * a2[s]), h[s], v.y * Bs[s]);
                        hist[tt][s] = h[s];
                        acc = fmaf(Cs[s], h[s], acc);
                    }
                    s_p[w][tt][lane] = acc;
                }
            }
        }

        // 3. walk the tile backwards
#pragma unroll
        for (int tt = T - 1; tt >= 0; --tt) {
            if (tt < nt) {
                const f32x4_t v = s_in[tt][lane];   // (delta, delta*u, u, dp)
                float Bs[S], Cs[S];
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    Bs[s] = s_bc[tt][0][w * S + s];
                    Cs[s] = s_bc[tt][1][w * S + s];
                }
                float du_p = 0.0f, dd_p = 0.0f, rv[NV];
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float lam = fmaf(Cs[s], v.w, G[s]);
                    const float hprev = tt > 0 ? hist[tt > 0 ? tt - 1 : 0][s] : hs[s];
                    const float e = hw_exp2(v.x * a2[s]);
                    const float ah = e * hprev;
                    const float lamd = lam * v.x;
                    dA_acc[s] = fmaf(lamd, ah, dA_acc[s]);
                    dd_p = fmaf(lam, fmaf(Aw[s], ah, Bs[s] * v.z), dd_p);
                    du_p = fmaf(lamd, Bs[s], du_p);
                    rv[s] = act ? lamd * v.z : 0.0f;            // dB contribution
                    rv[S + s] = act ? v.w * hist[tt][s] : 0.0f;  // dC contribution
                    G[s] = e * lam;
                }
                s_du[w][tt][lane] = du_p;
                s_dd[w][tt][lane] = dd_p;
                // sum rv over the 64 channels: transpose through LDS, each lane adds NV
                // entries of one value, then LPV lanes combine with DPP
#pragma unroll
                for (int k = 0; k < NV; ++k) s_red[w][k][lane] = rv[k];
                wave_lds_sync();
                const int k = lane / LPV, grp = lane % LPV;
                float part = 0.0f;
#pragma unroll
                for (int i = 0; i < NV; ++i) part += s_red[w][k][grp * NV + i];
                wave_lds_sync();
                part = group_sum<LPV>(part);
                if (grp == LPV - 1) {
                    const int64_t o = (row0 + t0 + tt) * N + w * S + (k % S);
                    unsafeAtomicAdd(k < S ? dB + o : dC + o, part);
                }
            }
        }
        __syncthreads();

        // 4. finish the per-element gradients
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tt = p * RPP + rsub;
            if (tt < nt && qact) {
                float o_du[V], o_dd[V], o_dz[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const int c = cq + v;
                    float pp = fmaf(Dq[v], ku[p][v], s_p[0][tt][c]);
                    float gu = fmaf(Dq[v], kdp[p][v], s_du[0][tt][c]);
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
                    if (gated) {
                        const float sz = sigmoid_f32(kz[p][v]);
                        o_dz[v] = kdy[p][v] * pp * (sz * fmaf(kz[p][v], 1.0f - sz, 1.0f));
                    }
                    const bool ok = VEC || d0 + c < D;
                    if (ok) {
                        dD_acc[v] = fmaf(kdp[p][v], ku[p][v], dD_acc[v]);
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

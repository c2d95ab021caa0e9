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
// With the exact zero-order hold (ZOH) the input term's coefficient delta becomes
// m = (exp(delta A) - 1) / A, so du_t = D dp_t + sum_n lambda m B, dB += lambda m u, the input
// part of d delta_t is sum_n lambda exp(delta A) B u (d m / d delta = exp(delta A)) and dA gains
// lambda (d m / dA) B u, with d m / dA from zoh_weight_da.
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
//      across the wave's lanes in registers (a reduce-scatter over lane exchanges), added to
//      global memory atomically,
//   4. finishes du, d delta, dz and the dD / d delta_bias sums per element (all threads).
// dA, dB, dC, dD and d delta_bias are sums over workgroups and are accumulated with atomic
// adds into buffers the host has zeroed; their summation order is not fixed.
//
// Split schedule (n_split > 0), as in the forward kernel but mirrored in time: the grid holds
// n_full + 2 n_split workgroups; ids [0, n_full) take whole tiles, ids [n_full, n_full +
// n_split) take the tokens from j_mid * kBwdTile to the end of tiles n_full .. n_tiles-1 and
// hand over the adjoint G they reach at that token (hand, then hflag), ids [n_full + n_split,
// n_full + 2 n_split) wait for it and take tokens [0, j_mid * kBwdTile) of the same tiles.
// Every CU then holds the same amount of work (two whole tiles and one part at 2.5 tiles per
// CU).  The per-element gradients are bitwise those of the whole tile.  A second part whose
// hand-over does not come within wait_ticks forms G itself from the adjoint recurrence
// alone over the first part's tokens (G <- exp(delta A) (C dp + G), no states needed), so no
// placement can hang the kernel and no contribution is counted twice.  hflag must be zero at
// launch.
//
// seq_lens (nullable): sequence b has seq_lens[b] tokens (clamped to [0, L]); its walk starts
// at its last token with the adjoint dlast, tokens past it are identity steps like tokens past
// L (nothing read from them), and du, d delta, dz there are written as zeros (the gradient of
// inputs that reach no output).
#pragma once

#include "scan_kernels.h"

namespace ssm {

constexpr int kBwdTile = kCkptEvery;   // tokens per backward tile: one checkpoint each
constexpr int kPartBatch = 2;          // dB / dC sums stored per this many walked tokens

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

// Sums over the wave's 64 lanes of NV values per lane (NV = 2, 4 or 8), as a reduce-scatter
// in registers: value j ends up summed in the lanes of group j (64 / NV consecutive lanes),
// whose last lane returns the total.  The halves of the values are exchanged between lanes
// l and l ^ 32 (v_permlane32_swap: the upper 32 lanes of its first operand trade places with
// the lower 32 of its second) and added, then between l and l ^ 16 (v_permlane16_swap: odd
// 16-lane rows of the first operand with even rows of the second), then, for NV = 8, between
// l and l ^ 8 within each row (DPP row rotation by 8); each step halves the values per lane.
// The remaining group is summed with group_sum.
template <int NV>
__device__ __forceinline__ float lanes_reduce_scatter(const float (&v)[NV], int lane) {
    static_assert(NV == 2 || NV == 4 || NV == 8, "2, 4 or 8 values");
    auto add_pair = [](float a, float b, bool rows16) {
        const auto p = rows16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                              : __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    };
    float r[NV / 2];
#pragma unroll
    for (int k = 0; k < NV / 2; ++k) r[k] = add_pair(v[k], v[k + NV / 2], false);   // [v_k | v_k+NV/2]
    if constexpr (NV == 2) {
        return group_sum<32>(r[0]);
    } else {
        float q[NV / 4];
#pragma unroll
        for (int k = 0; k < NV / 4; ++k) q[k] = add_pair(r[k], r[k + NV / 4], true);
        if constexpr (NV == 4) {
            return group_sum<16>(q[0]);   // row j holds value j
        } else {
            // rows hold (v0, v2, v4, v6) in q[0] and (v1, v3, v5, v7) in q[1]: lanes 0-7 of a
            // row keep q[0], lanes 8-15 keep q[1], each adding the other half's copy
            const bool lo = (lane & 8) == 0;
            const float keep = lo ? q[0] : q[1];
            const float send = lo ? q[1] : q[0];
            const float t = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x128, 0xf,
                                                                              0xf, false));   // row_ror:8
            return group_sum<8>(t);
        }
    }
}

// Register budget: with 4 waves per workgroup three workgroups share a CU (LDS allows it),
// which needs at most 168 VGPRs per lane.
template <int N, typename IO, bool VEC, bool ZOH = false>
__global__ void __launch_bounds__(64 * BwdShape<N>::K)
__attribute__((amdgpu_waves_per_eu(BwdShape<N>::K == 4 ? 3 : 1)))
scan_bwd_kernel(const IO *__restrict__ u, const IO *__restrict__ delta, const IO *__restrict__ z,
                const IO *__restrict__ dy, const float *__restrict__ A, const float *__restrict__ Dv,
                const float *__restrict__ bias, const IO *__restrict__ Bm, const IO *__restrict__ Cm,
                const float *__restrict__ ckpt, const float *__restrict__ dlast, IO *__restrict__ du,
                IO *__restrict__ ddelta, IO *__restrict__ dz, float *__restrict__ dA, float *__restrict__ dB,
                float *__restrict__ dC, float *__restrict__ dD, float *__restrict__ dbias,
                float *__restrict__ dh0, int64_t L, int64_t D, int tiles_per_b, int softplus, int n_full = 0,
                int n_split = 0, int j_mid = 0, float *__restrict__ hand = nullptr, int *__restrict__ hflag = nullptr,
                unsigned long long wait_ticks = 0, const int32_t *__restrict__ seq_lens = nullptr,
                int *__restrict__ prog = nullptr) {
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

    __shared__ f32x2_t s_dk[T][kChanTile];         // (delta, delta*u) per (token, channel); (delta, u) with ZOH
    __shared__ f32x2_t s_ud[T][kChanTile];         // (u, dp)
    __shared__ float s_p[K][T][kChanTile];         // partial readouts, per wave
    __shared__ float s_du[K][T][kChanTile];        // partial du, per wave
    __shared__ float s_dd[K][T][kChanTile];        // partial d delta, per wave
    __shared__ float s_bc[T][2][N];                // the tile's B and C rows, widened to fp32
    __shared__ float s_dbc[T][2][N];               // the tile's dB / dC sums over its 64 channels
    static_assert(T * 2 * N <= 64 * K, "one B / C element per thread");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rsub = tid / GPR;
    const int cq = (tid % GPR) * V;
    int tile = blockIdx.x, role = kWhole;
    if (n_split > 0 && tile >= n_full) {
        if (tile < n_full + n_split) {
            role = kFirstPart;   // the later tokens, first
        } else {
            tile -= n_split;
            role = kSecondPart;  // the earlier tokens, from the handed-over adjoint
        }
    }
    const int b = tile / tiles_per_b;
    const int64_t d0 = (int64_t)(tile - b * tiles_per_b) * kChanTile;
    const int64_t d = d0 + lane;
    const bool act = d < D;
    const bool qact = d0 + cq < D;
    const int64_t dq = qact ? d0 + cq : (D - V) / V * V;
    const int64_t row0 = (int64_t)b * L;
    const int64_t Lb = seq_lens ? min((int64_t)max(seq_lens[b], 0), L) : L;   // this sequence's tokens
    const bool gated = z != nullptr;
    const int64_t n_ckpt = (L + kCkptEvery - 1) / kCkptEvery;

    float a2[S], G[S], dA_acc[S], inv_a[ZOH ? S : 1];   // a2 = A log2(e); 1 / A for the exact ZOH
#pragma unroll
    for (int s = 0; s < S; ++s) {
        a2[s] = act ? A[d * N + w * S + s] * kLog2e : 0.0f;
        if constexpr (ZOH) inv_a[s] = act ? 1.0f / A[d * N + w * S + s] : 0.0f;
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

    const int n_tiles = (int)((Lb + T - 1) / T);   // (of this sequence)
    const int j_first = (role == kSecondPart ? min(j_mid, n_tiles) : n_tiles) - 1;   // tiles j_first down to j_last
    const int j_last = role == kFirstPart ? j_mid : 0;
    const int rk = lane / LPV, rgrp = lane % LPV;   // the dB / dC entry this lane sums
    Raw ru[P], rx[P], ry[P], rz[P];
    uint32_t rbc = 0;
    float hn[S];
    auto fetch = [&](int jj) {   // tile jj's inputs, its B / C rows and its checkpoint
        const int64_t tb = (int64_t)jj * T;
        const int ntj = (int)min((int64_t)T, Lb - tb);
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
            hn[s] = act ? ckpt[ckpt_index(b, jj, n_ckpt, w, K, D, d, S, s)] : 0.0f;
    };
    if (role == kFirstPart) __builtin_amdgcn_s_setprio(3);
    if (role == kSecondPart) {
        // wait for the first part's adjoint (wave 0 polls; the others wait at the barrier)
        __shared__ int s_handed;
        if (tid < 64) {
            const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
            int okh = 0;
            for (;;) {
                if (__hip_atomic_load(&hflag[tile - n_full], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                    okh = 1;
                    break;
                }
                if (__builtin_amdgcn_s_memrealtime() - w0 > wait_ticks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (tid == 0) s_handed = okh;
        }
        __syncthreads();
        if (s_handed) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (act) {
#pragma unroll
                for (int s = 0; s < S; ++s) G[s] = hand[((int64_t)(tile - n_full) * kChanTile + lane) * N + w * S + s];
            }
        } else if (act) {
            // no hand-over: the adjoint over the first part's tokens, from dlast, with the
            // arithmetic of the reverse walk below (lambda = C dp + G, G = exp(delta A) lambda)
            const float bb = bias ? bias[d] : 0.0f;
            for (int64_t t = Lb - 1; t >= (int64_t)j_mid * T; --t) {
                const int64_t e = (row0 + t) * D + d;
                const float x = io<IO>::ld(delta, e) + bb;
                float sg;
                const float dl = softplus ? (sizeof(IO) == 2 ? softplus_short_f32(x, sg) : softplus_f32(x, sg)) : x;
                const float yy = io<IO>::ld(dy, e);
                float dp = yy;
                if (gated) {
                    const float zz = io<IO>::ld(z, e);
                    dp = yy * (zz * sigmoid_f32(zz));
                }
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float cc = io<IO>::ld(Cm, (row0 + t) * N + w * S + s);
                    const float lam = fmaf(cc, dp, G[s]);
                    G[s] = hw_exp2(dl * a2[s]) * lam;
                }
            }
        }
        __builtin_amdgcn_s_setprio(2);
    }
    // Pacing of the two whole tiles that share a CU (as in the forward's split schedule): each
    // publishes its progress every 4 tiles in prog[id] and reads its sibling's (id +- C,
    // C = grid / 3); the one behind runs at priority 1.  Issue order only: no value depends on it.
    const int n_grid = n_full + 2 * n_split;
    const int c_slots = n_grid / 3;
    const int gid = (int)blockIdx.x;
    const int sib = gid < c_slots ? gid + c_slots : gid - c_slots;
    const bool pace = prog != nullptr && role == kWhole && n_split > 0 && sib >= 0 && sib < n_full;
    int sib_done = 0, steps = 0;
    if (j_first >= j_last) fetch(j_first);
    for (int j = j_first; j >= j_last; --j) {
        if (pace && (steps & 3) == 0) {
            if (sib_done > steps) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            if (w == 0) __hip_atomic_store(&prog[gid], steps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sib_done = __hip_atomic_load(&prog[sib], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        ++steps;
        const int64_t t0 = (int64_t)j * T;
        const int nt = (int)min((int64_t)T, Lb - t0);

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
                // (the forward's step size: the short softplus for bf16 I/O)
                const float sp = softplus ? (sizeof(IO) == 2 ? softplus_short_f32(x, sg) : softplus_f32(x, sg)) : x;
                const float dl = live ? sp : 0.0f;
                float g = 1.0f, gz = 0.0f;
                if (gated) {   // silu(z) = z sigmoid(z), silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
                    const float zz = widen(rz[p], v);
                    const float sz = sigmoid_f32(zz);
                    g = zz * sz;
                    gz = yy * (sz * fmaf(zz, 1.0f - sz, 1.0f));
                }
                const float dp = live ? yy * g : 0.0f;
                s_dk[tt][cq + v] = f32x2_t{dl, ZOH ? uu : dl * uu};
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
        if (j > j_last) fetch(j - 1);
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
                    // (the forward kernel's arithmetic, in its order)
                    const float ya = v.x * a2[s];
                    ex[tt][s] = hw_exp2(ya);
                    float bu = v.y * s_bc[tt][0][w * S + s];
                    if constexpr (ZOH) bu *= zoh_weight(ya, ex[tt][s], v.x, inv_a[s]);
                    h[s] = fmaf(ex[tt][s], h[s], bu);
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
        // The dB / dC sums over the wave's 64 channels are reduced across lanes in registers
        // (lanes_reduce_scatter); the last lane of group rk writes entry rk to LDS.
        float rvp[NV], parts[T];
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
            float q = 0.0f, qe = 0.0f, ddA = 0.0f;   // ddA = sum_n A r / ln 2
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const float lam = fmaf(Cs[s], ud.y, G[s]);
                G[s] = ex[tt][s] * lam;
                const float r = G[s] * (tt > 0 ? hist[tt > 0 ? tt - 1 : 0][s] : hs[s]);
                dA_acc[s] = fmaf(dk.x, r, dA_acc[s]);
                ddA = fmaf(a2[s], r, ddA);
                if constexpr (ZOH) {
                    // m and d m / dA from the recomputed decay (dk.y = u)
                    const float ya = dk.x * a2[s];
                    const float m = zoh_weight(ya, ex[tt][s], dk.x, inv_a[s]);
                    const float mda = zoh_weight_da(ya, ex[tt][s], m, dk.x, inv_a[s]);
                    const float lm = lam * m;
                    dA_acc[s] = fmaf(lam * mda, dk.y * Bs[s], dA_acc[s]);
                    q = fmaf(lm, Bs[s], q);          // du: sum lambda m B
                    qe = fmaf(G[s], Bs[s], qe);      // d delta: u sum lambda exp(delta A) B
                    rvp[s] = lm * dk.y;              // dB contribution
                } else {
                    q = fmaf(lam, Bs[s], q);
                    rvp[s] = lam * dk.y;             // dB contribution
                }
                rvp[S + s] = ud.y * hist[tt][s];     // dC contribution
            }
            s_du[w][tt][lane] = ZOH ? q : dk.x * q;
            s_dd[w][tt][lane] = fmaf(ud.x, ZOH ? qe : q, ddA * kLn2);
            parts[tt] = lanes_reduce_scatter<NV>(rvp, lane);
            // (stored every kPartBatch tokens: a lane-masked store per token splits the unrolled
            // walk and serializes each token's DPP chain behind its wait states -- 38 s_nop per
            // tile, 16 in pairs; B8 L2048 D5120 N16 bf16 backward 1,344 -> 1,333 us -- while all
            // eight held to the end spill to scratch at the 168-register bound)
            if (tt % kPartBatch == 0 && rgrp == LPV - 1) {
#pragma unroll
                for (int k = 0; k < kPartBatch; ++k) s_dbc[tt + k][rk < S ? 0 : 1][w * S + rk % S] = parts[tt + k];
            }
        }
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

    // inputs past this sequence's length reach no output: their gradients are zero (written
    // by the part that covers the sequence's end)
    if (Lb < L && role != kSecondPart && qact) {
        float zv[V];
#pragma unroll
        for (int v = 0; v < V; ++v) zv[v] = 0.0f;
        for (int64_t t = Lb + rsub; t < L; t += RPP) {
            const int64_t idx = (row0 + t) * D + d0 + cq;
            st(du, idx, zv);
            st(ddelta, idx, zv);
            if (gated) st(dz, idx, zv);
        }
    }

    // per-channel sums over this workgroup's tokens (and, through the atomics, the batch)
    if (act) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            unsafeAtomicAdd(dA + d * N + w * S + s, dA_acc[s]);
            if (role == kFirstPart)
                hand[((int64_t)(tile - n_full) * kChanTile + lane) * N + w * S + s] = G[s];
            else if (dh0)
                dh0[((int64_t)b * D + d) * N + w * S + s] = G[s];
        }
    }
    if (role == kFirstPart) {
        // hand the adjoint over: stores, release at device scope, then the flag
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&hflag[tile - n_full], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

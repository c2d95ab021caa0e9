// The causal depthwise convolution over time that produces the scan's input in the block's
// main branch, followed by SiLU (azimuth.plus/paper/mamba, block architecture section: a
// short 1-D convolution of kernel size 4, then SiLU, before the selective SSM).
//
//   out[b, t, d] = act(bias[d] + sum_{k < W} w[d, k] * x[b, t - (W-1) + k, d])
//
// with the inputs before token 0 taken from a state of W-1 rows (zeros without one).
//
// Layout: a thread owns V consecutive channels (one vector access when vectorised) and a
// run of R consecutive tokens of one sequence: kConvRun, or the whole sequence when the
// state is updated in place (so that the thread that reads the old state also writes the
// new one).  Consecutive threads take consecutive channel groups of the same rows, so every
// row access of a wave is one contiguous span.  The W-1 inputs before the run are loaded
// first (from x, or the state before token 0); the run's rows then come kConvBatch at a
// time into two register buffers, the next batch requested before the current one is
// used, and the sliding window of the last W-1 inputs stays in registers.  Every load is
// issued unconditionally (rows clamped into the run; inputs before token 0 without a state
// are loaded from row 0 and replaced by zeros): a conditional load leaves the compiler a
// merge of old and new register values, and the copies it makes there wait for the loads at
// once.  The run that
// ends the sequence writes the final window as the state that continues it.  Bound: HBM
// (x read and out written once; the W-1 halo rows of a run are the previous run's last
// rows, read again).
#pragma once

#include "device_math.h"

namespace ssm {

constexpr int kConvRun = 32;   // tokens per thread
constexpr int kConvBatch = 8;  // rows requested together; the next batch loads while one is used
constexpr int kConvVec = 4;    // channels per thread (8-byte bf16 / 16-byte fp32 accesses)

template <typename IO, int W, int V, bool VEC, bool SILU>
__global__ void __launch_bounds__(256)
conv1d_kernel(const IO *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
              const IO *st_in, IO *__restrict__ out, IO *st_out, int64_t L, int64_t D, int64_t groups,
              int64_t runs, int64_t pairs, int R) {
    using VIO = vec<V, IO>;
    constexpr int WD = VEC ? V * (int)sizeof(IO) / 4 : 1;   // 32-bit words per row access
    constexpr int H = W - 1;                                 // history rows
    // x: channel groups; y: (sequence, run) pairs, uniform over the workgroup, so that row
    // addresses are a scalar base plus the lane's channel offset
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= groups) return;
    const int64_t d0 = g * V;

    float wk[V][W], bv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int k = 0; k < W; ++k) wk[i][k] = w[(d0 + i) * W + k];
        bv[i] = bias ? bias[d0 + i] : 0.0f;
    }
    for (int64_t pr = blockIdx.y; pr < pairs; pr += gridDim.y) {
        const int64_t b = pr / runs;
        const int64_t run = pr - b * runs;
        const int64_t t0 = run * R;
        const int64_t t1 = min(L, t0 + R);
        // a row kept as raw I/O words until it is used (half the registers for bf16)
        auto load_raw = [&](const IO *p, int64_t row, uint32_t (&r)[WD]) {
            if constexpr (VEC && WD == 2) {   // a plain (cached) load: the halo rows are read twice
                const u32x2_t v = *reinterpret_cast<const u32x2_t *>(p + row * D + d0);
                r[0] = v.x;
                r[1] = v.y;
            } else if constexpr (VEC && WD == 4) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p + row * D + d0);
                r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
            } else if constexpr (VEC) VIO::load(p, row * D + d0, r);
            else if constexpr (sizeof(IO) == 2) r[0] = p[row * D + d0];
            else r[0] = __float_as_uint(p[row * D + d0]);
        };
        auto widen = [&](const uint32_t (&r)[WD], int i) -> float {
            if constexpr (VEC) return VIO::get(r, i);
            else if constexpr (sizeof(IO) == 2) return bf16_to_f32((uint16_t)r[0]);
            else return __uint_as_float(r[0]);
        };
        auto store_row = [&](IO *p, int64_t row, const float (&v)[V]) {
            if constexpr (VEC) VIO::store(p, row * D + d0, v);   // streaming (non-temporal) stores
            else io<IO>::st(p, row * D + d0, v[0]);
        };

        // the window: the H inputs before token t0, oldest first (all loads issued, then used)
        float win[H > 0 ? H : 1][V];
        {
            uint32_t wr[H > 0 ? H : 1][WD];
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const int64_t t = t0 - H + j;
                const bool from_x = t >= 0 || !st_in;   // (one load instruction either way)
                load_raw(from_x ? x : st_in, from_x ? b * L + max(t, (int64_t)0) : b * H + (t + H), wr[j]);
            }
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const bool zero = t0 - H + j < 0 && !st_in;
#pragma unroll
                for (int i = 0; i < V; ++i) win[j][i] = zero ? 0.0f : widen(wr[j], i);
            }
        }
        // the run in batches of kConvBatch rows, two register buffers: the next batch's rows are
        // requested before the current batch is used (rows past the run: the run's last row again)
        auto load_batch = [&](int64_t tb, uint32_t (&buf)[kConvBatch][WD]) {
#pragma unroll
            for (int r = 0; r < kConvBatch; ++r) load_raw(x, b * L + min(tb + r, t1 - 1), buf[r]);
        };
        auto use_batch = [&](int64_t tb, const uint32_t (&buf)[kConvBatch][WD]) {
#pragma unroll
            for (int r = 0; r < kConvBatch; ++r) {
                if (tb + r < t1) {
                    float o[V], xr[V];
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        xr[i] = widen(buf[r], i);
                        float acc = bv[i];
#pragma unroll
                        for (int k = 0; k < H; ++k) acc = fmaf(wk[i][k], win[k][i], acc);
                        acc = fmaf(wk[i][H], xr[i], acc);
                        o[i] = SILU ? silu_f32(acc) : acc;
                    }
                    store_row(out, b * L + tb + r, o);
#pragma unroll
                    for (int k = 0; k + 1 < H; ++k)
#pragma unroll
                        for (int i = 0; i < V; ++i) win[k][i] = win[k + 1][i];
                    if constexpr (H > 0) {
#pragma unroll
                        for (int i = 0; i < V; ++i) win[H - 1][i] = xr[i];
                    }
                }
            }
        };
        uint32_t ba[kConvBatch][WD], bb[kConvBatch][WD];
        load_batch(t0, ba);
        for (int64_t tb = t0; tb < t1; tb += 2 * kConvBatch) {
            load_batch(tb + kConvBatch, bb);
            use_batch(tb, ba);
            load_batch(tb + 2 * kConvBatch, ba);
            use_batch(tb + kConvBatch, bb);
        }
        // the run that ends the sequence leaves the state that continues it
        if (st_out && t1 == L) {
#pragma unroll
            for (int j = 0; j < H; ++j) store_row(st_out, b * H + j, win[j]);
        }
    }
}

// The backward pass of the convolution: given dout = dLoss/dout, with
//   g[t]     = dout[t] * act'(pre[t])       (act' = silu'(p) = s (1 + p (1 - s)), s = sigmoid(p);
//                                            1 without the activation)
//   dx[t]    = sum_k w[k] g[t + (W-1) - k]   (g = 0 past the end of the sequence)
//   dw[k]   += g[t] x[t - (W-1) + k],   dbias += g[t]     (sums over sequences and tokens)
//   dstate[r] = sum_{k <= r} w[k] g[r - k]   (the gradient of the W-1 inputs before token 0)
// Layout: lane = a group of V consecutive channels (64 groups per workgroup), wave = one run
// of kConvBwdRun tokens; the four waves of a workgroup take four consecutive runs, whose
// shared halo rows then come from the cache.  A run walks its tokens and the W-1 after them
// in order, with the last W-1 inputs and the last W-1 values of g in registers: at token t
// it forms pre[t] and g[t] and emits dx[t - (W-1)], whose taps then all lie in the window.
// A full run takes a path without per-token branches: its first W-1 tokens (which emit
// nothing, or the state's gradient in the first run) come first, then kConvBwdRun tokens in
// batches of kConvBatch rows that all emit dx; only the last batch tests its tokens against
// the end of the run and of the sequence, with selects.  (A branch per token splits the code
// into blocks between which the compiler copies the two windows into fixed registers.)  A
// run cut short by the end of the sequence takes a general walk.  x and dout rows come a
// batch at a time into two register buffers, the next batch requested before the current
// one is used (rows clamped into the sequence, as in the forward).  The dw / dbias sums stay
// in registers over the runs a thread walks, are added over the workgroup's four waves in
// LDS, and reach global memory with one atomic add per value and workgroup.  Token indices
// are 32-bit (the entry point bounds the sequence length).  Bound: HBM (x, dout read and dx
// written once; halo rows are read again from the cache).
constexpr int kConvBwdRun = 64;    // tokens per run (a multiple of 2 * kConvBatch)
constexpr int kConvBwdWaves = 4;   // runs per workgroup, one per wave
constexpr int kConvBwdVec = 2;     // channels per thread (4-byte bf16 / 8-byte fp32 accesses)

// Zeros two arrays in one launch (the sums the backward adds into).
static __global__ void __launch_bounds__(256) fill_zero2_kernel(float *__restrict__ p, int64_t n, float *__restrict__ q,
                                                         int64_t m) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
    else if (q && i < n + m) q[i - n] = 0.0f;
}

template <typename IO, int W, int V, bool VEC, bool SILU, bool EXACT>
__global__ void __launch_bounds__(64 * kConvBwdWaves)
conv1d_bwd_kernel(const IO *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
                  const IO *__restrict__ st_in, const IO *__restrict__ dout, IO *__restrict__ dx,
                  float *__restrict__ dw, float *__restrict__ dbias, IO *__restrict__ dst, int L, int64_t D,
                  int64_t groups, int runs, int64_t pairs) {
    using VIO = vec<V, IO>;
    constexpr int WD = VEC ? V * (int)sizeof(IO) / 4 : 1;
    constexpr int H = W - 1;
    constexpr int R = kConvBwdRun;
    constexpr int KB = kConvBatch;
    constexpr int NC = V * (W + 1);   // a thread's sums: W taps and the bias per channel
    static_assert(R % (2 * KB) == 0 && R >= 2 * KB && H < KB, "run must split into batch pairs");
    __shared__ float red[kConvBwdWaves][NC][64];
    const int lane = threadIdx.x & 63;
    const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t g = (int64_t)blockIdx.x * 64 + lane;
    // EXACT: the grid covers the channel groups exactly, every lane works
    const bool act = EXACT || g < groups;
    const int64_t d0 = (act ? g : groups - 1) * V;   // idle lanes read a valid group, store nothing

    float wk[V][W], bv[V], sw[V][W], sb[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int k = 0; k < W; ++k) {
            wk[i][k] = w[(d0 + i) * W + k];
            sw[i][k] = 0.0f;
        }
        bv[i] = bias ? bias[d0 + i] : 0.0f;
        sb[i] = 0.0f;
    }
    // A row is addressed as a workgroup-uniform base plus the lane's 32-bit byte offset, which
    // the load and store instructions take as they are (no per-lane 64-bit address arithmetic).
    const uint32_t lofs = (uint32_t)(d0 * (int64_t)sizeof(IO));
    static_assert(!VEC || WD <= 2, "a thread's row access is one 4- or 8-byte word");
    auto load_raw = [&](const IO *p, int64_t row, uint32_t (&r)[WD]) {
        // plain (cached) loads: halo rows are read again
        const char *a = reinterpret_cast<const char *>(p + row * D) + lofs;
        if constexpr (VEC && WD == 2) {
            const u32x2_t v = *reinterpret_cast<const u32x2_t *>(a);
            r[0] = v.x;
            r[1] = v.y;
        } else if constexpr (VEC || sizeof(IO) == 4) {
            r[0] = *reinterpret_cast<const uint32_t *>(a);
        } else {
            r[0] = *reinterpret_cast<const uint16_t *>(a);
        }
    };
    auto widen = [&](const uint32_t (&r)[WD], int i) -> float {
        if constexpr (VEC) return VIO::get(r, i);
        else if constexpr (sizeof(IO) == 2) return bf16_to_f32((uint16_t)r[0]);
        else return __uint_as_float(r[0]);
    };
    auto store_row = [&](IO *p, int64_t row, const float (&v)[V]) {   // streaming (non-temporal) stores
        if (!act) return;
        char *a = reinterpret_cast<char *>(p + row * D) + lofs;
        if constexpr (sizeof(IO) == 2 && V == 2) {
            __builtin_nontemporal_store(f32x2_to_bf16x2(v[0], v[1]), reinterpret_cast<uint32_t *>(a));
        } else if constexpr (sizeof(IO) == 4 && V == 2) {
            const u32x2_t w2 = {__float_as_uint(v[0]), __float_as_uint(v[1])};
            __builtin_nontemporal_store(w2, reinterpret_cast<u32x2_t *>(a));
        } else if constexpr (sizeof(IO) == 2) {
            __builtin_nontemporal_store(f32_to_bf16(v[0]), reinterpret_cast<uint16_t *>(a));
        } else {
            __builtin_nontemporal_store(__float_as_uint(v[0]), reinterpret_cast<uint32_t *>(a));
        }
    };

    for (int64_t q = (int64_t)blockIdx.y * kConvBwdWaves + slot; q < pairs;
         q += (int64_t)gridDim.y * kConvBwdWaves) {
        const int b = (int)(q / runs);
        const int t0 = (int)(q - (int64_t)b * runs) * R;
        const int t1 = min(L, t0 + R);
        const int64_t rb = (int64_t)b * L;   // the sequence's first row
        // the H inputs before t0, oldest first (from x, the state, or zeros); g before t0 is
        // taken as 0: its terms belong to the previous run's dx
        float win[H > 0 ? H : 1][V], gw[H > 0 ? H : 1][V];
        {
            uint32_t wr[H > 0 ? H : 1][WD];
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const int t = t0 - H + j;
                const bool from_x = t >= 0 || !st_in;   // (one load instruction either way)
                load_raw(from_x ? x : st_in, from_x ? rb + max(t, 0) : (int64_t)b * H + (t + H), wr[j]);
            }
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const bool zero = t0 - H + j < 0 && !st_in;
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    win[j][i] = zero ? 0.0f : widen(wr[j], i);
                    gw[j][i] = 0.0f;
                }
            }
        }
        // one token: g from the window and the row, the sums (when in the run), the emitted
        // value o = dx[t - H] (or the state's gradient), the windows advanced
        auto step = [&](const uint32_t (&xw)[WD], const uint32_t (&gwd)[WD], bool in_run, bool in_seq,
                        float (&o)[V]) {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const float xr = widen(xw, i);
                float pre = bv[i];
#pragma unroll
                for (int k = 0; k < H; ++k) pre = fmaf(wk[i][k], win[k][i], pre);
                pre = fmaf(wk[i][H], xr, pre);
                float gg = widen(gwd, i);
                if constexpr (SILU) {
                    const float sg = sigmoid_f32(pre);
                    gg *= sg * fmaf(pre, 1.0f - sg, 1.0f);
                }
                gg = in_seq ? gg : 0.0f;
                const float gr = in_run ? gg : 0.0f;
#pragma unroll
                for (int k = 0; k < H; ++k) sw[i][k] = fmaf(gr, win[k][i], sw[i][k]);
                sw[i][H] = fmaf(gr, xr, sw[i][H]);
                sb[i] += gr;
                // dx[t - H] = w[0] g[t] + w[1] g[t-1] + ... + w[H] g[t-H]
                float e = wk[i][0] * gg;
#pragma unroll
                for (int j = 0; j < H; ++j) e = fmaf(wk[i][H - j], gw[j][i], e);
                o[i] = e;
#pragma unroll
                for (int k = 0; k + 1 < H; ++k) {
                    win[k][i] = win[k + 1][i];
                    gw[k][i] = gw[k + 1][i];
                }
                if constexpr (H > 0) {
                    win[H - 1][i] = xr;
                    gw[H - 1][i] = gg;
                }
            }
        };
        auto load_batch = [&](int tb, uint32_t (&bx)[KB][WD], uint32_t (&bd)[KB][WD]) {
#pragma unroll
            for (int r = 0; r < KB; ++r) {
                const int64_t row = rb + min(tb + r, L - 1);
                load_raw(x, row, bx[r]);
                load_raw(dout, row, bd[r]);
            }
        };
        uint32_t xa[KB][WD], da[KB][WD], xb[KB][WD], db[KB][WD];
        if (t1 - t0 == R) {
            // a full run: tokens t0 .. t0+H-1 first (their dx belongs to the previous run; in the
            // first run they give the state's gradient), then R tokens that each emit
            // dx[t - H], the last H of them past the run (and perhaps past the sequence)
            uint32_t px[H > 0 ? H : 1][WD], pd[H > 0 ? H : 1][WD];
#pragma unroll
            for (int j = 0; j < H; ++j) {
                load_raw(x, rb + t0 + j, px[j]);
                load_raw(dout, rb + t0 + j, pd[j]);
            }
            load_batch(t0 + H, xa, da);
#pragma unroll
            for (int j = 0; j < H; ++j) {
                float o[V];
                step(px[j], pd[j], true, true, o);
                if (t0 == 0 && dst) store_row(dst, (int64_t)b * H + j, o);
            }
            auto use_full = [&](int tb, const uint32_t (&bx)[KB][WD], const uint32_t (&bd)[KB][WD]) {
#pragma unroll
                for (int r = 0; r < KB; ++r) {
                    float o[V];
                    step(bx[r], bd[r], true, true, o);
                    store_row(dx, rb + tb + r - H, o);
                }
            };
            int tb = t0 + H;
#pragma unroll 1
            for (int it = 0; it < R / (2 * KB) - 1; ++it, tb += 2 * KB) {
                load_batch(tb + KB, xb, db);
                use_full(tb, xa, da);
                load_batch(tb + 2 * KB, xa, da);
                use_full(tb + KB, xb, db);
            }
            load_batch(tb + KB, xb, db);
            use_full(tb, xa, da);
            // the last batch: its last H tokens lie past the run, and past the sequence when
            // the run ends it
            tb += KB;
#pragma unroll
            for (int r = 0; r < KB; ++r) {
                float o[V];
                const bool past = r >= KB - H;
                step(xb[r], db[r], !past, !past || tb + r < L, o);
                store_row(dx, rb + tb + r - H, o);
            }
        } else {
            // a run cut short by the end of the sequence: the general walk over [t0, t1 + H)
            const int te = t1 + H;
            auto use_batch = [&](int tb, const uint32_t (&bx)[KB][WD], const uint32_t (&bd)[KB][WD]) {
#pragma unroll
                for (int r = 0; r < KB; ++r) {
                    const int t = tb + r;
                    if (t < te) {
                        float o[V];
                        step(bx[r], bd[r], t < t1, t < L, o);
                        if (t - H >= t0) store_row(dx, rb + t - H, o);
                        else if (t0 == 0 && dst) store_row(dst, (int64_t)b * H + t, o);   // an input before token 0
                    }
                }
            };
            load_batch(t0, xa, da);
            for (int tb = t0; tb < te; tb += 2 * KB) {
                load_batch(tb + KB, xb, db);
                use_batch(tb, xa, da);
                load_batch(tb + 2 * KB, xa, da);
                use_batch(tb + KB, xb, db);
            }
        }
    }
    // the workgroup's sums over its four waves, then one atomic add per value
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int k = 0; k < W; ++k) red[slot][i * (W + 1) + k][lane] = sw[i][k];
        red[slot][i * (W + 1) + W][lane] = sb[i];
    }
    __syncthreads();
    for (int c = slot; c < NC; c += kConvBwdWaves) {
        float s = red[0][c][lane];
#pragma unroll
        for (int j = 1; j < kConvBwdWaves; ++j) s += red[j][c][lane];
        const int i = c / (W + 1), k = c - i * (W + 1);
        if (act) {
            if (k < W) unsafeAtomicAdd(dw + (d0 + i) * W + k, s);
            else if (dbias) unsafeAtomicAdd(dbias + d0 + i, s);
        }
    }
}

}  // namespace ssm

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

}  // namespace ssm

// Selective-scan kernels for gfx950.
//
// Work decomposition (a work item = one sequence b x a tile of 64 channels x one chunk of
// tokens, processed by one workgroup of K = N / S waves):
//  * wave w owns states n in [w*S, (w+1)*S) of all 64 channels, lane = channel.  The
//    fp32 state h and A*log2(e) for those states live in VGPRs for the whole chunk.
//  * B_t and C_t are the same for every channel of a sequence, so for a wave they are
//    uniform: each wave reads its S-wide slice of them with scalar loads into SGPRs
//    (bf16 pairs are widened to fp32 on the scalar ALU), and every per-(token, state)
//    instruction takes them as its scalar operand.
//  * Per-token, per-channel work (the step-size activation, delta*u, the skip term, the
//    SiLU gate, the output rounding) is done once per element, spread over all K waves:
//    a "prep" pass writes (delta, delta*u) for a tile of T tokens into LDS, the waves run
//    the recurrence over the tile writing partial readouts sum_{n in slice} C h into LDS,
//    and an "epilogue" pass adds the K partials, the skip term and the gate and stores y.
//  * Global loads and stores of u, delta, z and y are along channels (lane = channel), so a
//    wave touches 64 consecutive elements of one token row.
// Per (token, channel, state) the recurrence costs one multiply (delta*A), one exp2, one
// multiply (delta*u*B), one FMA (state) and one FMA (readout) -- no more.
//
// Work items (MODE):
//  * kFull / kSummary: one workgroup per (tile, chunk) of the grid -- the single pass, and the
//    first and last passes of the chunk carry (see carry_kernel.h).
#pragma once

#include "device_math.h"

namespace ssm {

constexpr int kChanTile = 64;    // channels per workgroup (one per lane)

enum ScanMode { kFull = 0, kSummary = 1, kCheckpoint = 2 };

// Roles of a workgroup under the split schedule (kFull only): a whole tile, the first part of a
// tile (tokens [0, l_mid), handing its final state over), or the rest of that tile (tokens
// [l_mid, L), starting from the handed-over state).
enum SplitRole { kWhole = 0, kFirstPart = 1, kSecondPart = 2 };

// The second part's wait for its hand-over is bounded (wait_ticks of the 100 MHz constant clock,
// s_memrealtime; the host passes 20 ms by default): a first part takes a few hundred
// microseconds, and the bound only guarantees progress when the first part cannot run.

// kCheckpoint stores the state before every kCkptEvery-th token (for the backward pass).
constexpr int kCkptEvery = 8;

// Index of state s of wave w (states w*S .. w*S+S-1 of channel d) in checkpoint ck of sequence b:
// the layout is [b][ck][w][d][S], so that the S states of the 64 channels a wave holds are one
// contiguous span (its store and its load are whole cache lines).
__device__ __forceinline__ int64_t ckpt_index(int64_t b, int64_t ck, int64_t n_ckpt, int w, int K, int64_t D,
                                              int64_t d, int S, int s) {
    return (((b * n_ckpt + ck) * K + w) * D + d) * S + s;
}

// s_waitcnt immediate that waits for all LDS and scalar-memory operations (lgkmcnt = 0) and
// leaves the vector-memory and export counters unconstrained (gfx9 encoding).
constexpr int kWaitLgkm0 = 0xC07F;

// Element s of a slice of B or C held as raw 32-bit words (bf16 pairs, low half first).
template <typename IO, int BW>
__device__ __forceinline__ float word_f32(const uint32_t (&w)[BW], int s) {
    if constexpr (sizeof(IO) == 2)
        return __uint_as_float((s & 1) ? (w[s >> 1] & 0xffff0000u) : (w[s >> 1] << 16));
    else
        return __uint_as_float(w[s]);
}

// S consecutive B or C values starting at element `off` (a wave-uniform offset), widened
// to fp32.  bf16 pairs are read as 32-bit words (the offset is even whenever S is).
template <int S, typename IO>
__device__ __forceinline__ void load_slice(const IO *__restrict__ p, int64_t off, float (&out)[S]) {
    if constexpr (sizeof(IO) == 2 && S % 2 == 0) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(p + off);
#pragma unroll
        for (int i = 0; i < S / 2; ++i) {
            const uint32_t v = q[i];
            out[2 * i] = __uint_as_float(v << 16);
            out[2 * i + 1] = __uint_as_float(v & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) out[s] = io<IO>::ld(p, off + s);
    }
}

// The scan over (tile, chunk) work items.
//   kFull:    start from the state before the chunk -- for chunk 0 the initial state h0
//             (zero if h0 is null), for a later chunk the carried state cstate[b][c-1], or,
//             with fold, that state composed here from the chunk summaries cstate[b][k] and
//             cdsum[b][k] of the chunks k < c and h0 (no carry pass runs then) --
//             run the recurrence with readout, write y; the last chunk writes last_state.
//             With several chunks and the carry pass the initial state is read from its copy
//             in slot cstate[b][nchunk-1] (written by the carry pass), never from h0, so h0
//             may be the last_state buffer (the host does not fold then).
//   kSummary: start from h = 0, no readout; write the chunk's local final state to
//             cstate[b][c] and the chunk's sum of step sizes to cdsum[b][c].
//   kCheckpoint: one pass from h0 without readout, storing the state before every
//             kCkptEvery-th token to cstate at checkpoint t / kCkptEvery (ckpt_index: the
//             backward pass's recomputation points).
//   CK (kFull): the same checkpoints, to ckpt_out, from the forward itself (a training
//             forward; the backward then skips its kCheckpoint pass).  With the convolution
//             (CW > 0) the training forward scans u rounded to the I/O type, the values the
//             backward reads back from u_out; kSummary takes CK for that rounding alone, so
//             that the chunk states it carries are those of the same u.
//   Split schedule (kFull, n_split > 0): the grid holds n_full + 2 n_split workgroups.  Ids
//             [0, n_full) take whole tiles 0 .. n_full-1; ids [n_full, n_full + n_split)
//             take tokens [0, l_mid) of tiles n_full .. n_tiles-1, store their final state in
//             hand[tile - n_full] and then set hflag[tile - n_full] (release, device scope);
//             ids [n_full + n_split, n_full + 2 n_split) wait for that flag (acquire), start
//             from the handed-over state and take tokens [l_mid, L).  The states are those of
//             the single pass, so the results are bitwise the same.  With 3 workgroups
//             resident per CU and workgroups dispatched round-robin over the CUs, ids c,
//             c + C and c + 2C share CU c, so every CU gets two whole tiles and one part (for
//             n_tiles = 2.5 C): the same work everywhere instead of 3 tiles on half the CUs and
//             2 on the rest.  First parts run at wave priority 3 and second parts at 2 once
//             they start, so the hand-over comes early and the parts do not form the tail.
//             A second part that waits longer than wait_ticks computes the whole tile itself
//             (same values), so no schedule or placement can hang the kernel.  hflag must be
//             zero at launch.
//   seq_lens (nullable): per-sequence token counts; sequence b is scanned over its first
//             seq_lens[b] tokens (clamped to [0, L]): no later token is read or written, and
//             its final state is the state after that many tokens.
//   N: state size; S: states per wave (K = N/S waves); T: tokens per LDS tile.
//   VEC: the prep and epilogue move V consecutive channels of one token per thread
//        (one 16-byte access for 8 bf16); needs D % 8 == 0 and 16-byte aligned u, delta,
//        z, y.  Otherwise one element per access.
//   ZOH: the input term is the exact zero-order hold (exp(delta A) - 1) / A * B * u
//        instead of delta * B * u (the decay is the same).
//   CW:  0, or the width of a causal depthwise convolution + SiLU that produces the scan's
//        input in the kernel: `u` then holds the block's projected input x, and
//        u_t = silu(cb + sum_k cw[k] x_{t-CW+1+k}) (azimuth.plus/paper/mamba, block
//        architecture section), from a zero history before token 0; u_out (if not null)
//        receives it.  The x rows of a tile go into an LDS ring of T + CW - 1 rows (the
//        tile and the CW - 1 rows before it), filled one tile ahead from the prefetched
//        registers; a conv phase with lane = channel (each wave takes the rows its own
//        threads prepare, its CW taps in registers) writes u where the prep reads it.
// (N = 16: three workgroups of four waves must fit on a CU -- the split schedule and the
// one-pass grid are planned for it -- so the register budget is held to 168.)
template <int N, int S, int T, typename IO, int MODE, bool VEC, bool ZOH = false, int CW = 0, bool CK = false>
__global__ void __launch_bounds__(64 * (N / S)) __attribute__((amdgpu_waves_per_eu(N == 16 ? 3 : 1)))
scan_chunk_kernel(const IO *__restrict__ u, const IO *__restrict__ delta,
                  const IO *__restrict__ z, IO *__restrict__ y,
                  const float *__restrict__ A, const float *__restrict__ Dv,
                  const float *__restrict__ bias, const IO *__restrict__ Bm,
                  const IO *__restrict__ Cm, const float *__restrict__ h0, float *__restrict__ last_state,
                  float *__restrict__ cstate, float *__restrict__ cdsum, int64_t L, int64_t D,
                  int tiles_per_b, int n_tiles, int64_t chunk_len, int nchunk, int softplus,
                  const float *__restrict__ conv_w = nullptr, const float *__restrict__ conv_b = nullptr,
                  IO *__restrict__ u_out = nullptr, float *__restrict__ ckpt_out = nullptr,
                  int n_full = 0, int n_split = 0, int64_t l_mid = 0, float *__restrict__ hand = nullptr,
                  int *__restrict__ hflag = nullptr, unsigned long long wait_ticks = 0,
                  const int32_t *__restrict__ seq_lens = nullptr, int *__restrict__ prog = nullptr,
                  int fold = 0) {
    constexpr int K = N / S;
    constexpr int J = T / K;                   // prep / epilogue elements per thread per tile
    constexpr int V = VEC ? (J < 8 ? J : 8) : 1;  // consecutive channels per thread access
    constexpr int P = J / V;                   // accesses per thread per tile
    constexpr int GPR = kChanTile / V;         // threads per token row
    constexpr int RPP = 64 * K / GPR;          // token rows per access round
    constexpr bool READOUT = MODE == kFull;
    static_assert(MODE != kCheckpoint || T % kCkptEvery == 0, "checkpoints fall on tile halves");
    static_assert(T % K == 0 && J % V == 0 && RPP * P == T, "tile must split evenly over the threads");
    using VIO = vec<V, IO>;
    constexpr int W = VEC ? V * (int)sizeof(IO) / 4 : 1;
    // token loop pipelining: groups of G tokens; B / C slices read as BW 32-bit words.  Two
    // groups' slices of B and C live in SGPRs: 32 of them for bf16 at four tokens a group; fp32
    // slices take twice the words, so their groups are two tokens (at four, the 64 SGPRs spilled
    // into VGPR lanes inside the loop: B2 L2048 D1536 fp32 61.2 us against 62.8)
    constexpr bool PIPE = !(sizeof(IO) == 2 && S % 2 == 1) && T % 8 == 0;
    constexpr int G = (sizeof(IO) == 4 && S == 4) ? 2 : 4;
    constexpr int BW = PIPE ? S * (int)sizeof(IO) / 4 : 1;
    // (delta, delta*u) of token tt, channel c at s_dk[tt][sdk(c)]: the 16-byte channel pairs of
    // a row are XOR-permuted by (c / 8) % 8, so that the prep's pair writes (eight threads of a
    // row, 8 channels apart) fall in distinct banks while a row read by lane = channel stays
    // one contiguous span
    __shared__ __attribute__((aligned(16))) f32x2_t s_dk[T][kChanTile];
    // per-wave partial readouts, channel c at s_yp[k][tt][syp(c)]: 16-byte units XOR-permuted
    // by (c / 32) % 2, so that the epilogue's 16-byte reads (eight threads of a row, 32 bytes
    // apart) fall in distinct banks
    __shared__ __attribute__((aligned(16))) float s_yp[READOUT ? K : 1][T][kChanTile];
    constexpr int RS = CW > 0 ? T + CW - 1 : 1;   // rows of the x ring
    __shared__ IO s_x[RS][kChanTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto sdk = [](int c) { return c ^ (((c >> 3) & 7) << 1); };
    auto syp = [](int c) { return c ^ (((c >> 5) & 1) << 2); };
    const int sl = sdk(lane);                  // this lane's channel slot in s_dk
    const int yl = syp(lane);                  // ... in s_yp
    // prep / epilogue mapping: access p of this thread covers token row p*RPP + tid/GPR,
    // channels cq .. cq+V-1 of the tile
    const int rsub = tid / GPR;
    auto row_of = [&](int p) -> int { return p * RPP + rsub; };   // token row of access p
    const int cq = (tid % GPR) * V;
    const bool gated = READOUT && z != nullptr;
    const IO *__restrict__ zsrc = gated ? z : u;
    const int64_t n_items = (int64_t)n_tiles * nchunk;

    const int64_t item = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    int role = kWhole, c = 0, tile;
    if ((MODE == kFull || MODE == kCheckpoint) && n_split > 0) {
        const int g = (int)item;
        if (g >= n_full + 2 * n_split) return;
        if (g < n_full) {
            tile = g;
        } else if (g < n_full + n_split) {
            tile = g;
            role = kFirstPart;
        } else {
            tile = g - n_split;
            role = kSecondPart;
        }
    } else {
        if (item >= n_items) return;
        c = (int)(item / n_tiles);
        tile = (int)(item - (int64_t)c * n_tiles);
    }
    const int b = tile / tiles_per_b;
    const int64_t d0 = (int64_t)(tile - b * tiles_per_b) * kChanTile;
    const int64_t d = d0 + lane;            // channel of this lane in the recurrence
    const bool act = d < D;
    int64_t t_begin = (int64_t)c * chunk_len;
    int64_t t_end = min(L, t_begin + chunk_len);
    if (role == kFirstPart) t_end = l_mid;
    if (role == kSecondPart) t_begin = l_mid;
    // variable lengths: sequence b has seq_lens[b] tokens (clamped to [0, L]); the item's range
    // ends there and may be empty (no token read or written; the state passes through)
    const int64_t len_b = seq_lens ? min((int64_t)max(seq_lens[b], 0), L) : L;
    t_end = min(t_end, len_b);
    if (t_begin > t_end) t_begin = t_end;
    const int64_t row0 = (int64_t)b * L;
    const bool qact = d0 + cq < D;          // whole group in or out (D % V == 0 when VEC)
    const int64_t dq = qact ? d0 + cq : (D - V) / V * V;  // in-bounds channel for loads

    float a2[S], h[S], inv_a[ZOH ? S : 1];   // (1 / A for the zero-order hold)
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float a = act ? A[d * N + w * S + s] : 0.0f;
        a2[s] = a * kLog2e;
        if constexpr (ZOH) inv_a[s] = act ? 1.0f / a : 0.0f;
        h[s] = 0.0f;
    }
    if (role == kFirstPart) __builtin_amdgcn_s_setprio(3);
    if (role == kSecondPart) {
        // wait for the first part's state (wave 0 polls; the others wait at the barrier)
        __shared__ int s_handed;
        if (tid < 64) {
            const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
            int ok = 0;
            for (;;) {
                if (__hip_atomic_load(&hflag[tile - n_full], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
                    ok = 1;
                    break;
                }
                if (__builtin_amdgcn_s_memrealtime() - w0 > wait_ticks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (tid == 0) s_handed = ok;
        }
        __syncthreads();
        if (s_handed) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        } else {
            role = kWhole;   // no hand-over: the whole tile from the initial state
            t_begin = 0;
        }
        __builtin_amdgcn_s_setprio(2);
    }
    if (role == kSecondPart && act) {
#pragma unroll
        for (int s = 0; s < S; ++s) h[s] = hand[((int64_t)(tile - n_full) * kChanTile + lane) * N + w * S + s];
    } else if (MODE == kFull && fold && nchunk > 1 && act) {
        // the state before this chunk composed from the chunk summaries (local final state
        // from zero and summed step size of each earlier chunk), in chunk order:
        // h <- exp(A * sum of delta over chunk k) h + local_k, from the initial state
        if (h0) {
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = h0[((int64_t)b * D + d) * N + w * S + s];
        }
#pragma unroll 4
        for (int k = 0; k < c; ++k) {
            const int64_t row = (int64_t)b * nchunk + k;
            const float ds = cdsum[row * D + d];
            const float *loc = cstate + (row * D + d) * N + w * S;
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = fmaf(hw_exp2(a2[s] * ds), h[s], loc[s]);
        }
    } else if ((MODE == kFull || MODE == kCheckpoint) && act) {
        // the state before this chunk: carried from chunk c-1, or the initial state (read
        // from h0 itself in a single pass, from the copy in slot nchunk-1 otherwise)
        const float *src = nullptr;
        if (c > 0 || (h0 && nchunk > 1))
            src = cstate + (((int64_t)b * nchunk + (c + nchunk - 1) % nchunk) * D + d) * N;
        else if (h0)
            src = h0 + ((int64_t)b * D + d) * N;
        if (src) {
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = src[w * S + s];
        }
    }
    float Dq[V], bq[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const bool ok = qact && (VEC || d0 + cq + v < D);
        Dq[v] = (ok && Dv) ? Dv[dq + v] : 0.0f;
        bq[v] = (ok && bias) ? bias[dq + v] : 0.0f;
    }
    // the convolution's taps and bias for this lane's channel (an in-bounds one for lanes
    // past D, whose values are never stored)
    float cwl[CW > 0 ? CW : 1], cbl = 0.0f;
    if constexpr (CW > 0) {
        const int64_t dc = act ? d : D - 1;
#pragma unroll
        for (int k = 0; k < CW; ++k) cwl[k] = conv_w[dc * CW + k];
        cbl = conv_b ? conv_b[dc] : 0.0f;
    }
    float dsum = 0.0f;

    // Raw inputs of a tile, in two register buffers: the loads of tile i+2 are issued
    // as soon as tile i has been read out of its buffer, so that two tiles of recurrence
    // hide their latency; indices are clamped so every load is in bounds.
    struct Raw { uint32_t u[P][W], d[P][W], z[P][W]; };   // (u holds x with the convolution)
    Raw r0, r1;
    auto load_tile = [&](int64_t t0, Raw &r) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int64_t t = max(min(t0 + row_of(p), t_end - 1), (int64_t)0);
            const int64_t idx = (row0 + t) * D + dq;
            // (z is loaded unconditionally -- from u when there is no gate -- so that the
            // buffer registers carry no conditional value around the loop)
            if constexpr (VEC) {
                // (kept in this order everywhere -- also before the tile loop -- so that
                // the waits for them in the loop can count on a fixed issue order)
                VIO::load(u, idx, r.u[p]);
                __builtin_amdgcn_sched_barrier(0);
                VIO::load(delta, idx, r.d[p]);
                __builtin_amdgcn_sched_barrier(0);
                VIO::load(zsrc, idx, r.z[p]);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                r.u[p][0] = __float_as_uint(io<IO>::ld(u, idx));
                r.d[p][0] = __float_as_uint(io<IO>::ld(delta, idx));
                r.z[p][0] = __float_as_uint(io<IO>::ld(zsrc, idx));
            }
        }
    };
    auto raw = [&](const uint32_t (&r)[W], int v) -> float {
        if constexpr (VEC) return VIO::get(r, v);
        else return __uint_as_float(r[0]);
    };
    load_tile(t_begin, r0);
    load_tile(t_begin + T, r1);
    // The x ring (convolution only): token t of the chunk lives in row
    // (t - t_begin + CW - 1) mod RS.  The base rb of a tile is (its first token - t_begin)
    // mod RS, carried from tile to tile (rb_cur below), so token t0 + tt (tt >= 1 - CW)
    // is in row ring_row(rb, tt).
    auto ring_row = [&](int rb, int tt) -> int {
        const int x = rb + tt + (CW - 1);
        return x >= RS ? x - RS : x;
    };
    auto ring_next = [&](int rb) -> int { return rb + T >= RS ? rb + T - RS : rb + T; };
    int rb_cur = 0;   // ring base of the tile being processed
    // x rows of the tile with ring base rb from a raw buffer into the ring (rows past the
    // end hold clamped copies, never used)
    auto ring_fill = [&](int rb, const Raw &r) {
        if constexpr (CW > 0) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                IO *dst = &s_x[ring_row(rb, row_of(p))][cq];
                if constexpr (VEC) {
#pragma unroll
                    for (int i = 0; i < W; ++i) reinterpret_cast<uint32_t *>(dst)[i] = r.u[p][i];
                } else if constexpr (sizeof(IO) == 2) {
                    dst[0] = (IO)(__float_as_uint(raw(r.u[p], 0)) >> 16);
                } else {
                    dst[0] = raw(r.u[p], 0);
                }
            }
        }
    };
    // the conv phase of the tile at t0: lane = channel; wave w computes u for exactly the
    // rows its own threads prepare (rows p*RPP + w*V .. + V-1 of each access round p), so
    // the prep needs only this wave's LDS writes to be done.  u goes to s_dk[tt][sdk(lane)].x
    // for the prep (and to u_out).
    auto conv_phase = [&](int64_t t0, int rb, int nt) {
        if constexpr (CW > 0) {
            auto xr = [&](int tt) -> float {
                const IO v = s_x[ring_row(rb, tt)][lane];
                if constexpr (sizeof(IO) == 2) return bf16_to_f32(v);
                else return v;
            };
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int tb = p * RPP + w * V;
                float xw[CW];
#pragma unroll
                for (int k = 0; k < CW - 1; ++k) xw[k] = xr(tb - (CW - 1) + k);
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    xw[CW - 1] = xr(tb + i);
                    float acc = cbl;
#pragma unroll
                    for (int k = 0; k < CW; ++k) acc = fmaf(cwl[k], xw[k], acc);
                    float uu = silu_f32(acc);
                    // the training forward scans u as the backward will read it back from
                    // u_out (rounded to the I/O type), so that its checkpoints are that
                    // input's states
                    if constexpr (CK && sizeof(IO) == 2) uu = bf16_to_f32(f32_to_bf16(uu));
                    s_dk[tb + i][sl] = f32x2_t{uu, uu};
#pragma unroll
                    for (int k = 0; k + 1 < CW; ++k) xw[k] = xw[k + 1];
                }
            }
            if (u_out && act) {   // the convolution's output, for the backward pass
                IO *dst = u_out + (row0 + t0) * D + d;
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int tb = p * RPP + w * V;
#pragma unroll
                    for (int i = 0; i < V; ++i)
                        if (tb + i < nt) io<IO>::st(dst, (int64_t)(tb + i) * D, s_dk[tb + i][sl].x);
                }
            }
            // this wave's LDS writes are performed before its later reads (a wavefront's LDS
            // operations complete in order); keep the compiler from moving them
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    };
    if constexpr (CW > 0) {
        // the CW - 1 rows before the chunk (zero before token 0), and the first tile
        for (int i = tid; i < (CW - 1) * kChanTile; i += 64 * K) {
            const int j = i / kChanTile, c = i % kChanTile;
            const int64_t t = t_begin - (CW - 1) + j;
            IO v = IO(0);
            if (t >= 0 && d0 + c < D) v = u[(row0 + t) * D + d0 + c];
            s_x[j][c] = v;   // ring rows 0 .. CW-2 hold the tokens before the chunk
        }
        ring_fill(0, r0);
        __syncthreads();
    }
    // kCheckpoint (and kFull with CK, the training forward): the state before token t (t a
    // multiple of kCkptEvery) into cstate (ckpt_out) at checkpoint t / kCkptEvery
    const int64_t n_ckpt = (L + kCkptEvery - 1) / kCkptEvery;
    auto checkpoint = [&](int64_t t) {
        if ((MODE == kCheckpoint || (MODE == kFull && CK)) && act && t < t_end) {
            float *dst = (MODE == kCheckpoint ? cstate : ckpt_out) + ckpt_index(b, t / kCkptEvery, n_ckpt, w, K, D, d, S, 0);
            // (non-temporal: the checkpoints are read back only by the backward pass, after
            // everything else this kernel touches)
            if constexpr (S == 4) {
                __builtin_nontemporal_store(f32x4_t{h[0], h[1], h[2], h[3]}, reinterpret_cast<f32x4_t *>(dst));
            } else {
#pragma unroll
                for (int s = 0; s < S; ++s) __builtin_nontemporal_store(h[s], dst + s);
            }
        }
    };
    // epilogue of a tile: y = (sum of the K partial readouts + D u) * silu(z), read from
    // s_yp after the recurrence of that tile
    // (the skip term is applied as one explicit FMA, D u + partial_0, so that no tile
    // position is left to the compiler's choice of contraction: results are bitwise the
    // same wherever a tile falls)
    struct DG { float u[P][V], g[P][V]; };
    auto epilogue = [&](int64_t t0, const DG &dg) {
        if (!READOUT) return;
        const int nt = (int)max((int64_t)0, min((int64_t)T, t_end - t0));
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tt = row_of(p);
            if (tt < nt && qact) {
                float part[K][V];   // the K partials of the thread's V channels (4-float units when V % 4 == 0)
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if constexpr (V % 4 == 0) {
#pragma unroll
                        for (int v = 0; v < V; v += 4) {
                            const f32x4_t q = *reinterpret_cast<const f32x4_t *>(&s_yp[k][tt][syp(cq + v)]);
                            part[k][v] = q.x; part[k][v + 1] = q.y; part[k][v + 2] = q.z; part[k][v + 3] = q.w;
                        }
                    } else {
#pragma unroll
                        for (int v = 0; v < V; ++v) part[k][v] = s_yp[k][tt][syp(cq + v)];
                    }
                }
                float yv[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    float a = fmaf(Dq[v], dg.u[p][v], part[0][v]);
#pragma unroll
                    for (int k = 1; k < K; ++k) a += part[k][v];
                    yv[v] = a * dg.g[p][v];
                }
                const int64_t idx = (row0 + t0 + tt) * D + d0 + cq;
                if constexpr (VEC) {
                    VIO::store(y, idx, yv);
                } else {
                    io<IO>::st(y, idx, yv[0]);
                }
            }
        }
    };
    // One tile: the prep of this tile (from loads issued two tiles ago), the epilogue of
    // the previous tile (its stores then retire while this tile runs), the prefetch of the
    // tile after next into the buffer just read, and the recurrence.  A tile past the end
    // is empty (nt = 0).
    auto do_tile = [&](int64_t t0, Raw &r, const Raw &rn, const DG &prev, DG &cur, bool has_prev) {
        const int nt = (int)max((int64_t)0, min((int64_t)T, t_end - t0));
        conv_phase(t0, rb_cur, nt);
        // prep: (delta, delta*u) into LDS (delta*u*log2(e) for the zero-order hold); skip
        // and gate factors kept in registers
        // (without a gate the factors keep the 1.0 they start with)
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int tt = row_of(p);
            f32x2_t dk[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                // (with the convolution, u comes from the conv phase through s_dk)
                const float uu = CW > 0 ? s_dk[tt][sdk(cq + v)].x : raw(r.u[p], v);
                const float x = raw(r.d[p], v) + bq[v];
                const float dl = softplus ? (sizeof(IO) == 2 ? softplus_short_f32(x) : softplus_f32(x)) : x;
                dk[v] = f32x2_t{dl, ZOH ? uu : dl * uu};
                if (READOUT) {
                    cur.u[p][v] = uu;
                    if (gated) cur.g[p][v] = silu_f32(raw(r.z[p], v));
                }
            }
            // (written unmasked: rows of tokens past the end are never read by the
            // recurrence, and lanes of channels past D hold values loaded from an in-bounds
            // channel and are never stored); two channels per 16-byte write when V is even
            if constexpr (V % 2 == 0) {
#pragma unroll
                for (int v = 0; v < V; v += 2)
                    *reinterpret_cast<f32x4_t *>(&s_dk[tt][sdk(cq + v)]) =
                        f32x4_t{dk[v].x, dk[v].y, dk[v + 1].x, dk[v + 1].y};
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) s_dk[tt][sdk(cq + v)] = dk[v];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (has_prev) epilogue(t0 - T, prev);
        // (issued only after the prep has read the buffer, and unconditionally -- past the
        // end the clamped loads are merely redundant -- so that the loads land in the same
        // registers, with no copies and no wait for them at the loop back-edge)
        __builtin_amdgcn_sched_barrier(0);
        load_tile(t0 + 2 * T, r);
        __syncthreads();
        if constexpr (CW > 0) {
            rb_cur = ring_next(rb_cur);
            ring_fill(rb_cur, rn);   // the next tile's x rows (the ring rows this tile read are free)
        }
        // recurrence over the tile: lane = channel, this wave's S states
        checkpoint(t0);
        if (PIPE && nt == T) {
            // A full tile, software-pipelined in groups of G tokens (two register sets,
            // ping-pong): after the wait for the current group, the LDS (delta, delta*u)
            // reads and the scalar B / C loads of the next group are issued, then the
            // current group is computed.  All indices are compile-time constants.
            f32x2_t va[G], vb[G];
            uint32_t ba[G][BW], ca[G][BW], bb[G][BW], cb[G][BW];
            const IO *btile = Bm + (row0 + t0) * N + w * S;
            const IO *ctile = Cm + (row0 + t0) * N + w * S;
            auto gload = [&](int g0, f32x2_t (&v)[G], uint32_t (&bw)[G][BW], uint32_t (&cw)[G][BW]) {
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    // the prefetch after the last group runs past the tile: clamp (unused)
                    const int tt = g0 + i < T ? g0 + i : T - 1;
                    v[i] = s_dk[tt][sl];
                    const uint32_t *bp = reinterpret_cast<const uint32_t *>(btile + tt * N);
                    const uint32_t *cp = reinterpret_cast<const uint32_t *>(ctile + tt * N);
#pragma unroll
                    for (int k = 0; k < BW; ++k) {
                        bw[i][k] = bp[k];
                        cw[i][k] = READOUT ? cp[k] : 0u;
                    }
                }
            };
            auto gcomp = [&](int g0, const f32x2_t (&v)[G], const uint32_t (&bw)[G][BW],
                             const uint32_t (&cw)[G][BW]) {
                // the group's decays first (they depend on the step sizes only): issued back to
                // back, the exponentials run ahead of the state updates that use them (the
                // headline layer 344.7 / 346.0 -> 339.9 / 341.4 us; with each token's decays
                // issued during the previous token's updates instead: 352.7 / 354.0)
                float yg[G][S], eg[G][S];
#pragma unroll
                for (int i = 0; i < G; ++i)
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        yg[i][s] = v[i].x * a2[s];
                        eg[i][s] = hw_exp2(yg[i][s]);
                    }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    float acc = 0.0f;
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        const float ya = yg[i][s];
                        const float e = eg[i][s];
                        float bu = v[i].y * word_f32<IO>(bw[i], s);
                        if constexpr (ZOH) bu *= zoh_weight(ya, e, v[i].x, inv_a[s]);
                        h[s] = fmaf(e, h[s], bu);
                        if (READOUT) acc = fmaf(word_f32<IO>(cw[i], s), h[s], acc);
                    }
                    if (READOUT)
                        s_yp[w][g0 + i][yl] = acc;
                    else if (MODE == kSummary)
                        dsum += v[i].x;
                }
            };
            gload(0, va, ba, ca);
#pragma unroll
            for (int g0 = 0; g0 < T; g0 += 2 * G) {
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                gload(g0 + G, vb, bb, cb);
                __builtin_amdgcn_sched_barrier(0);
                if (g0 > 0 && g0 % kCkptEvery == 0) checkpoint(t0 + g0);
                gcomp(g0, va, ba, ca);
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                gload(g0 + 2 * G, va, ba, ca);
                __builtin_amdgcn_sched_barrier(0);
                gcomp(g0 + G, vb, bb, cb);
            }
        } else {
            // a partial tile (or a slice shape the pipelined loop does not take)
#pragma unroll 4
            for (int tt = 0; tt < nt; ++tt) {
                if (tt > 0 && tt % kCkptEvery == 0) checkpoint(t0 + tt);
                const f32x2_t v = s_dk[tt][sl];
                const int64_t boff = (row0 + t0 + tt) * N + w * S;
                float Bs[S], Cs[S];
                load_slice<S>(Bm, boff, Bs);
                if (READOUT) load_slice<S>(Cm, boff, Cs);
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float ya = v.x * a2[s];
                    const float e = hw_exp2(ya);
                    float bu = v.y * Bs[s];
                    if constexpr (ZOH) bu *= zoh_weight(ya, e, v.x, inv_a[s]);
                    h[s] = fmaf(e, h[s], bu);
                    if (READOUT) acc = fmaf(Cs[s], h[s], acc);
                }
                if (READOUT)
                    s_yp[w][tt][yl] = acc;
                else if (MODE == kSummary)
                    dsum += v.x;
            }
        }
        __syncthreads();
    };
    // Pacing of whole tiles under the split schedule (prog not null): the two whole tiles that
    // share a CU (ids g and g +- C, C = grid / 3, when workgroups are dispatched round-robin
    // over the C CUs) would otherwise progress at different rates -- the older workgroup's
    // waves win the issue arbitration -- and the later one would run its last ~20 % alone on
    // the CU, at one wave per SIMD.  Before each pair of tiles, each publishes the number of
    // pairs it has done in prog[g] and reads its sibling's (used one pair later: no wait on the
    // load); the one behind runs its waves at priority 1, the other at 0 (parts stay above, at
    // 3 and 2).  This only
    // orders issue: the values computed do not depend on it, nor on where the workgroups run.
    const int n_grid = n_full + 2 * n_split;
    const int c_slots = n_grid / 3;
    const int sib = (int)item < c_slots ? (int)item + c_slots : (int)item - c_slots;
    const bool pace = (MODE == kFull || MODE == kCheckpoint) && prog != nullptr && role == kWhole &&
                      n_split > 0 && sib >= 0 && sib < n_full;
    int sib_done = 0;
    // tiles in pairs (two input buffers, two skip/gate sets); the second tile of the last
    // pair may be empty, and its epilogue-of-the-previous-tile still runs
    DG dg0, dg1;
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int v = 0; v < V; ++v) dg0.g[p][v] = dg1.g[p][v] = 1.0f;
    int pairs_done = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * T) {
        if (pace) {
            if (sib_done > pairs_done) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            if (w == 0) __hip_atomic_store(&prog[item], pairs_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sib_done = __hip_atomic_load(&prog[sib], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        do_tile(t0, r0, r1, dg1, dg0, t0 > t_begin);
        do_tile(t0 + T, r1, r0, dg0, dg1, true);
        ++pairs_done;
    }
    {
        // the last pair's second tile (empty or not) still owes its epilogue (no pair: an
        // empty range, nothing to write)
        const int64_t npair = (t_end - t_begin + 2 * T - 1) / (2 * T);
        if (npair > 0) epilogue(t_begin + (2 * npair - 1) * T, dg1);
    }

    if (MODE == kSummary) {
        if (act) {
#pragma unroll
            for (int s = 0; s < S; ++s) cstate[(((int64_t)b * nchunk + c) * D + d) * N + w * S + s] = h[s];
            if (w == 0) cdsum[((int64_t)b * nchunk + c) * D + d] = dsum;
        }
    } else if (role == kFirstPart) {
        // hand the state over: stores, release at device scope, then the flag
        if (act) {
#pragma unroll
            for (int s = 0; s < S; ++s) hand[((int64_t)(tile - n_full) * kChanTile + lane) * N + w * S + s] = h[s];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&hflag[tile - n_full], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (c == nchunk - 1) {
        if (last_state && act) {
#pragma unroll
            for (int s = 0; s < S; ++s) last_state[((int64_t)b * D + d) * N + w * S + s] = h[s];
        }
    }
}

// Copies n elements (a scan of zero tokens leaves the initial state as the final one).
template <typename TP>
__global__ void __launch_bounds__(256) copy_kernel(TP *__restrict__ dst, const TP *__restrict__ src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// Zeros up to kMaxFill buffers of 32-bit words in one launch (the backward's accumulators and
// hand-over flags), each by a grid-stride loop.
constexpr int kMaxFill = 8;
struct FillList {
    uint32_t *p[kMaxFill];
    int64_t n[kMaxFill];
    int count;
};
static __global__ void __launch_bounds__(256) fill_zero_many_kernel(FillList f) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int k = 0; k < f.count; ++k)
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < f.n[k]; i += stride) f.p[k][i] = 0u;
}

// Writes zeros (a scan of zero tokens leaves the zero initial state).
template <typename TP>
__global__ void __launch_bounds__(256) fill_zero_kernel(TP *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = TP(0);
}

}  // namespace ssm

// libssmscan's kernel launches: the schedule (Plan) and, per operation, the templates that
// pick a kernel instantiation for the arguments and launch it on the caller's stream.  The
// templates are instantiated in the inst_*.hip translation units (compiled in parallel) and
// called from the C ABI in ssmscan.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "ssmscan.h"
#include "carry_kernel.h"
#include "scan_kernels.h"
#include "step_kernel.h"
#include "bwd_kernel.h"
#include "conv_kernel.h"
#include "ssd_kernel.h"

namespace ssmlib {

// The status and message of the calling thread's last failure (ssm_last_error); defined in
// ssmscan.hip.
int fail(int code, const char *fmt, ...);
int ok();
// How long a second half of the split schedule waits for its hand-over (ssmscan.hip).
unsigned long long handover_wait_ticks();

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

enum Schedule { kGrid = 0, kCarry = 1, kSplit = 2 };

struct Plan {
    int schedule = kGrid;
    int64_t nchunk = 1;      // chunks per sequence (work items per tile)
    int64_t chunk_len = 0;   // tokens per chunk
    int64_t n_full = 0, n_split = 0, l_mid = 0;   // the split schedule
    bool fold = false;       // chunk carry: the final pass composes the chunk summaries itself
    size_t off_cstate = 0, off_cdsum = 0, off_hand = 0, off_flags = 0, bytes = 0;
};

// One workgroup per (sequence, 64-channel tile) fills the GPU once there are about two
// tiles per CU or more; with fewer tiles the tokens are split into chunks as well (the
// chunk carry), which costs an extra summary pass over all but the last chunk.
// align_ckpt: the call also stores the backward pass's checkpoints (the state before every
// kCkptEvery-th token); each chunk's first token must then be one of those points, so a
// carry chunk length is rounded up to a multiple of kCkptEvery (fewer chunks, never more
// workspace than the plan without the flag).
// Kernel shape per state size: S states per wave (K = N/S waves per workgroup) and T
// tokens per LDS tile.
template <int N> struct ScanShape;
// TC: tokens per LDS tile under the chunk carry.  At N = 16 the carry's many short work items
// run faster with 16-token tiles (B1 L131072 D2048: 1,615 -> 1,499 us; B2 L2048 D1536 fp32:
// 74 -> 69 us), the one-pass and split grids with 32 (B8 L2048 D5120: 367 against 380 us).
template <> struct ScanShape<1> { static constexpr int S = 1, T = 32, TC = 32; };
template <> struct ScanShape<2> { static constexpr int S = 2, T = 32, TC = 32; };
template <> struct ScanShape<4> { static constexpr int S = 4, T = 32, TC = 32; };
template <> struct ScanShape<8> { static constexpr int S = 4, T = 32, TC = 32; };
template <> struct ScanShape<16> { static constexpr int S = 4, T = 32, TC = 16; };

// The fused causal convolution of the scan's input (conv entry point only).
struct ConvArgs {
    const float *w;
    const float *b;
    void *u_out;
};

// Whether three workgroups of a kernel fit on a CU: the split schedule's balance assumes it.
// (Asked of the runtime once per instantiation; on an error the assumption stands and the
// error is cleared so that it is not reported by the next launch.)
inline bool three_per_cu(const void *kernel, int block) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, 0) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return n >= 3;
}

// (CK: the full pass also stores the backward pass's checkpoints to ckpt)
template <int N, int T, typename IO, bool VEC, bool ZOH, int CW, bool CK>
void launch_scan_kernels_t(const IO *u, const IO *dl, const float *A, const IO *B, const IO *C, const float *Dv,
                           const IO *z, const float *bias, int softplus, const float *h0, IO *y, float *last_state,
                           const ssm_dims *dm, const Plan &p, void *ws, hipStream_t st, const ConvArgs &cv,
                           float *ckpt, const int32_t *seq_lens) {
    constexpr int S = ScanShape<N>::S;
    constexpr int K = N / S;
    const int64_t bsz = dm->batch, L = dm->seqlen, D = dm->dim;
    const int tiles_per_b = (int)((D + ssm::kChanTile - 1) / ssm::kChanTile);
    const int n_tiles = (int)(bsz * tiles_per_b);
    const dim3 block(64 * K);
    float *cstate = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_cstate);
    float *cdsum = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_cdsum);
    const int64_t cl = p.chunk_len;
    const int nc = (int)p.nchunk;
    if (p.schedule == kCarry) {
        // (CK also here: with the fused convolution, the training forward scans u rounded to the
        // I/O type, so the summary pass must carry the states of that same u)
        hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kSummary, VEC, ZOH, CW, CK>),
                           dim3((unsigned)n_tiles, (unsigned)(nc - 1)), block, 0, st, u, dl, (const IO *)nullptr,
                           (IO *)nullptr, A, (const float *)nullptr, bias, B, C, (const float *)nullptr,
                           (float *)nullptr, cstate, cdsum, L, D, tiles_per_b, n_tiles, cl, nc, softplus, cv.w, cv.b,
                           (IO *)nullptr, (float *)nullptr, 0, 0, (int64_t)0, (float *)nullptr, (int *)nullptr, 0ull,
                           seq_lens);
        if (!p.fold) {
            const int col_tiles = (int)((D * N + 63) / 64);
            hipLaunchKernelGGL((ssm::carry_scan_kernel<N>), dim3((unsigned)(bsz * col_tiles)), dim3(256), 0, st,
                               cstate, (const float *)cdsum, A, h0, D, nc, col_tiles);
        }
    }
    // An instantiation that needs more registers than three workgroups per CU allow (the fp32
    // fused convolution's) runs a split plan as the one-pass grid, whose outputs are the same:
    // at two per CU the halves queue behind the whole tiles (B8 L2048 D5120 fp32: 615 us split,
    // 570 us one pass).  The plan then has one chunk of L tokens.
    static const bool split_fits = three_per_cu(
        reinterpret_cast<const void *>(&ssm::scan_chunk_kernel<N, S, T, IO, ssm::kFull, VEC, ZOH, CW, CK>), 64 * K);
    if (p.schedule == kSplit && split_fits) {
        // the hand-over flags start at zero (a fill kernel: no memset node if the caller captures a graph)
        int *flags = reinterpret_cast<int *>(static_cast<char *>(ws) + p.off_flags);
        float *hand = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_hand);
        // (the flags are followed by the whole tiles' progress counters, zeroed with them)
        hipLaunchKernelGGL(ssm::fill_zero_kernel<int>, dim3((unsigned)((p.n_split + p.n_full + 255) / 256)), dim3(256), 0,
                           st, flags, p.n_split + p.n_full);
        hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kFull, VEC, ZOH, CW, CK>),
                           dim3((unsigned)(p.n_full + 2 * p.n_split), 1), block, 0, st, u, dl, z, y, A, Dv, bias, B, C,
                           h0, last_state, cstate, cdsum, L, D, tiles_per_b, n_tiles, cl, nc, softplus, cv.w, cv.b,
                           static_cast<IO *>(cv.u_out), ckpt, (int)p.n_full, (int)p.n_split, p.l_mid, hand, flags,
                           handover_wait_ticks(), seq_lens, flags + p.n_split);
        return;
    }
    hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kFull, VEC, ZOH, CW, CK>),
                       dim3((unsigned)n_tiles, (unsigned)nc), block, 0, st, u, dl, z, y, A, Dv, bias, B, C, h0,
                       last_state, cstate, cdsum, L, D, tiles_per_b, n_tiles, cl, nc, softplus, cv.w, cv.b,
                       static_cast<IO *>(cv.u_out), ckpt, 0, 0, (int64_t)0, (float *)nullptr, (int *)nullptr, 0ull,
                       seq_lens, (int *)nullptr, p.schedule == kCarry && p.fold ? 1 : 0);
}

// The scan's launches with the plan's tile length (TC under the chunk carry, else T).
template <int N, typename IO, bool VEC, bool ZOH, int CW = 0, bool CK = false>
void launch_scan_kernels(const IO *u, const IO *dl, const float *A, const IO *B, const IO *C, const float *Dv,
                         const IO *z, const float *bias, int softplus, const float *h0, IO *y, float *last_state,
                         const ssm_dims *dm, const Plan &p, void *ws, hipStream_t st,
                         const ConvArgs &cv = ConvArgs{nullptr, nullptr, nullptr}, float *ckpt = nullptr,
                         const int32_t *seq_lens = nullptr) {
    constexpr int T = ScanShape<N>::T, TC = ScanShape<N>::TC;
    if (TC != T && p.schedule == kCarry)
        launch_scan_kernels_t<N, TC, IO, VEC, ZOH, CW, CK>(u, dl, A, B, C, Dv, z, bias, softplus, h0, y, last_state,
                                                           dm, p, ws, st, cv, ckpt, seq_lens);
    else
        launch_scan_kernels_t<N, T, IO, VEC, ZOH, CW, CK>(u, dl, A, B, C, Dv, z, bias, softplus, h0, y, last_state,
                                                          dm, p, ws, st, cv, ckpt, seq_lens);
}

template <int N, typename IO>
int launch_scan(const void *u, const void *delta, const float *A, const void *B, const void *C,
                const float *Dv, const void *z, const float *bias, int flags, const float *h0, void *y,
                float *last_state, const ssm_dims *dm, const Plan &p, void *ws, hipStream_t st,
                const ConvArgs *cv, float *ckpt, const int32_t *seq_lens) {
    const int softplus = (flags & SSM_SCAN_SOFTPLUS) != 0;
    const bool zoh = (flags & SSM_SCAN_EXACT_ZOH) != 0;
    const IO *u_ = static_cast<const IO *>(u);
    const IO *dl_ = static_cast<const IO *>(delta);
    const IO *z_ = static_cast<const IO *>(z);
    const IO *B_ = static_cast<const IO *>(B);
    const IO *C_ = static_cast<const IO *>(C);
    IO *y_ = static_cast<IO *>(y);
    // 16-byte prep/epilogue accesses need whole groups of 8 channels and aligned rows
    const bool vec = dm->dim % 8 == 0 && aligned(u, 16) && aligned(delta, 16) && aligned(y, 16) &&
                     (!z || aligned(z, 16));
    if (cv) {
        // the fused convolution (width 4; no exact ZOH, checked by the caller), with or without
        // the backward pass's checkpoints
        if (vec && ckpt)
            launch_scan_kernels<N, IO, true, false, 4, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                             last_state, dm, p, ws, st, *cv, ckpt, seq_lens);
        else if (ckpt)
            launch_scan_kernels<N, IO, false, false, 4, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                              last_state, dm, p, ws, st, *cv, ckpt, seq_lens);
        else if (vec)
            launch_scan_kernels<N, IO, true, false, 4>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state,
                                                       dm, p, ws, st, *cv, nullptr, seq_lens);
        else
            launch_scan_kernels<N, IO, false, false, 4>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                        last_state, dm, p, ws, st, *cv, nullptr, seq_lens);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    if (ckpt) {
        // the training forward: the backward pass's checkpoints too
        const ConvArgs none{nullptr, nullptr, nullptr};
        if (vec && zoh)
            launch_scan_kernels<N, IO, true, true, 0, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                            last_state, dm, p, ws, st, none, ckpt, seq_lens);
        else if (vec)
            launch_scan_kernels<N, IO, true, false, 0, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                             last_state, dm, p, ws, st, none, ckpt, seq_lens);
        else if (zoh)
            launch_scan_kernels<N, IO, false, true, 0, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                             last_state, dm, p, ws, st, none, ckpt, seq_lens);
        else
            launch_scan_kernels<N, IO, false, false, 0, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                              last_state, dm, p, ws, st, none, ckpt, seq_lens);
    } else if (vec && zoh)
        launch_scan_kernels<N, IO, true, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm, p,
                                               ws, st, ConvArgs{nullptr, nullptr, nullptr}, nullptr, seq_lens);
    else if (vec)
        launch_scan_kernels<N, IO, true, false>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm,
                                                p, ws, st, ConvArgs{nullptr, nullptr, nullptr}, nullptr, seq_lens);
    else if (zoh)
        launch_scan_kernels<N, IO, false, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm,
                                                p, ws, st, ConvArgs{nullptr, nullptr, nullptr}, nullptr, seq_lens);
    else
        launch_scan_kernels<N, IO, false, false>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm,
                                                 p, ws, st, ConvArgs{nullptr, nullptr, nullptr}, nullptr, seq_lens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// act: 0 -- delta is the activated step size; 1 -- the raw input, activated as the scan does
// (bias, softplus); 2 -- as 1 with the exact zero-order-hold input term.
template <int N, typename IO, int ACT, bool VP>
void launch_step_kernel(dim3 grid, hipStream_t st, float *state, const IO *u, const IO *dl, const float *A,
                        const IO *B, const IO *C, const float *Dv, const IO *z, IO *y, const ssm_dims *dm,
                        const float *bias, int softplus) {
    hipLaunchKernelGGL((ssm::step_kernel<N, IO, VP, ACT>), grid, dim3(256), 0, st, state, u, dl, A, B, C, Dv, z, y,
                       dm->batch, dm->dim, bias, softplus);
}

template <int N, typename IO>
int launch_step(float *state, const void *u, const void *delta, const float *A, const void *B,
                const void *C, const float *Dv, const void *z, void *y, const ssm_dims *dm, hipStream_t st,
                const float *bias, int softplus, int act) {
    constexpr int G = N >= 4 ? N / 4 : 1;
    constexpr int SP = ssm::kStepSeqPerThread;
    const int64_t threads = (dm->batch + SP - 1) / SP * dm->dim * G;
    const dim3 grid((unsigned)((threads + 255) / 256));
    // vector reads of the A, B, C slices of a lane need them aligned to the slice
    const size_t es = sizeof(IO);
    const bool vp = N >= 4 && aligned(A, 16) && aligned(B, 4 * es) && aligned(C, 4 * es);
    const IO *u_ = static_cast<const IO *>(u), *dl_ = static_cast<const IO *>(delta);
    const IO *B_ = static_cast<const IO *>(B), *C_ = static_cast<const IO *>(C), *z_ = static_cast<const IO *>(z);
    IO *y_ = static_cast<IO *>(y);
    if (act == 0) {
        if (vp) launch_step_kernel<N, IO, 0, true>(grid, st, state, u_, dl_, A, B_, C_, Dv, z_, y_, dm, nullptr, 0);
        else launch_step_kernel<N, IO, 0, false>(grid, st, state, u_, dl_, A, B_, C_, Dv, z_, y_, dm, nullptr, 0);
    } else if (act == 1) {
        if (vp) launch_step_kernel<N, IO, 1, true>(grid, st, state, u_, dl_, A, B_, C_, Dv, z_, y_, dm, bias, softplus);
        else launch_step_kernel<N, IO, 1, false>(grid, st, state, u_, dl_, A, B_, C_, Dv, z_, y_, dm, bias, softplus);
    } else {
        if (vp) launch_step_kernel<N, IO, 2, true>(grid, st, state, u_, dl_, A, B_, C_, Dv, z_, y_, dm, bias, softplus);
        else launch_step_kernel<N, IO, 2, false>(grid, st, state, u_, dl_, A, B_, C_, Dv, z_, y_, dm, bias, softplus);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

template <typename TP>
void fill_zero(TP *p, int64_t n, hipStream_t st) {
    if (p && n > 0)
        hipLaunchKernelGGL(ssm::fill_zero_kernel<TP>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
}

struct BwdArgs {
    const float *h0;
    const void *u, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    const float *bias;
    int softplus;
    const void *dy;
    const float *dlast;
    void *du, *ddelta;
    float *dA, *dB, *dC, *dD;
    void *dz;
    float *dbias, *dh0;
    bool ckpt_given;   // the workspace already holds the checkpoints (written by the training forward)
    bool zoh;          // the exact zero-order-hold input term
    ssm::FillList zero;   // the accumulators to zero before the walk (the hand-over flags are added)
    const int32_t *seq_lens = nullptr;   // per-sequence token counts (device), or null
};

// Adds a buffer of n 32-bit words to a fill list (skipped when null or empty).
inline void fill_list_add(ssm::FillList &f, void *p, int64_t n) {
    if (p && n > 0 && f.count < ssm::kMaxFill) {
        f.p[f.count] = static_cast<uint32_t *>(p);
        f.n[f.count] = n;
        ++f.count;
    }
}

inline void launch_fill_list(const ssm::FillList &f, hipStream_t st) {
    int64_t most = 0;
    for (int k = 0; k < f.count; ++k) most = f.n[k] > most ? f.n[k] : most;
    if (most == 0) return;
    const int64_t blocks = std::min<int64_t>((most + 255) / 256, 2048);
    hipLaunchKernelGGL(ssm::fill_zero_many_kernel, dim3((unsigned)blocks), dim3(256), 0, st, f);
}

// sp: the plan of the checkpoint pass (the split schedule, or a one-pass grid); its workspace
// follows the checkpoints, at ckpt_bytes.
template <int N, typename IO>
int launch_bwd(const BwdArgs &a, const ssm_dims *dm, const Plan &sp, size_t ckpt_bytes, void *ws, hipStream_t st) {
    constexpr int S = ScanShape<N>::S, T = ScanShape<N>::T, K = N / S;
    constexpr int KB = ssm::BwdShape<N>::K;
    const int64_t bsz = dm->batch, L = dm->seqlen, D = dm->dim;
    const int tiles_per_b = (int)((D + ssm::kChanTile - 1) / ssm::kChanTile);
    const int n_tiles = (int)(bsz * tiles_per_b);
    const IO *u = static_cast<const IO *>(a.u), *dl = static_cast<const IO *>(a.delta);
    const IO *B = static_cast<const IO *>(a.B), *C = static_cast<const IO *>(a.C);
    const IO *z = static_cast<const IO *>(a.z), *dy = static_cast<const IO *>(a.dy);
    IO *du = static_cast<IO *>(a.du), *ddl = static_cast<IO *>(a.ddelta), *dz = static_cast<IO *>(a.dz);
    float *ckpt = static_cast<float *>(ws);
    // the split schedule's hand-over scratch follows the checkpoints: the checkpoint pass and
    // the reverse walk use its states in turn, each with flags of its own (a second flag array
    // after the plan's); the flags are cleared with the accumulators, in one launch
    const bool split = sp.schedule == kSplit;
    char *spw = static_cast<char *>(ws) + ckpt_bytes;
    int *flags = split ? reinterpret_cast<int *>(spw + sp.off_flags) : nullptr;
    int *wflags = split ? reinterpret_cast<int *>(spw + sp.bytes) : nullptr;
    float *hand = split ? reinterpret_cast<float *>(spw + sp.off_hand) : nullptr;
    ssm::FillList zl = a.zero;
    if (split) {
        // (each flag array is followed by the whole tiles' progress counters)
        fill_list_add(zl, flags, sp.n_split + sp.n_full);
        fill_list_add(zl, wflags, sp.n_split + sp.n_full);
    }
    launch_fill_list(zl, st);
    // forward in checkpoint mode: the state before every kCkptEvery-th token (unless the
    // training forward has stored them already)
    const bool vf = D % 8 == 0 && aligned(u, 16) && aligned(dl, 16);
    if (!a.ckpt_given) {
        // (under the split schedule, as the forward: part of the tiles as two token halves, the
        // second started from the state the first hands over; the checkpoints are the same)
        // (a kernel that cannot hold three workgroups per CU runs the one-pass grid instead)
        auto ckpt_pass = [&](auto vec_c, auto zoh_c) {
            static const bool fits = three_per_cu(
                reinterpret_cast<const void *>(&ssm::scan_chunk_kernel<N, S, T, IO, ssm::kCheckpoint,
                                                                      decltype(vec_c)::value, decltype(zoh_c)::value>),
                64 * K);
            const bool split = sp.schedule == kSplit && fits;
            const unsigned groups = split ? (unsigned)(sp.n_full + 2 * sp.n_split) : (unsigned)n_tiles;
            hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kCheckpoint, decltype(vec_c)::value,
                                                       decltype(zoh_c)::value>),
                               dim3(groups, 1), dim3(64 * K), 0, st, u, dl, (const IO *)nullptr, (IO *)nullptr, a.A,
                               (const float *)nullptr, a.bias, B, C, a.h0, (float *)nullptr, ckpt, (float *)nullptr,
                               L, D, tiles_per_b, n_tiles, L, 1, a.softplus, (const float *)nullptr,
                               (const float *)nullptr, (IO *)nullptr, (float *)nullptr, split ? (int)sp.n_full : 0,
                               split ? (int)sp.n_split : 0, split ? sp.l_mid : (int64_t)0, hand, flags,
                               split ? handover_wait_ticks() : 0ull, a.seq_lens, split ? flags + sp.n_split : nullptr);
        };
        using T1 = std::true_type;
        using F0 = std::false_type;
        if (vf && a.zoh) ckpt_pass(T1{}, T1{});
        else if (vf) ckpt_pass(T1{}, F0{});
        else if (a.zoh) ckpt_pass(F0{}, T1{});
        else ckpt_pass(F0{}, F0{});
    }
    // the reverse walk; 16-byte (or 8-byte) element access when every (token, channel) tensor allows it
    const bool vb = D % 8 == 0 && aligned(u, 16) && aligned(dl, 16) && aligned(dy, 16) && aligned(du, 16) &&
                    aligned(ddl, 16) && (!z || (aligned(z, 16) && aligned(dz, 16)));
    // (under the split schedule too: the later half of a split tile hands the adjoint over;
    // the one-pass grid where three workgroups of the kernel do not fit on a CU)
    auto walk = [&](auto vec_c, auto zoh_c) {
        static const bool fits = three_per_cu(
            reinterpret_cast<const void *>(
                &ssm::scan_bwd_kernel<N, IO, decltype(vec_c)::value, decltype(zoh_c)::value>),
            64 * KB);
        const bool split = sp.schedule == kSplit && fits;
        const unsigned wgroups = split ? (unsigned)(sp.n_full + 2 * sp.n_split) : (unsigned)n_tiles;
        hipLaunchKernelGGL((ssm::scan_bwd_kernel<N, IO, decltype(vec_c)::value, decltype(zoh_c)::value>),
                           dim3(wgroups), dim3(64 * KB), 0, st, u, dl, z, dy, a.A, a.D, a.bias, B, C, ckpt, a.dlast, du,
                           ddl, dz, a.dA, a.dB, a.dC, a.dD, a.dbias, a.dh0, L, D, tiles_per_b, a.softplus,
                           split ? (int)sp.n_full : 0, split ? (int)sp.n_split : 0,
                           split ? (int)(sp.l_mid / ssm::kBwdTile) : 0, hand, wflags,
                           split ? handover_wait_ticks() : 0ull, a.seq_lens, split ? wflags + sp.n_split : nullptr);
    };
    if (vb && a.zoh) walk(std::true_type{}, std::true_type{});
    else if (vb) walk(std::true_type{}, std::false_type{});
    else if (a.zoh) walk(std::false_type{}, std::true_type{});
    else walk(std::false_type{}, std::false_type{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// --- the causal depthwise convolution of the block's main branch ---------------------------

template <typename IO, int W, bool VEC, bool SILU>
void launch_conv_w(const IO *x, const float *w, const float *bias, const IO *st_in, IO *out, IO *st_out,
                   const ssm_dims *dm, hipStream_t st) {
    constexpr int V = VEC ? ssm::kConvVec : 1;
    const int64_t bsz = dm->batch, L = dm->seqlen, D = dm->dim;
    // a state updated in place is read and written by the same thread: one run per sequence
    const bool in_place = st_out && st_out == st_in && W > 1;
    const int64_t R = in_place ? L : ssm::kConvRun;
    const int64_t runs = (L + R - 1) / R;
    const int64_t groups = D / V;
    const int64_t pairs = bsz * runs;
    const dim3 grid((unsigned)((groups + 255) / 256), (unsigned)std::min<int64_t>(pairs, 65535));
    hipLaunchKernelGGL((ssm::conv1d_kernel<IO, W, V, VEC, SILU>), grid, dim3(256), 0, st, x, w, bias, st_in, out,
                       st_out, L, D, groups, runs, pairs, (int)R);
}

template <typename IO, bool VEC, bool SILU>
void launch_conv_v(int width, const IO *x, const float *w, const float *bias, const IO *st_in, IO *out,
                   IO *st_out, const ssm_dims *dm, hipStream_t st) {
    switch (width) {
        case 1: launch_conv_w<IO, 1, VEC, SILU>(x, w, bias, st_in, out, st_out, dm, st); break;
        case 2: launch_conv_w<IO, 2, VEC, SILU>(x, w, bias, st_in, out, st_out, dm, st); break;
        case 3: launch_conv_w<IO, 3, VEC, SILU>(x, w, bias, st_in, out, st_out, dm, st); break;
        default: launch_conv_w<IO, 4, VEC, SILU>(x, w, bias, st_in, out, st_out, dm, st); break;
    }
}

template <typename IO>
int launch_conv(int width, bool silu, const void *x, const float *w, const float *bias, const void *st_in,
                void *out, void *st_out, const ssm_dims *dm, hipStream_t st) {
    const IO *x_ = static_cast<const IO *>(x);
    const IO *si = static_cast<const IO *>(st_in);
    IO *o = static_cast<IO *>(out);
    IO *so = static_cast<IO *>(st_out);
    const size_t va = ssm::kConvVec * sizeof(IO);   // bytes of one vector access
    const bool vec = dm->dim % ssm::kConvVec == 0 && aligned(x, va) && aligned(out, va) &&
                     (!st_in || aligned(st_in, va)) && (!st_out || aligned(st_out, va));
    if (vec && silu) launch_conv_v<IO, true, true>(width, x_, w, bias, si, o, so, dm, st);
    else if (vec) launch_conv_v<IO, true, false>(width, x_, w, bias, si, o, so, dm, st);
    else if (silu) launch_conv_v<IO, false, true>(width, x_, w, bias, si, o, so, dm, st);
    else launch_conv_v<IO, false, false>(width, x_, w, bias, si, o, so, dm, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

template <typename IO, int W, bool VEC, bool SILU>
void launch_conv_bwd_w(const IO *x, const float *w, const float *bias, const IO *st_in, const IO *dout, IO *dx,
                       float *dw, float *dbias, IO *dst, const ssm_dims *dm, hipStream_t st) {
    constexpr int V = VEC ? ssm::kConvBwdVec : 1;
    const int64_t bsz = dm->batch, L = dm->seqlen, D = dm->dim;
    const int64_t R = ssm::kConvBwdRun;
    const int64_t runs = (L + R - 1) / R;
    const int64_t groups = D / V;
    const int64_t pairs = bsz * runs;
    const int64_t quads = (pairs + ssm::kConvBwdWaves - 1) / ssm::kConvBwdWaves;
    const dim3 grid((unsigned)((groups + 63) / 64), (unsigned)std::min<int64_t>(quads, 65535));
    const dim3 block(64 * ssm::kConvBwdWaves);
    if (groups % 64 == 0)
        hipLaunchKernelGGL((ssm::conv1d_bwd_kernel<IO, W, V, VEC, SILU, true>), grid, block, 0, st, x, w, bias, st_in,
                           dout, dx, dw, dbias, dst, (int)L, D, groups, (int)runs, pairs);
    else
        hipLaunchKernelGGL((ssm::conv1d_bwd_kernel<IO, W, V, VEC, SILU, false>), grid, block, 0, st, x, w, bias,
                           st_in, dout, dx, dw, dbias, dst, (int)L, D, groups, (int)runs, pairs);
}

template <typename IO, bool VEC, bool SILU>
void launch_conv_bwd_v(int width, const IO *x, const float *w, const float *bias, const IO *st_in, const IO *dout,
                       IO *dx, float *dw, float *dbias, IO *dst, const ssm_dims *dm, hipStream_t st) {
    switch (width) {
        case 1: launch_conv_bwd_w<IO, 1, VEC, SILU>(x, w, bias, st_in, dout, dx, dw, dbias, dst, dm, st); break;
        case 2: launch_conv_bwd_w<IO, 2, VEC, SILU>(x, w, bias, st_in, dout, dx, dw, dbias, dst, dm, st); break;
        case 3: launch_conv_bwd_w<IO, 3, VEC, SILU>(x, w, bias, st_in, dout, dx, dw, dbias, dst, dm, st); break;
        default: launch_conv_bwd_w<IO, 4, VEC, SILU>(x, w, bias, st_in, dout, dx, dw, dbias, dst, dm, st); break;
    }
}

template <typename IO>
void launch_conv_bwd(int width, bool silu, const void *x, const float *w, const float *bias, const void *st_in,
                     const void *dout, void *dx, float *dw, float *dbias, void *dst, const ssm_dims *dm,
                     hipStream_t st) {
    const IO *x_ = static_cast<const IO *>(x);
    const IO *si = static_cast<const IO *>(st_in);
    const IO *go = static_cast<const IO *>(dout);
    IO *gx = static_cast<IO *>(dx);
    IO *gs = static_cast<IO *>(dst);
    const size_t va = ssm::kConvBwdVec * sizeof(IO);
    const bool vec = dm->dim % ssm::kConvBwdVec == 0 && aligned(x, va) && aligned(dout, va) && aligned(dx, va) &&
                     (!st_in || aligned(st_in, va)) && (!dst || aligned(dst, va));
    if (vec && silu) launch_conv_bwd_v<IO, true, true>(width, x_, w, bias, si, go, gx, dw, dbias, gs, dm, st);
    else if (vec) launch_conv_bwd_v<IO, true, false>(width, x_, w, bias, si, go, gx, dw, dbias, gs, dm, st);
    else if (silu) launch_conv_bwd_v<IO, false, true>(width, x_, w, bias, si, go, gx, dw, dbias, gs, dm, st);
    else launch_conv_bwd_v<IO, false, false>(width, x_, w, bias, si, go, gx, dw, dbias, gs, dm, st);
}


// The SSD layer's launch (inst_misc.hip).
void launch_ssd(const void *x, const void *dt, const float *A, const void *B, const void *C, const float *D,
                const void *z, const float *dt_bias, int softplus, void *y, float *last_state, int64_t bsz,
                int64_t L, int64_t H, int64_t G, hipStream_t st, const float *h0, int64_t P, int64_t N, bool f32);

}  // namespace ssmlib

// libssmscan: C ABI, argument validation, planning and kernel launches.
// The declarations and the contract of every entry point are in include/ssmscan.h.
#include <hip/hip_runtime.h>
#include <algorithm>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "ssmscan.h"
#include "carry_kernel.h"
#include "scan_kernels.h"
#include "step_kernel.h"
#include "bwd_kernel.h"
#include "conv_kernel.h"
#include "ssd_kernel.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return SSM_OK;
}

bool n_supported(int64_t n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 46;
constexpr int kMaxChunks = 65535;  // grid.y limit
constexpr int kTargetGroups = 768; // 3 workgroups per CU on a 256-CU MI355X

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shape checks shared by scan and step.  Returns SSM_OK or a status (message set).
int check_dims(const ssm_dims *dm, bool scan) {
    if (!dm) return fail(SSM_ERR_NULL, "dims is NULL");
    if (dm->batch < 0 || dm->dim < 0 || dm->dstate < 0 || (scan && dm->seqlen < 0))
        return fail(SSM_ERR_SHAPE, "negative size (batch=%lld seqlen=%lld dim=%lld dstate=%lld)",
                    (long long)dm->batch, (long long)dm->seqlen, (long long)dm->dim, (long long)dm->dstate);
    if (dm->io_dtype != SSM_IO_F32 && dm->io_dtype != SSM_IO_BF16)
        return fail(SSM_ERR_DTYPE, "io_dtype %d is not SSM_IO_F32 (0) or SSM_IO_BF16 (1)", dm->io_dtype);
    if (!n_supported(dm->dstate))
        return fail(SSM_ERR_UNSUPPORTED_N, "dstate %lld not supported (1, 2, 4, 8 or 16)", (long long)dm->dstate);
    if (dm->dim > kMaxDim || dm->batch > kMaxDim)
        return fail(SSM_ERR_SHAPE, "dim or batch larger than 2^30");
    if (dm->batch > 0 && dm->dim > (int64_t(1) << 36) / dm->batch)
        return fail(SSM_ERR_SHAPE, "batch*dim exceeds 2^36 (grid size)");
    const int64_t L = scan ? dm->seqlen : 1;
    if (L > kMaxElems || (dm->batch > 0 && dm->dim > 0 && L > kMaxElems / dm->batch / dm->dim))
        return fail(SSM_ERR_SHAPE, "batch*seqlen*dim exceeds 2^46 elements");
    if (scan && dm->chunk_len < -1)
        return fail(SSM_ERR_SHAPE, "chunk_len %d invalid (-1, 0 or > 0)", dm->chunk_len);
    return SSM_OK;
}

enum Schedule { kGrid = 0, kCarry = 1 };

struct Plan {
    int schedule = kGrid;
    int64_t nchunk = 1;      // chunks per sequence (work items per tile)
    int64_t chunk_len = 0;   // tokens per chunk
    size_t off_cstate = 0, off_cdsum = 0, bytes = 0;
};

// One workgroup per (sequence, 64-channel tile) fills the GPU once there are about two
// tiles per CU or more; with fewer tiles the tokens are split into chunks as well (the
// chunk carry), which costs an extra summary pass over all but the last chunk.
Plan make_plan(const ssm_dims *dm) {
    Plan p;
    const int64_t bsz = dm->batch, L = dm->seqlen, D = dm->dim, N = dm->dstate;
    if (bsz == 0 || L == 0 || D == 0) return p;
    const int64_t tiles = bsz * ((D + ssm::kChanTile - 1) / ssm::kChanTile);
    int64_t clen = L;
    if (dm->chunk_len > 0) {
        p.schedule = kCarry;
        clen = dm->chunk_len < L ? dm->chunk_len : L;
        if ((L + clen - 1) / clen > kMaxChunks) clen = (L + kMaxChunks - 1) / kMaxChunks;
    } else if (dm->chunk_len == 0 && tiles < 512 && L >= 512) {
        // too few channel tiles to fill the GPU: split the tokens too.  At least one round of
        // resident workgroups, and chunks of at most 512 tokens so that long sequences give
        // many items (the grid then balances itself over the CUs); chunks of at least 128
        // tokens keep the per-item start-up and the carry small.  (Short sequences stay one
        // pass: three launches would cost more than they save.)
        const int64_t want = std::max((kTargetGroups + tiles - 1) / tiles, (L + 511) / 512);
        const int64_t most = (L + 127) / 128;
        int64_t nchunk = want < most ? want : most;
        if (nchunk < 1) nchunk = 1;
        if (nchunk > kMaxChunks) nchunk = kMaxChunks;
        if (nchunk > 1) {
            p.schedule = kCarry;
            clen = (L + nchunk - 1) / nchunk;
            clen = (clen + 31) / 32 * 32;
        }
    }
    p.chunk_len = clen;
    p.nchunk = (L + clen - 1) / clen;
    if (p.schedule == kCarry && p.nchunk == 1) p.schedule = kGrid;
    if (p.schedule == kCarry) {
        size_t cs = align256((size_t)(bsz * p.nchunk * D * N) * sizeof(float));
        size_t cd = align256((size_t)(bsz * p.nchunk * D) * sizeof(float));
        p.off_cstate = 0;
        p.off_cdsum = cs;
        p.bytes = cs + cd;
    }
    return p;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Kernel shape per state size: S states per wave (K = N/S waves per workgroup) and T
// tokens per LDS tile.
template <int N> struct ScanShape;
template <> struct ScanShape<1> { static constexpr int S = 1, T = 32; };
template <> struct ScanShape<2> { static constexpr int S = 2, T = 32; };
template <> struct ScanShape<4> { static constexpr int S = 4, T = 32; };
template <> struct ScanShape<8> { static constexpr int S = 4, T = 32; };
template <> struct ScanShape<16> { static constexpr int S = 4, T = 32; };

// The fused causal convolution of the scan's input (conv entry point only).
struct ConvArgs {
    const float *w;
    const float *b;
    void *u_out;
};

// (CK: the full pass also stores the backward pass's checkpoints to ckpt)
template <int N, typename IO, bool VEC, bool ZOH, int CW = 0, bool CK = false>
void launch_scan_kernels(const IO *u, const IO *dl, const float *A, const IO *B, const IO *C, const float *Dv,
                         const IO *z, const float *bias, int softplus, const float *h0, IO *y, float *last_state,
                         const ssm_dims *dm, const Plan &p, void *ws, hipStream_t st,
                         const ConvArgs &cv = ConvArgs{nullptr, nullptr, nullptr}, float *ckpt = nullptr) {
    constexpr int S = ScanShape<N>::S;
    constexpr int T = ScanShape<N>::T;
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
        hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kSummary, VEC, ZOH, CW>),
                           dim3((unsigned)n_tiles, (unsigned)(nc - 1)), block, 0, st, u, dl, (const IO *)nullptr,
                           (IO *)nullptr, A, (const float *)nullptr, bias, B, C, (const float *)nullptr,
                           (float *)nullptr, cstate, cdsum, L, D, tiles_per_b, n_tiles, cl, nc, softplus, cv.w, cv.b,
                           (IO *)nullptr);
        const int col_tiles = (int)((D * N + 63) / 64);
        hipLaunchKernelGGL((ssm::carry_scan_kernel<N>), dim3((unsigned)(bsz * col_tiles)), dim3(256), 0, st,
                           cstate, (const float *)cdsum, A, h0, D, nc, col_tiles);
    }
    hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kFull, VEC, ZOH, CW, CK>),
                       dim3((unsigned)n_tiles, (unsigned)nc), block, 0, st, u, dl, z, y, A, Dv, bias, B, C, h0,
                       last_state, cstate, cdsum, L, D, tiles_per_b, n_tiles, cl, nc, softplus, cv.w, cv.b,
                       static_cast<IO *>(cv.u_out), ckpt);
}

template <int N, typename IO>
int launch_scan(const void *u, const void *delta, const float *A, const void *B, const void *C,
                const float *Dv, const void *z, const float *bias, int flags, const float *h0, void *y,
                float *last_state, const ssm_dims *dm, const Plan &p, void *ws, hipStream_t st,
                const ConvArgs *cv, float *ckpt) {
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
                                                             last_state, dm, p, ws, st, *cv, ckpt);
        else if (ckpt)
            launch_scan_kernels<N, IO, false, false, 4, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                              last_state, dm, p, ws, st, *cv, ckpt);
        else if (vec)
            launch_scan_kernels<N, IO, true, false, 4>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state,
                                                       dm, p, ws, st, *cv);
        else
            launch_scan_kernels<N, IO, false, false, 4>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                        last_state, dm, p, ws, st, *cv);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    if (ckpt) {
        // the training forward: the backward pass's checkpoints too (no exact ZOH, checked by the caller)
        const ConvArgs none{nullptr, nullptr, nullptr};
        if (vec)
            launch_scan_kernels<N, IO, true, false, 0, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                             last_state, dm, p, ws, st, none, ckpt);
        else
            launch_scan_kernels<N, IO, false, false, 0, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_,
                                                              last_state, dm, p, ws, st, none, ckpt);
    } else if (vec && zoh)
        launch_scan_kernels<N, IO, true, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm, p,
                                               ws, st);
    else if (vec)
        launch_scan_kernels<N, IO, true, false>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm,
                                                p, ws, st);
    else if (zoh)
        launch_scan_kernels<N, IO, false, true>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm,
                                                p, ws, st);
    else
        launch_scan_kernels<N, IO, false, false>(u_, dl_, A, B_, C_, Dv, z_, bias, softplus, h0, y_, last_state, dm,
                                                 p, ws, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

template <typename IO>
int dispatch_scan(int64_t N, const void *u, const void *delta, const float *A, const void *B,
                  const void *C, const float *Dv, const void *z, const float *bias, int flags, const float *h0,
                  void *y, float *ls, const ssm_dims *dm, const Plan &p, void *ws, hipStream_t st,
                  const ConvArgs *cv, float *ckpt) {
    switch (N) {
        case 1: return launch_scan<1, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt);
        case 2: return launch_scan<2, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt);
        case 4: return launch_scan<4, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt);
        case 8: return launch_scan<8, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt);
        case 16: return launch_scan<16, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt);
    }
    return fail(SSM_ERR_UNSUPPORTED_N, "dstate %lld not supported", (long long)N);
}

template <int N, typename IO>
int launch_step(float *state, const void *u, const void *delta, const float *A, const void *B,
                const void *C, const float *Dv, const void *z, void *y, const ssm_dims *dm, hipStream_t st) {
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
    if (vp)
        hipLaunchKernelGGL((ssm::step_kernel<N, IO, true>), grid, dim3(256), 0, st, state, u_, dl_, A, B_, C_, Dv,
                           z_, y_, dm->batch, dm->dim);
    else
        hipLaunchKernelGGL((ssm::step_kernel<N, IO, false>), grid, dim3(256), 0, st, state, u_, dl_, A, B_, C_, Dv,
                           z_, y_, dm->batch, dm->dim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

template <typename IO>
int dispatch_step(int64_t N, float *state, const void *u, const void *delta, const float *A, const void *B,
                  const void *C, const float *Dv, const void *z, void *y, const ssm_dims *dm, hipStream_t st) {
    switch (N) {
        case 1: return launch_step<1, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st);
        case 2: return launch_step<2, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st);
        case 4: return launch_step<4, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st);
        case 8: return launch_step<8, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st);
        case 16: return launch_step<16, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st);
    }
    return fail(SSM_ERR_UNSUPPORTED_N, "dstate %lld not supported", (long long)N);
}

// ---- backward ----------------------------------------------------------------------------

size_t bwd_workspace_bytes(const ssm_dims *dm) {
    const int64_t n_ckpt = (dm->seqlen + ssm::kCkptEvery - 1) / ssm::kCkptEvery;
    return align256((size_t)(dm->batch * n_ckpt * dm->dim * dm->dstate) * sizeof(float));
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
};

template <int N, typename IO>
int launch_bwd(const BwdArgs &a, const ssm_dims *dm, void *ws, hipStream_t st) {
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
    // forward in checkpoint mode: the state before every kCkptEvery-th token (unless the
    // training forward has stored them already)
    const bool vf = D % 8 == 0 && aligned(u, 16) && aligned(dl, 16);
    if (!a.ckpt_given) {
        if (vf)
            hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kCheckpoint, true>), dim3((unsigned)n_tiles, 1),
                               dim3(64 * K), 0, st, u, dl, (const IO *)nullptr, (IO *)nullptr, a.A,
                               (const float *)nullptr, a.bias, B, C, a.h0, (float *)nullptr, ckpt, (float *)nullptr, L,
                               D, tiles_per_b, n_tiles, L, 1, a.softplus);
        else
            hipLaunchKernelGGL((ssm::scan_chunk_kernel<N, S, T, IO, ssm::kCheckpoint, false>),
                               dim3((unsigned)n_tiles, 1), dim3(64 * K), 0, st, u, dl, (const IO *)nullptr,
                               (IO *)nullptr, a.A, (const float *)nullptr, a.bias, B, C, a.h0, (float *)nullptr, ckpt,
                               (float *)nullptr, L, D, tiles_per_b, n_tiles, L, 1, a.softplus);
    }
    // the reverse walk; 16-byte (or 8-byte) element access when every (token, channel) tensor allows it
    const bool vb = D % 8 == 0 && aligned(u, 16) && aligned(dl, 16) && aligned(dy, 16) && aligned(du, 16) &&
                    aligned(ddl, 16) && (!z || (aligned(z, 16) && aligned(dz, 16)));
    if (vb)
        hipLaunchKernelGGL((ssm::scan_bwd_kernel<N, IO, true>), dim3((unsigned)n_tiles), dim3(64 * KB), 0, st, u, dl,
                           z, dy, a.A, a.D, a.bias, B, C, ckpt, a.dlast, du, ddl, dz, a.dA, a.dB, a.dC, a.dD, a.dbias,
                           a.dh0, L, D, tiles_per_b, a.softplus);
    else
        hipLaunchKernelGGL((ssm::scan_bwd_kernel<N, IO, false>), dim3((unsigned)n_tiles), dim3(64 * KB), 0, st, u, dl,
                           z, dy, a.A, a.D, a.bias, B, C, ckpt, a.dlast, du, ddl, dz, a.dA, a.dB, a.dC, a.dD, a.dbias,
                           a.dh0, L, D, tiles_per_b, a.softplus);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

template <typename IO>
int dispatch_bwd(int64_t N, const BwdArgs &a, const ssm_dims *dm, void *ws, hipStream_t st) {
    switch (N) {
        case 1: return launch_bwd<1, IO>(a, dm, ws, st);
        case 2: return launch_bwd<2, IO>(a, dm, ws, st);
        case 4: return launch_bwd<4, IO>(a, dm, ws, st);
        case 8: return launch_bwd<8, IO>(a, dm, ws, st);
        case 16: return launch_bwd<16, IO>(a, dm, ws, st);
    }
    return fail(SSM_ERR_UNSUPPORTED_N, "dstate %lld not supported", (long long)N);
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

}  // namespace

static int scan_impl(const float *h0, const void *u, const void *delta, const float *A, const void *B,
                     const void *C, const float *D, const void *z, const float *delta_bias, int flags,
                     void *y, float *last_state, const ssm_dims *dims, void *workspace, size_t workspace_bytes,
                     void *stream, const ConvArgs *cv = nullptr) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    if (flags & ~(SSM_SCAN_SOFTPLUS | SSM_SCAN_EXACT_ZOH | SSM_SCAN_CHECKPOINTS))
        return fail(SSM_ERR_FLAGS, "unknown flag bits 0x%x", flags);
    const bool want_ckpt = (flags & SSM_SCAN_CHECKPOINTS) != 0;
    if (want_ckpt && (flags & SSM_SCAN_EXACT_ZOH))
        return fail(SSM_ERR_FLAGS, "checkpoints for the backward pass are not available with the exact ZOH");
    const int64_t bsz = dims->batch, L = dims->seqlen, Dm = dims->dim, N = dims->dstate;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (bsz == 0 || Dm == 0) return ok();
    if (h0 && !aligned(h0, 4)) return fail(SSM_ERR_ALIGN, "initial_state not 4-byte aligned");
    if (L == 0) {
        // no tokens: the final state is the initial one (zero without it)
        if (last_state && last_state != h0) {
            if (!aligned(last_state, 4)) return fail(SSM_ERR_ALIGN, "last_state not 4-byte aligned");
            const int64_t n = bsz * Dm * N;
            const dim3 grid((unsigned)((n + 255) / 256));
            if (h0)
                hipLaunchKernelGGL(ssm::copy_kernel<float>, grid, dim3(256), 0, st, last_state, h0, n);
            else
                hipLaunchKernelGGL(ssm::fill_zero_kernel<float>, grid, dim3(256), 0, st, last_state, n);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        }
        return ok();
    }
    if (!u || !delta || !A || !B || !C || !y)
        return fail(SSM_ERR_NULL, "required pointer is NULL (u=%p delta=%p A=%p B=%p C=%p y=%p)", u, delta,
                    (const void *)A, B, C, y);
    const size_t es = dims->io_dtype == SSM_IO_BF16 ? 2 : 4;
    if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(y, es) ||
        (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
        (delta_bias && !aligned(delta_bias, 4)) || (last_state && !aligned(last_state, 4)))
        return fail(SSM_ERR_ALIGN, "a tensor pointer is not aligned to its element size");
    if (dims->io_dtype == SSM_IO_BF16 && N >= 2 && (!aligned(B, 4) || !aligned(C, 4)))
        return fail(SSM_ERR_ALIGN, "bf16 B and C must be 4-byte aligned");
    if (cv) {
        if (!aligned(cv->u_out, es)) return fail(SSM_ERR_ALIGN, "u_out not aligned to its element size");
        if (!cv->w) return fail(SSM_ERR_NULL, "conv_w is NULL");
        if (!aligned(cv->w, 4) || !aligned(cv->b, 4)) return fail(SSM_ERR_ALIGN, "conv_w / conv_b not 4-byte aligned");
        if (flags & SSM_SCAN_EXACT_ZOH)
            return fail(SSM_ERR_FLAGS, "the exact zero-order hold is not available with the fused convolution");
    }
    Plan p = make_plan(dims);
    // with checkpoints the workspace holds them first (the backward pass's layout), then the plan's carry area
    const size_t ck_bytes = want_ckpt ? bwd_workspace_bytes(dims) : 0, need = ck_bytes + p.bytes;
    if (need > 0 && !workspace) return fail(SSM_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                    need);
    if (need > 0 && !aligned(workspace, 16)) return fail(SSM_ERR_ALIGN, "workspace not 16-byte aligned");
    float *ckpt = want_ckpt ? static_cast<float *>(workspace) : nullptr;
    void *carry_ws = p.bytes > 0 ? static_cast<void *>(static_cast<char *>(workspace) + ck_bytes) : workspace;
    if (dims->io_dtype == SSM_IO_BF16)
        return dispatch_scan<uint16_t>(N, u, delta, A, B, C, D, z, delta_bias, flags, h0, y, last_state, dims, p,
                                       carry_ws, st, cv, ckpt);
    return dispatch_scan<float>(N, u, delta, A, B, C, D, z, delta_bias, flags, h0, y, last_state, dims, p,
                                carry_ws, st, cv, ckpt);
}


extern "C" {

int ssm_version(void) { return SSMSCAN_VERSION; }

const char *ssm_last_error(void) { return g_err.c_str(); }

size_t ssm_scan_workspace_bytes(const ssm_dims *dims) {
    if (check_dims(dims, true) != SSM_OK) return 0;
    return make_plan(dims).bytes;
}

int64_t ssm_scan_plan(const ssm_dims *dims, int64_t *chunk_len_out) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    Plan p = make_plan(dims);
    if (chunk_len_out) *chunk_len_out = p.chunk_len;
    ok();
    return p.schedule == kCarry ? p.nchunk : 1;
}

int ssm_scan_fwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int flags,
                 void *y, float *last_state, const ssm_dims *dims,
                 void *workspace, size_t workspace_bytes, void *stream) {
    return scan_impl(nullptr, u, delta, A, B, C, D, z, delta_bias, flags, y, last_state, dims, workspace,
                     workspace_bytes, stream);
}

int ssm_scan_fwd_from(const float *initial_state, const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z, const float *delta_bias,
                      int flags, void *y, float *last_state, const ssm_dims *dims, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return scan_impl(initial_state, u, delta, A, B, C, D, z, delta_bias, flags, y, last_state, dims,
                     workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_conv(const void *x, const float *conv_w, const float *conv_b, int conv_width, const void *delta,
                      const float *A, const void *B, const void *C, const float *D, const void *z,
                      const float *delta_bias, int flags, void *y, float *last_state, void *u_out,
                      const ssm_dims *dims, void *workspace, size_t workspace_bytes, void *stream) {
    if (conv_width != 4)
        return fail(SSM_ERR_SHAPE, "the fused convolution has width 4 (got %d); use ssm_conv1d_fwd + ssm_scan_fwd",
                    conv_width);
    const ConvArgs cv{conv_w, conv_b, u_out};
    return scan_impl(nullptr, x, delta, A, B, C, D, z, delta_bias, flags, y, last_state, dims, workspace,
                     workspace_bytes, stream, &cv);
}

int ssm_step(float *state, const void *u, const void *delta, const float *A, const void *B,
             const void *C, const float *D, const void *z, void *y, const ssm_dims *dims, void *stream) {
    int rc = check_dims(dims, false);
    if (rc != SSM_OK) return rc;
    const int64_t S = dims->batch, Dm = dims->dim, N = dims->dstate;
    if (S == 0 || Dm == 0) return ok();
    if (!state || !u || !delta || !A || !B || !C || !y)
        return fail(SSM_ERR_NULL, "required pointer is NULL (state=%p u=%p delta=%p A=%p B=%p C=%p y=%p)",
                    (void *)state, u, delta, (const void *)A, B, C, y);
    const size_t es = dims->io_dtype == SSM_IO_BF16 ? 2 : 4;
    if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(y, es) ||
        (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) || !aligned(state, N >= 4 ? 16 : 4))
        return fail(SSM_ERR_ALIGN, "a tensor pointer is not aligned (state needs 16 bytes when dstate >= 4)");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dims->io_dtype == SSM_IO_BF16)
        return dispatch_step<uint16_t>(N, state, u, delta, A, B, C, D, z, y, dims, st);
    return dispatch_step<float>(N, state, u, delta, A, B, C, D, z, y, dims, st);
}

size_t ssm_scan_bwd_workspace_bytes(const ssm_dims *dims) {
    if (check_dims(dims, true) != SSM_OK) return 0;
    return bwd_workspace_bytes(dims);
}

int ssm_scan_bwd(const float *initial_state, const void *u, const void *delta, const float *A, const void *B,
                 const void *C, const float *D, const void *z, const float *delta_bias, int flags,
                 const void *dy, const float *dlast_state, void *du, void *ddelta, float *dA, float *dB,
                 float *dC, float *dD, void *dz, float *ddelta_bias, float *dinitial_state, const ssm_dims *dims,
                 void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    if (flags & ~(SSM_SCAN_SOFTPLUS | SSM_SCAN_CHECKPOINTS))
        return fail(SSM_ERR_FLAGS,
                    "flags 0x%x: the backward pass takes the softplus and checkpoints flags only (no exact ZOH)", flags);
    const int64_t bsz = dims->batch, L = dims->seqlen, Dm = dims->dim, N = dims->dstate;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!A || !dA || (bsz > 0 && L > 0 && Dm > 0 && (!u || !delta || !B || !C || !dy || !du || !ddelta || !dB || !dC)))
        return fail(SSM_ERR_NULL, "required pointer is NULL");
    if (z && !dz) return fail(SSM_ERR_NULL, "z is given but dz is NULL");
    const size_t es = dims->io_dtype == SSM_IO_BF16 ? 2 : 4;
    if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(dy, es) ||
        !aligned(du, es) || !aligned(ddelta, es) || (z && (!aligned(z, es) || !aligned(dz, es))) ||
        !aligned(A, 4) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(dC, 4) || (D && !aligned(D, 4)) ||
        (dD && !aligned(dD, 4)) || (delta_bias && !aligned(delta_bias, 4)) ||
        (ddelta_bias && !aligned(ddelta_bias, 4)) || (initial_state && !aligned(initial_state, 4)) ||
        (dlast_state && !aligned(dlast_state, 4)) || (dinitial_state && !aligned(dinitial_state, 4)))
        return fail(SSM_ERR_ALIGN, "a tensor pointer is not aligned to its element size");
    if (dims->io_dtype == SSM_IO_BF16 && N >= 2 && (!aligned(B, 4) || !aligned(C, 4)))
        return fail(SSM_ERR_ALIGN, "bf16 B and C must be 4-byte aligned");
    const size_t need = bwd_workspace_bytes(dims);
    if (bsz > 0 && L > 0 && Dm > 0) {
        if (!workspace) return fail(SSM_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                        need);
        if (!aligned(workspace, 16)) return fail(SSM_ERR_ALIGN, "workspace not 16-byte aligned");
    }
    // the summed gradients are accumulated atomically: start them from zero
    fill_zero(dA, Dm * N, st);
    fill_zero(dB, bsz * L * N, st);
    fill_zero(dC, bsz * L * N, st);
    fill_zero(dD, Dm, st);
    fill_zero(ddelta_bias, Dm, st);
    if (bsz == 0 || Dm == 0) return ok();
    if (L == 0) {
        // no tokens: the state's gradient passes straight through
        if (dinitial_state) {
            const int64_t n = bsz * Dm * N;
            if (dlast_state)
                hipLaunchKernelGGL(ssm::copy_kernel<float>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                                   dinitial_state, dlast_state, n);
            else
                fill_zero(dinitial_state, n, st);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    BwdArgs a{initial_state, u, delta, A, B, C, D, z, delta_bias, (flags & SSM_SCAN_SOFTPLUS) != 0, dy, dlast_state, du, ddelta,
              dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, (flags & SSM_SCAN_CHECKPOINTS) != 0};
    if (dims->io_dtype == SSM_IO_BF16) return dispatch_bwd<uint16_t>(N, a, dims, workspace, st);
    return dispatch_bwd<float>(N, a, dims, workspace, st);
}

int ssm_conv1d_fwd(const void *x, const float *w, const float *bias, int width, const void *state_in, int flags,
                   void *out, void *state_out, const ssm_dims *dims, void *stream) {
    if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
    ssm_dims d = *dims;   // dstate and chunk_len do not apply
    d.dstate = 1;
    d.chunk_len = 0;
    int rc = check_dims(&d, true);
    if (rc != SSM_OK) return rc;
    if (width < 1 || width > 4) return fail(SSM_ERR_SHAPE, "conv width %d not supported (1 to 4)", width);
    if (flags & ~SSM_CONV_SILU) return fail(SSM_ERR_FLAGS, "unknown flag bits 0x%x", flags);
    const int64_t bsz = d.batch, L = d.seqlen, Dm = d.dim, H = width - 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t es = d.io_dtype == SSM_IO_BF16 ? 2 : 4;
    if (!aligned(x, es) || !aligned(out, es) || !aligned(state_in, es) || !aligned(state_out, es) ||
        !aligned(w, 4) || !aligned(bias, 4))
        return fail(SSM_ERR_ALIGN, "a tensor pointer is not aligned to its element size");
    if (bsz == 0 || Dm == 0) return ok();
    if (!w) return fail(SSM_ERR_NULL, "w is NULL");
    if (L == 0) {
        // no tokens: the state passes through (zero without one)
        if (state_out && state_out != state_in && H > 0) {
            const int64_t n = bsz * H * Dm;
            const dim3 grid((unsigned)((n + 255) / 256));
            if (es == 2) {
                if (state_in)
                    hipLaunchKernelGGL(ssm::copy_kernel<uint16_t>, grid, dim3(256), 0, st,
                                       static_cast<uint16_t *>(state_out), static_cast<const uint16_t *>(state_in), n);
                else
                    hipLaunchKernelGGL(ssm::fill_zero_kernel<uint16_t>, grid, dim3(256), 0, st,
                                       static_cast<uint16_t *>(state_out), n);
            } else {
                if (state_in)
                    hipLaunchKernelGGL(ssm::copy_kernel<float>, grid, dim3(256), 0, st, static_cast<float *>(state_out),
                                       static_cast<const float *>(state_in), n);
                else
                    hipLaunchKernelGGL(ssm::fill_zero_kernel<float>, grid, dim3(256), 0, st,
                                       static_cast<float *>(state_out), n);
            }
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        }
        return ok();
    }
    if (!x || !out) return fail(SSM_ERR_NULL, "x or out is NULL");
    const bool silu = (flags & SSM_CONV_SILU) != 0;
    if (es == 2) return launch_conv<uint16_t>(width, silu, x, w, bias, state_in, out, state_out, &d, st);
    return launch_conv<float>(width, silu, x, w, bias, state_in, out, state_out, &d, st);
}

int ssm_conv1d_bwd(const void *x, const float *w, const float *bias, int width, const void *state_in, int flags,
                   const void *dout, void *dx, float *dw, float *dbias, void *dstate_in, const ssm_dims *dims,
                   void *stream) {
    if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
    ssm_dims d = *dims;   // dstate and chunk_len do not apply
    d.dstate = 1;
    d.chunk_len = 0;
    int rc = check_dims(&d, true);
    if (rc != SSM_OK) return rc;
    if (width < 1 || width > 4) return fail(SSM_ERR_SHAPE, "conv width %d not supported (1 to 4)", width);
    if (flags & ~SSM_CONV_SILU) return fail(SSM_ERR_FLAGS, "unknown flag bits 0x%x", flags);
    const int64_t bsz = d.batch, L = d.seqlen, Dm = d.dim, H = width - 1;
    if (L > (int64_t(1) << 30)) return fail(SSM_ERR_SHAPE, "seqlen %lld exceeds 2^30", (long long)L);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t es = d.io_dtype == SSM_IO_BF16 ? 2 : 4;
    if (!aligned(x, es) || !aligned(dout, es) || !aligned(dx, es) || !aligned(state_in, es) ||
        !aligned(dstate_in, es) || !aligned(w, 4) || !aligned(bias, 4) || !aligned(dw, 4) || !aligned(dbias, 4))
        return fail(SSM_ERR_ALIGN, "a tensor pointer is not aligned to its element size");
    if (Dm == 0) return ok();
    if (!w || !dw) return fail(SSM_ERR_NULL, "w or dw is NULL");
    if (bsz > 0 && L > 0 && (!x || !dout || !dx)) return fail(SSM_ERR_NULL, "x, dout or dx is NULL");
    // the sums start from zero (and stay zero without tokens)
    {
        const int64_t n = Dm * width + (dbias ? Dm : 0);
        hipLaunchKernelGGL(ssm::fill_zero2_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dw,
                           Dm * width, dbias, dbias ? Dm : int64_t(0));
    }
    if (bsz > 0 && L == 0 && dstate_in && H > 0) {   // no output depends on the state
        if (es == 2) fill_zero(static_cast<uint16_t *>(dstate_in), bsz * H * Dm, st);
        else fill_zero(static_cast<float *>(dstate_in), bsz * H * Dm, st);
    }
    if (bsz > 0 && L > 0) {
        const bool silu = (flags & SSM_CONV_SILU) != 0;
        if (es == 2)
            launch_conv_bwd<uint16_t>(width, silu, x, w, bias, state_in, dout, dx, dw, dbias, H > 0 ? dstate_in : nullptr,
                                      &d, st);
        else
            launch_conv_bwd<float>(width, silu, x, w, bias, state_in, dout, dx, dw, dbias, H > 0 ? dstate_in : nullptr,
                                   &d, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int ssm_ssd_fwd(const void *x, const void *dt, const float *A, const void *B, const void *C, const float *D,
                const void *z, const float *dt_bias, int flags, void *y, float *last_state, const ssm_ssd_dims *dims,
                void *stream) {
    if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
    const int64_t bsz = dims->batch, L = dims->seqlen, H = dims->nheads, P = dims->headdim, G = dims->ngroups,
                  N = dims->dstate;
    if (bsz < 0 || L < 0 || H < 0 || P < 0 || G < 1 || N < 0)
        return fail(SSM_ERR_SHAPE, "negative size or ngroups < 1");
    if (dims->io_dtype != SSM_IO_BF16) return fail(SSM_ERR_DTYPE, "the SSD layer takes bf16 I/O only");
    if (P != ssm::kSsdP || N != ssm::kSsdN)
        return fail(SSM_ERR_SHAPE, "headdim %lld and dstate %lld: the SSD kernel supports 64 and 64", (long long)P,
                    (long long)N);
    if (H % G != 0) return fail(SSM_ERR_SHAPE, "nheads %lld is not a multiple of ngroups %lld", (long long)H,
                                (long long)G);
    if (H > kMaxDim || bsz > kMaxDim || (bsz > 0 && H > (int64_t(1) << 31) / bsz))
        return fail(SSM_ERR_SHAPE, "batch*nheads exceeds 2^31 (grid size)");
    if (bsz > 0 && H > 0 && L > kMaxElems / bsz / H / P) return fail(SSM_ERR_SHAPE, "too many elements");
    if (H * P > (int64_t(1) << 24))   // a chunk's rows are addressed with 32-bit offsets
        return fail(SSM_ERR_SHAPE, "nheads*headdim %lld exceeds 2^24", (long long)(H * P));
    if (flags & ~SSM_SCAN_SOFTPLUS) return fail(SSM_ERR_FLAGS, "flags 0x%x: the SSD layer takes the softplus flag only",
                                                flags);
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(z, 16) ||
        !aligned(dt, 2) || !aligned(A, 4) || !aligned(D, 4) || !aligned(dt_bias, 4) || !aligned(last_state, 4))
        return fail(SSM_ERR_ALIGN, "x, z, y, B, C must be 16-byte aligned and the others aligned to their element size");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (bsz == 0 || H == 0) return ok();
    if (!A || (L > 0 && (!x || !dt || !B || !C || !y))) return fail(SSM_ERR_NULL, "required pointer is NULL");
    if (L == 0) {
        if (last_state) fill_zero(last_state, bsz * H * P * N, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    hipLaunchKernelGGL(ssm::ssd_chunk_kernel, dim3((unsigned)(bsz * H)), dim3(ssm::kSsdThreads), 0, st,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dt), A,
                       static_cast<const uint16_t *>(B), static_cast<const uint16_t *>(C), D,
                       static_cast<const uint16_t *>(z), dt_bias, static_cast<uint16_t *>(y), last_state, L, (int)H,
                       (int)G, (flags & SSM_SCAN_SOFTPLUS) ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// libssmscan: C ABI, argument validation, planning and kernel launches.
// The declarations and the contract of every entry point are in include/ssmscan.h.
#include <hip/hip_runtime.h>
#include <algorithm>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "launch.h"

namespace ssmlib {


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

// How long a second half of the split schedule waits for its hand-over, in ticks of the
// 100 MHz constant clock: SSMSCAN_HANDOVER_WAIT_US microseconds (default 20000), read at each
// call.  0 makes every second half compute its whole tile (the time-out path; same results).
unsigned long long handover_wait_ticks() {
    const char *e = getenv("SSMSCAN_HANDOVER_WAIT_US");
    long long us = 20000;
    if (e && *e) {
        char *end = nullptr;
        const long long v = strtoll(e, &end, 10);
        if (end != e && v >= 0 && v <= 10000000) us = v;
    }
    return (unsigned long long)us * 100ull;
}


// The launch templates are instantiated in the inst_*.hip translation units.
#define SSM_EXTERN_N(N, IO) \
    extern template int launch_scan<N, IO>(const void *, const void *, const float *, const void *, const void *, \
                                           const float *, const void *, const float *, int, const float *, void *, \
                                           float *, const ssm_dims *, const Plan &, void *, hipStream_t, \
                                           const ConvArgs *, float *, const int32_t *); \
    extern template int launch_step<N, IO>(float *, const void *, const void *, const float *, const void *, \
                                           const void *, const float *, const void *, void *, const ssm_dims *, \
                                           hipStream_t, const float *, int, int); \
    extern template int launch_bwd<N, IO>(const BwdArgs &, const ssm_dims *, const Plan &, size_t, void *, hipStream_t);
#define SSM_EXTERN_IO(IO) SSM_EXTERN_N(1, IO) SSM_EXTERN_N(2, IO) SSM_EXTERN_N(4, IO) SSM_EXTERN_N(8, IO) \
    SSM_EXTERN_N(16, IO)
SSM_EXTERN_IO(float)
SSM_EXTERN_IO(uint16_t)
#undef SSM_EXTERN_IO
#undef SSM_EXTERN_N
extern template int launch_conv<float>(int, bool, const void *, const float *, const float *, const void *, void *,
                                       void *, const ssm_dims *, hipStream_t);
extern template int launch_conv<uint16_t>(int, bool, const void *, const float *, const float *, const void *,
                                          void *, void *, const ssm_dims *, hipStream_t);
extern template void launch_conv_bwd<float>(int, bool, const void *, const float *, const float *, const void *,
                                            const void *, void *, float *, float *, void *, const ssm_dims *,
                                            hipStream_t);
extern template void launch_conv_bwd<uint16_t>(int, bool, const void *, const float *, const float *,
                                               const void *, const void *, void *, float *, float *, void *,
                                               const ssm_dims *, hipStream_t);

}  // namespace ssmlib

namespace {

using namespace ssmlib;

bool n_supported(int64_t n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 46;
constexpr int kMaxChunks = 65535;  // grid.y limit
// With at most this many chunks per sequence the final pass composes the chunk summaries
// before its chunk itself (a few loads and exponentials per state) instead of a separate
// carry launch; with more, the carry kernel's scan over chunks is cheaper.
constexpr int64_t kFoldMaxChunks = 16;
// Scan workgroups resident per CU (N = 16: 133-137 VGPRs and 48 KB of LDS per 4-wave group),
// the basis of the schedules below.
constexpr int kGroupsPerCU = 3;
// CU count assumed when no device is visible (plan queries on a host without a GPU): MI355X.
constexpr int kDefaultCUs = 256;

// Compute units of the current device, cached per device.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return kDefaultCUs;
    }
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = kDefaultCUs;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

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

// cus: compute units of the device.  allow_split: the split schedule may be used (not when the
// initial state is the last_state buffer: a second part that found no hand-over would rewrite
// last_state while its first part may still read the initial state).
//
// The split schedule (N = 16, library's choice, 2 C < tiles <= 2.5 C for C CUs): with one
// workgroup per tile, tiles = 2.5 C puts 3 tiles on half the CUs and 2 on the rest, and the
// kernel lasts as long as 3.  Splitting 3 C - tiles of the tiles into two token halves (the
// second started from the first's handed-over state) gives 3 C workgroups, three per CU, and
// an equal share of tokens to every CU.
Plan make_plan(const ssm_dims *dm, int cus, bool align_ckpt = false, bool allow_split = true) {
    Plan p;
    const int64_t bsz = dm->batch, L = dm->seqlen, D = dm->dim, N = dm->dstate;
    if (bsz == 0 || L == 0 || D == 0) return p;
    if (cus <= 0) cus = kDefaultCUs;
    const int64_t tiles = bsz * ((D + ssm::kChanTile - 1) / ssm::kChanTile);
    const int64_t target_groups = (int64_t)kGroupsPerCU * cus;
    int64_t clen = L;
    if (dm->chunk_len > 0) {
        p.schedule = kCarry;
        clen = dm->chunk_len < L ? dm->chunk_len : L;
        if ((L + clen - 1) / clen > kMaxChunks) clen = (L + kMaxChunks - 1) / kMaxChunks;
    } else if (dm->chunk_len == 0 && tiles < 2 * (int64_t)cus && L >= 512) {
        // too few channel tiles to fill the GPU: split the tokens too.  At least one round of
        // resident workgroups, and chunks of at most 512 tokens so that long sequences give
        // many items (the grid then balances itself over the CUs); chunks of at least 128
        // tokens keep the per-item start-up and the carry small.  (Short sequences stay one
        // pass: three launches would cost more than they save.)
        const int64_t want = std::max((target_groups + tiles - 1) / tiles, (L + 511) / 512);
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
    if (align_ckpt && p.schedule == kCarry) {
        clen = (clen + ssm::kCkptEvery - 1) / ssm::kCkptEvery * ssm::kCkptEvery;
        if (clen > L) clen = L;
    }
    p.chunk_len = clen;
    p.nchunk = (L + clen - 1) / clen;
    if (p.schedule == kCarry && p.nchunk == 1) p.schedule = kGrid;
    if (p.schedule == kCarry) {
        // (not when the initial state is the last_state buffer: every chunk reads the initial
        // state while the last chunk writes last_state; the carry kernel copies it first)
        p.fold = p.nchunk <= kFoldMaxChunks && allow_split;
        size_t cs = align256((size_t)(bsz * p.nchunk * D * N) * sizeof(float));
        size_t cd = align256((size_t)(bsz * p.nchunk * D) * sizeof(float));
        p.off_cstate = 0;
        p.off_cdsum = cs;
        p.bytes = cs + cd;
    } else if (dm->chunk_len == 0 && allow_split && N == 16 && tiles > 2 * (int64_t)cus &&
               2 * tiles <= 5 * (int64_t)cus && L >= 128) {
        p.schedule = kSplit;
        p.n_split = target_groups - tiles;
        p.n_full = tiles - p.n_split;
        p.l_mid = (L / 2 + 31) / 32 * 32;   // a whole number of 32-token tiles (and of checkpoint spans)
        const size_t hb = align256((size_t)(p.n_split * ssm::kChanTile * N) * sizeof(float));
        const size_t fb = align256((size_t)(p.n_split + p.n_full) * sizeof(int));   // flags, then progress
        p.off_hand = 0;
        p.off_flags = hb;
        p.bytes = hb + fb;
    }
    return p;
}


// Kernel shape per state size: S states per wave (K = N/S waves per workgroup) and T
// tokens per LDS tile.

template <typename IO>
int dispatch_scan(int64_t N, const void *u, const void *delta, const float *A, const void *B,
                  const void *C, const float *Dv, const void *z, const float *bias, int flags, const float *h0,
                  void *y, float *ls, const ssm_dims *dm, const Plan &p, void *ws, hipStream_t st,
                  const ConvArgs *cv, float *ckpt, const int32_t *sl) {
    switch (N) {
        case 1: return launch_scan<1, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt, sl);
        case 2: return launch_scan<2, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt, sl);
        case 4: return launch_scan<4, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt, sl);
        case 8: return launch_scan<8, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt, sl);
        case 16:
            return launch_scan<16, IO>(u, delta, A, B, C, Dv, z, bias, flags, h0, y, ls, dm, p, ws, st, cv, ckpt, sl);
    }
    return fail(SSM_ERR_UNSUPPORTED_N, "dstate %lld not supported", (long long)N);
}

template <typename IO>
int dispatch_step(int64_t N, float *state, const void *u, const void *delta, const float *A, const void *B,
                  const void *C, const float *Dv, const void *z, void *y, const ssm_dims *dm, hipStream_t st,
                  const float *bias, int softplus, int act) {
    switch (N) {
        case 1: return launch_step<1, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st, bias, softplus, act);
        case 2: return launch_step<2, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st, bias, softplus, act);
        case 4: return launch_step<4, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st, bias, softplus, act);
        case 8: return launch_step<8, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st, bias, softplus, act);
        case 16: return launch_step<16, IO>(state, u, delta, A, B, C, Dv, z, y, dm, st, bias, softplus, act);
    }
    return fail(SSM_ERR_UNSUPPORTED_N, "dstate %lld not supported", (long long)N);
}

// The backward's checkpoint pass runs under the split schedule where the forward would (its
// chunk length setting aside); any other plan is the one-pass grid.
Plan bwd_ckpt_plan(const ssm_dims *dm) {
    ssm_dims d = *dm;
    d.chunk_len = 0;
    Plan p = make_plan(&d, device_cus());
    return p.schedule == kSplit ? p : Plan{};
}

size_t ckpt_bytes(const ssm_dims *dm) {
    const int64_t n_ckpt = (dm->seqlen + ssm::kCkptEvery - 1) / ssm::kCkptEvery;
    return align256((size_t)(dm->batch * n_ckpt * dm->dim * dm->dstate) * sizeof(float));
}

// the checkpoints, then the split schedule's scratch (hand-over states and the checkpoint
// pass's flags), then the reverse walk's flags
size_t bwd_workspace_bytes(const ssm_dims *dm) {
    const Plan p = bwd_ckpt_plan(dm);
    return ckpt_bytes(dm) + p.bytes + (p.schedule == kSplit ? align256((size_t)(p.n_split + p.n_full) * sizeof(int)) : 0);
}

template <typename IO>
int dispatch_bwd(int64_t N, const BwdArgs &a, const ssm_dims *dm, void *ws, hipStream_t st) {
    const Plan sp = bwd_ckpt_plan(dm);
    const size_t cb = ckpt_bytes(dm);
    switch (N) {
        case 1: return launch_bwd<1, IO>(a, dm, sp, cb, ws, st);
        case 2: return launch_bwd<2, IO>(a, dm, sp, cb, ws, st);
        case 4: return launch_bwd<4, IO>(a, dm, sp, cb, ws, st);
        case 8: return launch_bwd<8, IO>(a, dm, sp, cb, ws, st);
        case 16: return launch_bwd<16, IO>(a, dm, sp, cb, ws, st);
    }
    return fail(SSM_ERR_UNSUPPORTED_N, "dstate %lld not supported", (long long)N);
}

// The backward's entry (ssm_scan_bwd and ssm_scan_bwd_varlen): validation, zeroing, launches.
int bwd_impl(const float *initial_state, const int32_t *seq_lens, const void *u, const void *delta, const float *A,
             const void *B, const void *C, const float *D, const void *z, const float *delta_bias, int flags,
             const void *dy, const float *dlast_state, void *du, void *ddelta, float *dA, float *dB, float *dC,
             float *dD, void *dz, float *ddelta_bias, float *dinitial_state, const ssm_dims *dims, void *workspace,
             size_t workspace_bytes, void *stream);
// The step's entry (ssm_step and ssm_step_act).
int step_impl(float *state, const void *u, const void *delta, const float *A, const void *B, const void *C,
              const float *D, const void *z, const float *delta_bias, int flags, void *y, const ssm_dims *dims,
              void *stream, bool act);

}  // namespace

// ---- scratch for the entry point that allocates nothing ------------------------------------

// Device scratch of ssm_scan_fwd_noalloc: the carry's chunk states or the split schedule's
// handed-over states, in the code object itself, one copy per device (held until the process
// ends).  64 MiB covers the chunk carry of B1 L131072 D2048 N16 (35.7 MB).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The current device's copy of `scratch` (its device address, looked up once per device with
// that device current).  In host code the name `scratch` is only a host-side stand-in; kernels
// get this address.  Returns nullptr (message set) if the lookup fails.
void *scratch_address() {
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        fail(SSM_ERR_HIP, "no current device for the library's scratch");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

static int scan_impl(const float *h0, const void *u, const void *delta, const float *A, const void *B,
                     const void *C, const float *D, const void *z, const float *delta_bias, int flags,
                     void *y, float *last_state, const ssm_dims *dims, void *workspace, size_t workspace_bytes,
                     void *stream, const ConvArgs *cv = nullptr, const int32_t *seq_lens = nullptr) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    if (flags & ~(SSM_SCAN_SOFTPLUS | SSM_SCAN_EXACT_ZOH | SSM_SCAN_CHECKPOINTS))
        return fail(SSM_ERR_FLAGS, "unknown flag bits 0x%x", flags);
    const bool want_ckpt = (flags & SSM_SCAN_CHECKPOINTS) != 0;
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
    // (the split schedule is not used when the initial state is the last_state buffer)
    Plan p = make_plan(dims, device_cus(), want_ckpt, !(h0 && h0 == last_state));
    // with checkpoints the workspace holds them first (the backward pass's layout), then the plan's carry area
    const size_t ck_bytes = want_ckpt ? bwd_workspace_bytes(dims) : 0, need = ck_bytes + p.bytes;
    if (need > 0 && !workspace) return fail(SSM_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                    need);
    if (need > 0 && !aligned(workspace, 16)) return fail(SSM_ERR_ALIGN, "workspace not 16-byte aligned");
    float *ckpt = want_ckpt ? static_cast<float *>(workspace) : nullptr;
    void *carry_ws = p.bytes > 0 ? static_cast<void *>(static_cast<char *>(workspace) + ck_bytes) : workspace;
    if (seq_lens && !aligned(seq_lens, 4)) return fail(SSM_ERR_ALIGN, "seq_lens not 4-byte aligned");
    if (dims->io_dtype == SSM_IO_BF16)
        return dispatch_scan<uint16_t>(N, u, delta, A, B, C, D, z, delta_bias, flags, h0, y, last_state, dims, p,
                                       carry_ws, st, cv, ckpt, seq_lens);
    return dispatch_scan<float>(N, u, delta, A, B, C, D, z, delta_bias, flags, h0, y, last_state, dims, p,
                                carry_ws, st, cv, ckpt, seq_lens);
}


extern "C" {

int ssm_version(void) { return SSMSCAN_VERSION; }

const char *ssm_last_error(void) { return g_err.c_str(); }

size_t ssm_scan_workspace_bytes(const ssm_dims *dims) {
    if (check_dims(dims, true) != SSM_OK) return 0;
    return make_plan(dims, device_cus()).bytes;
}

int64_t ssm_scan_plan(const ssm_dims *dims, int64_t *chunk_len_out) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    Plan p = make_plan(dims, device_cus());
    if (chunk_len_out) *chunk_len_out = p.chunk_len;
    ok();
    return p.schedule == kCarry ? p.nchunk : 1;
}

int ssm_scan_plan_info(const ssm_dims *dims, int cu_count, ssm_plan_info *out) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    if (!out) return fail(SSM_ERR_NULL, "out is NULL");
    const int cus = cu_count > 0 ? cu_count : device_cus();
    Plan p = make_plan(dims, cus);
    out->cu_count = cus;
    out->nchunk = p.schedule == kCarry ? p.nchunk : 1;
    out->chunk_len = p.chunk_len;
    out->split_tiles = p.n_split;
    out->split_at = p.l_mid;
    out->workgroups = p.schedule == kSplit ? p.n_full + 2 * p.n_split
                      : (int64_t)dims->batch * ((dims->dim + ssm::kChanTile - 1) / ssm::kChanTile) * out->nchunk;
    out->workspace_bytes = p.bytes;
    return ok();
}

int ssm_scan_fwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int flags,
                 void *y, float *last_state, const ssm_dims *dims,
                 void *workspace, size_t workspace_bytes, void *stream) {
    return scan_impl(nullptr, u, delta, A, B, C, D, z, delta_bias, flags, y, last_state, dims, workspace,
                     workspace_bytes, stream);
}

int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A, const void *B, const void *C,
                         const float *D, const void *z, const float *delta_bias, int flags, void *y,
                         float *last_state, const ssm_dims *dims, void *stream) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    if (flags & SSM_SCAN_CHECKPOINTS)
        return fail(SSM_ERR_FLAGS, "the checkpoints outlive the call: use ssm_scan_fwd with a workspace");
    const size_t need = make_plan(dims, device_cus()).bytes;
    if (need > kNoAllocScratchBytes)
        return fail(SSM_ERR_WORKSPACE,
                    "this plan needs %zu bytes of scratch, more than the %zu the library holds per device; "
                    "use ssm_scan_fwd with a workspace", need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need > 0 && !(ws = scratch_address())) return SSM_ERR_HIP;
    return scan_impl(nullptr, u, delta, A, B, C, D, z, delta_bias, flags, y, last_state, dims, ws,
                     need > 0 ? kNoAllocScratchBytes : 0, stream);
}

int ssm_scan_fwd_from(const float *initial_state, const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z, const float *delta_bias,
                      int flags, void *y, float *last_state, const ssm_dims *dims, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return scan_impl(initial_state, u, delta, A, B, C, D, z, delta_bias, flags, y, last_state, dims,
                     workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_varlen(const float *initial_state, const int32_t *seq_lens, const void *u, const void *delta,
                        const float *A, const void *B, const void *C, const float *D, const void *z,
                        const float *delta_bias, int flags, void *y, float *last_state, const ssm_dims *dims,
                        void *workspace, size_t workspace_bytes, void *stream) {
    if (!seq_lens) return fail(SSM_ERR_NULL, "seq_lens is NULL (use ssm_scan_fwd_from for equal lengths)");
    return scan_impl(initial_state, u, delta, A, B, C, D, z, delta_bias, flags, y, last_state, dims, workspace,
                     workspace_bytes, stream, nullptr, seq_lens);
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
    return step_impl(state, u, delta, A, B, C, D, z, nullptr, 0, y, dims, stream, false);
}

int ssm_step_act(float *state, const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int flags, void *y, const ssm_dims *dims,
                 void *stream) {
    return step_impl(state, u, delta, A, B, C, D, z, delta_bias, flags, y, dims, stream, true);
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
    return bwd_impl(initial_state, nullptr, u, delta, A, B, C, D, z, delta_bias, flags, dy, dlast_state, du, ddelta,
                    dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, dims, workspace, workspace_bytes, stream);
}

int ssm_scan_bwd_varlen(const float *initial_state, const int32_t *seq_lens, const void *u, const void *delta,
                        const float *A, const void *B, const void *C, const float *D, const void *z,
                        const float *delta_bias, int flags, const void *dy, const float *dlast_state, void *du,
                        void *ddelta, float *dA, float *dB, float *dC, float *dD, void *dz, float *ddelta_bias,
                        float *dinitial_state, const ssm_dims *dims, void *workspace, size_t workspace_bytes,
                        void *stream) {
    if (!seq_lens) return fail(SSM_ERR_NULL, "seq_lens is NULL (use ssm_scan_bwd for equal lengths)");
    if (!aligned(seq_lens, 4)) return fail(SSM_ERR_ALIGN, "seq_lens not 4-byte aligned");
    return bwd_impl(initial_state, seq_lens, u, delta, A, B, C, D, z, delta_bias, flags, dy, dlast_state, du, ddelta,
                    dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, dims, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// ssm_step (activated step size, act = false) and ssm_step_act (the raw input with the scan's
// activation flags).
int step_impl(float *state, const void *u, const void *delta, const float *A, const void *B, const void *C,
              const float *D, const void *z, const float *delta_bias, int flags, void *y, const ssm_dims *dims,
              void *stream, bool act) {
    int rc = check_dims(dims, false);
    if (rc != SSM_OK) return rc;
    if (flags & ~(SSM_SCAN_SOFTPLUS | SSM_SCAN_EXACT_ZOH))
        return fail(SSM_ERR_FLAGS, "flags 0x%x: a step takes SSM_SCAN_SOFTPLUS and SSM_SCAN_EXACT_ZOH only", flags);
    const int64_t S = dims->batch, Dm = dims->dim, N = dims->dstate;
    if (S == 0 || Dm == 0) return ok();
    if (!state || !u || !delta || !A || !B || !C || !y)
        return fail(SSM_ERR_NULL, "required pointer is NULL (state=%p u=%p delta=%p A=%p B=%p C=%p y=%p)",
                    (void *)state, u, delta, (const void *)A, B, C, y);
    const size_t es = dims->io_dtype == SSM_IO_BF16 ? 2 : 4;
    if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(y, es) ||
        (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) || (delta_bias && !aligned(delta_bias, 4)) ||
        !aligned(state, N >= 4 ? 16 : 4))
        return fail(SSM_ERR_ALIGN, "a tensor pointer is not aligned (state needs 16 bytes when dstate >= 4)");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int mode = !act ? 0 : (flags & SSM_SCAN_EXACT_ZOH) ? 2 : 1;
    const int softplus = (flags & SSM_SCAN_SOFTPLUS) ? 1 : 0;
    if (dims->io_dtype == SSM_IO_BF16)
        return dispatch_step<uint16_t>(N, state, u, delta, A, B, C, D, z, y, dims, st, delta_bias, softplus, mode);
    return dispatch_step<float>(N, state, u, delta, A, B, C, D, z, y, dims, st, delta_bias, softplus, mode);
}

int bwd_impl(const float *initial_state, const int32_t *seq_lens, const void *u, const void *delta, const float *A,
             const void *B, const void *C, const float *D, const void *z, const float *delta_bias, int flags,
             const void *dy, const float *dlast_state, void *du, void *ddelta, float *dA, float *dB, float *dC,
             float *dD, void *dz, float *ddelta_bias, float *dinitial_state, const ssm_dims *dims, void *workspace,
             size_t workspace_bytes, void *stream) {
    int rc = check_dims(dims, true);
    if (rc != SSM_OK) return rc;
    if (flags & ~(SSM_SCAN_SOFTPLUS | SSM_SCAN_EXACT_ZOH | SSM_SCAN_CHECKPOINTS))
        return fail(SSM_ERR_FLAGS, "unknown flag bits 0x%x", flags);
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
    // the summed gradients are accumulated atomically: they start from zero (one fill launch,
    // with the split schedule's flags when the walk runs)
    ssm::FillList zero{};
    fill_list_add(zero, dA, Dm * N);
    fill_list_add(zero, dB, bsz * L * N);
    fill_list_add(zero, dC, bsz * L * N);
    fill_list_add(zero, dD, Dm);
    fill_list_add(zero, ddelta_bias, Dm);
    if (bsz == 0 || Dm == 0 || L == 0) launch_fill_list(zero, st);
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
              dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, (flags & SSM_SCAN_CHECKPOINTS) != 0,
              (flags & SSM_SCAN_EXACT_ZOH) != 0, zero, seq_lens};
    if (dims->io_dtype == SSM_IO_BF16) return dispatch_bwd<uint16_t>(N, a, dims, workspace, st);
    return dispatch_bwd<float>(N, a, dims, workspace, st);
}

}  // namespace

extern "C" {

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
    return ssm_ssd_fwd_from(nullptr, x, dt, A, B, C, D, z, dt_bias, flags, y, last_state, dims, stream);
}

int ssm_ssd_fwd_from(const float *initial_state, const void *x, const void *dt, const float *A, const void *B,
                     const void *C, const float *D, const void *z, const float *dt_bias, int flags, void *y,
                     float *last_state, const ssm_ssd_dims *dims, void *stream) {
    if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
    const int64_t bsz = dims->batch, L = dims->seqlen, H = dims->nheads, P = dims->headdim, G = dims->ngroups,
                  N = dims->dstate;
    if (bsz < 0 || L < 0 || H < 0 || P < 0 || G < 1 || N < 0)
        return fail(SSM_ERR_SHAPE, "negative size or ngroups < 1");
    if (dims->io_dtype != SSM_IO_BF16 && dims->io_dtype != SSM_IO_F32)
        return fail(SSM_ERR_DTYPE, "io_dtype %d is not SSM_IO_F32 (0) or SSM_IO_BF16 (1)", dims->io_dtype);
    const bool f32 = dims->io_dtype == SSM_IO_F32;
    if (!(P == 32 || (P >= 64 && P % 64 == 0)) || !(N == 32 || N == 64 || N == 128) || (N == 128 && P == 32))
        return fail(SSM_ERR_SHAPE,
                    "headdim %lld and dstate %lld: the SSD kernel supports headdim 32 or a multiple of 64 and dstate "
                    "32, 64 or 128 (dstate 128 with headdim a multiple of 64)", (long long)P, (long long)N);
    if (f32 && N == 128) return fail(SSM_ERR_SHAPE, "dstate 128 takes bf16 I/O (fp32 I/O: dstate 32 or 64)");
    if (H % G != 0) return fail(SSM_ERR_SHAPE, "nheads %lld is not a multiple of ngroups %lld", (long long)H,
                                (long long)G);
    if (H > kMaxDim || bsz > kMaxDim || (bsz > 0 && H * (P > 64 ? P / 64 : 1) > (int64_t(1) << 31) / bsz))
        return fail(SSM_ERR_SHAPE, "batch*nheads*(headdim/64) exceeds 2^31 (grid size)");
    if (bsz > 0 && H > 0 && L > kMaxElems / bsz / H / P) return fail(SSM_ERR_SHAPE, "too many elements");
    if (H * P > (int64_t(1) << 24))   // a chunk's rows are addressed with 32-bit offsets
        return fail(SSM_ERR_SHAPE, "nheads*headdim %lld exceeds 2^24", (long long)(H * P));
    if (flags & ~SSM_SCAN_SOFTPLUS) return fail(SSM_ERR_FLAGS, "flags 0x%x: the SSD layer takes the softplus flag only",
                                                flags);
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(z, 16) ||
        !aligned(dt, f32 ? 4 : 2) || !aligned(A, 4) || !aligned(D, 4) || !aligned(dt_bias, 4) || !aligned(last_state, 4) ||
        !aligned(initial_state, 4))
        return fail(SSM_ERR_ALIGN, "x, z, y, B, C must be 16-byte aligned and the others aligned to their element size");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (bsz == 0 || H == 0) return ok();
    if (!A || (L > 0 && (!x || !dt || !B || !C || !y))) return fail(SSM_ERR_NULL, "required pointer is NULL");
    if (L == 0) {
        // no tokens: the final state is the initial one
        const int64_t n = bsz * H * P * N;
        if (last_state && initial_state && initial_state != last_state)
            hipLaunchKernelGGL(ssm::copy_kernel<float>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, last_state,
                               initial_state, n);
        else if (last_state && !initial_state)
            fill_zero(last_state, n, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    launch_ssd(x, dt, A, B, C, D, z, dt_bias, (flags & SSM_SCAN_SOFTPLUS) ? 1 : 0, y, last_state, bsz, L, H, G, st,
               initial_state, P, N, f32);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

/*
 * libssmscan -- the Mamba selective state-space scan (S6) and its single-token
 * recurrent step on AMD MI355X (gfx950).
 *
 * What is computed (per channel d of sequence b, state index n):
 *   step size       dt_t   = softplus(delta_t + delta_bias[d])   with SSM_SCAN_SOFTPLUS
 *                          = delta_t + delta_bias[d]             otherwise
 *     (azimuth.plus/paper/mamba, "selection" section: delta_t = softplus(Linear(x_t)))
 *   discretisation  dA     = exp(dt_t * A[d,n])     (ZOH of a diagonal A;
 *                                                    yapayzekasozluk.tr, "Temel Matematiksel Cerceve")
 *                   input  = dt_t * B_t[n] * u_t    (simplified input matrix; the pages give no formula)
 *                   or, with SSM_SCAN_EXACT_ZOH, the zero-order hold of the same diagonal
 *                   system, (exp(dt_t A[d,n]) - 1) / A[d,n] * B_t[n] * u_t (dt_t B_t[n] u_t
 *                   where A = 0), under which Theorem 1 of azimuth.plus/paper/mamba (the
 *                   gated recurrence) holds exactly
 *   recurrence      h_t[n] = dA * h_{t-1}[n] + input
 *     (azimuth.plus/paper/mamba, hardware-aware algorithm section, parallel-scan bullet)
 *   readout         y_t    = (sum_n C_t[n] h_t[n] + D[d] u_t) * silu(z_t)
 *     (y = C h + D x: yapayzekasozluk.tr, same section; the SiLU gate branch multiplies
 *      the SSM branch: azimuth.plus/paper/mamba, block architecture section)
 * B_t and C_t are one N-vector per (sequence, token), shared by all channels; A is
 * fixed (one real value per channel and state).  The scan starts from h = 0.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory), row-major,
 *    densely packed, innermost index last.  Elements must be naturally aligned; bf16 B
 *    and C must also be 4-byte aligned when dstate >= 2 (they are read as 32-bit words).
 *  - The "I/O" tensors u, delta, z, y, B, C have the element type dims->io_dtype
 *    (SSM_IO_F32 = IEEE fp32, SSM_IO_BF16 = bfloat16 bit patterns).  A, D, delta_bias,
 *    last_state and state are always fp32.  Arithmetic and the state are fp32.
 *  - Outputs must not alias inputs (except ssm_step's state, updated in place).
 *  - The caller owns every buffer.  The library allocates and frees nothing, does not
 *    synchronise, and keeps no pointer after a call returns.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and runs asynchronously.
 *  - Every argument is validated before anything is enqueued.  A negative status means
 *    nothing was launched; ssm_last_error() then describes the problem.  Faults inside
 *    kernels surface at the caller's next synchronisation.
 *  - Supported state sizes: N in {1, 2, 4, 8, 16}.
 *  - Sizes of zero are valid: nothing is computed (a scan of L = 0 tokens writes a zero
 *    last_state when one is asked for).
 */
#ifndef SSMSCAN_H
#define SSMSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSMSCAN_VERSION 15

/* Bits of the `flags` argument of the scan entry points. */
#define SSM_SCAN_SOFTPLUS 1     /* step size = softplus(delta + delta_bias) */
#define SSM_SCAN_EXACT_ZOH 2    /* exact zero-order-hold input term */
#define SSM_SCAN_CHECKPOINTS 4  /* forward: also store the backward pass's checkpoints in the
                                   workspace; backward: the workspace already holds them */

#if defined(__GNUC__) || defined(__clang__)
#define SSMSCAN_API __attribute__((visibility("default")))
#else
#define SSMSCAN_API
#endif

typedef enum {
    SSM_IO_F32 = 0,
    SSM_IO_BF16 = 1
} ssm_io_dtype;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL = -1,            /* a required pointer is NULL */
    SSM_ERR_SHAPE = -2,           /* a size is negative or too large */
    SSM_ERR_DTYPE = -3,           /* io_dtype is not an ssm_io_dtype */
    SSM_ERR_ALIGN = -4,           /* a pointer is not aligned to its element size */
    SSM_ERR_UNSUPPORTED_N = -5,   /* dstate is not 1, 2, 4, 8 or 16 */
    SSM_ERR_WORKSPACE = -6,       /* workspace missing or smaller than required */
    SSM_ERR_HIP = -7,             /* the HIP runtime refused a launch */
    SSM_ERR_FLAGS = -8            /* unknown flag bits, or a flag the entry point does not take */
} ssm_status;

/* Problem sizes.
 *   batch     sequences in the batch (ssm_step: number of independent sequences S)
 *   seqlen    tokens per sequence L (ignored by ssm_step)
 *   dim       channels D
 *   dstate    state size N
 *   io_dtype  an ssm_io_dtype
 *   chunk_len scan plan: 0 = the library chooses; > 0 = split every sequence into
 *             chunks of this many tokens and combine the chunk states (two-pass chunk
 *             carry); -1 = one pass, one workgroup per 64 channels of a sequence.  With 0
 *             the library runs one pass when there are enough channel tiles to fill the
 *             GPU (with dstate 16 and 2 to 2.5 tiles per CU, the split schedule of
 *             ssm_scan_plan_info: bitwise the one pass's results) and the chunk carry
 *             otherwise.  Results agree up to fp32 rounding whatever the plan. */
typedef struct ssm_dims {
    int64_t batch;
    int64_t seqlen;
    int64_t dim;
    int64_t dstate;
    int32_t io_dtype;
    int32_t chunk_len;
} ssm_dims;

/* Bytes of device workspace ssm_scan_fwd needs for these sizes and plan on the current device
 * (256-byte aligned regions): the per-chunk carry states of a chunked plan, the handed-over
 * states, flags and progress counters of the split schedule (see ssm_scan_plan_info; the
 * library clears the flags and counters itself on every call), 0 for a plain single
 * pass.  Returns 0 for an invalid or empty problem. */
SSMSCAN_API size_t ssm_scan_workspace_bytes(const ssm_dims *dims);

/* The plan ssm_scan_fwd will use.  Returns the number of chunks each sequence is split
 * into for the chunk carry (1 = a single pass: every token's state is computed once) and
 * stores in *chunk_len_out (may be NULL) the tokens per work item: the carry chunk length,
 * or the whole sequence for a single pass.  Returns a negative ssm_status for invalid
 * sizes. */
SSMSCAN_API int64_t ssm_scan_plan(const ssm_dims *dims, int64_t *chunk_len_out);

/* The schedule the scan takes on a device with cu_count compute units (cu_count <= 0: the
 * current device; 256 when no device is visible).  The library plans from the device's CU
 * count: one workgroup of four waves per (sequence, 64-channel tile) in one pass; the chunk
 * carry when there are fewer than 2 tiles per CU and sequences of 512 tokens or more; and, for
 * dstate 16 with 2 to 2.5 tiles per CU, the split schedule: split_tiles of the tiles are run
 * as two token halves (the second from the state the first hands over through the workspace,
 * starting at token split_at), so that every CU gets the same number of tokens.  The results
 * are bitwise those of the one-pass schedule (dims->chunk_len = -1).  Fills *out; returns
 * SSM_OK or a negative ssm_status. */
typedef struct ssm_plan_info {
    int32_t cu_count;       /* the CU count the plan was made for */
    int64_t nchunk;         /* carry chunks per sequence (1: no carry) */
    int64_t chunk_len;      /* tokens per carry chunk (seqlen without the carry) */
    int64_t split_tiles;    /* tiles run as two token halves (0: not the split schedule) */
    int64_t split_at;       /* first token of the second halves */
    int64_t workgroups;     /* workgroups of the scan's main launch */
    size_t workspace_bytes; /* = ssm_scan_workspace_bytes on that device */
} ssm_plan_info;
SSMSCAN_API int ssm_scan_plan_info(const ssm_dims *dims, int cu_count, ssm_plan_info *out);

/* Selective scan forward over a batch of sequences, from a zero state.
 *   u, delta, z, y : [batch][seqlen][dim]   (io_dtype; z may be NULL = no gate)
 *   B, C           : [batch][seqlen][dstate] (io_dtype)
 *   A              : [dim][dstate] fp32
 *   D, delta_bias  : [dim] fp32, each may be NULL (= 0)
 *   flags          : SSM_SCAN_SOFTPLUS (apply softplus to delta + delta_bias),
 *                    SSM_SCAN_EXACT_ZOH (exact zero-order-hold input term) and
 *                    SSM_SCAN_CHECKPOINTS (see workspace); other bits are rejected with
 *                    SSM_ERR_FLAGS
 *   y              : output, written completely
 *   last_state     : [batch][dim][dstate] fp32 output h_L, may be NULL
 *   workspace      : device memory of at least ssm_scan_workspace_bytes(dims) bytes, 16-byte
 *                    aligned (contents on entry do not matter; scratch for this call: the
 *                    carry's chunk states, or the split schedule's handed-over states and
 *                    flags); may be NULL when that size is 0.  With SSM_SCAN_CHECKPOINTS (a training
 *                    forward) it must hold ssm_scan_bwd_workspace_bytes(dims) +
 *                    ssm_scan_workspace_bytes(dims) bytes, and the call leaves at its start
 *                    (batch * ceil(seqlen / 8) * dim * dstate fp32) the states ssm_scan_bwd
 *                    would otherwise recompute in a pass of its own: pass the same workspace and
 *                    flag to ssm_scan_bwd.  The checkpoints are the states before every 8th
 *                    token, so with this flag a chunked plan's chunk length (dims->chunk_len
 *                    > 0, or the library's choice) is rounded up to a multiple of 8
 * Returns SSM_OK or a negative ssm_status. */
SSMSCAN_API int ssm_scan_fwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int flags,
                 void *y, float *last_state, const ssm_dims *dims,
                 void *workspace, size_t workspace_bytes, void *stream);

/* ssm_scan_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same scan, arguments and results
 * (bitwise those of ssm_scan_fwd on the same plan), with no workspace argument.  Its scratch
 * (the carry's chunk states or the split schedule's handed-over states) is an array of
 * 64 MiB inside the library's code object, one copy per device, held until the process ends.
 * The call allocates and frees nothing.
 *   flags : SSM_SCAN_SOFTPLUS and SSM_SCAN_EXACT_ZOH; SSM_SCAN_CHECKPOINTS is rejected with
 *           SSM_ERR_FLAGS (the checkpoints must outlive the call: use ssm_scan_fwd)
 * A plan whose scratch exceeds 64 MiB (ssm_scan_workspace_bytes) returns SSM_ERR_WORKSPACE
 * before anything is launched.  All calls on one device share its scratch: calls that overlap
 * in time on one device (different streams or host threads) race and must not be issued;
 * calls in one stream are ordered and safe.  Returns SSM_OK or a negative ssm_status. */
SSMSCAN_API int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A, const void *B,
                                     const void *C, const float *D, const void *z, const float *delta_bias,
                                     int flags, void *y, float *last_state, const ssm_dims *dims, void *stream);

/* The same scan continued from a given state: h_0 = initial_state instead of zero.  The
 * recurrent form carries the whole history in the state (shakilmahmud.com section 3;
 * urworte.de "Methodische Grundlagen"), so scanning a sequence in pieces, each from the
 * last_state of the previous piece, gives the scan of the whole sequence (up to fp32
 * rounding); this is how a prompt is prefilled in pieces or a decode state is rebuilt.
 *   initial_state  : [batch][dim][dstate] fp32, or NULL (= zero: exactly ssm_scan_fwd).
 *                    It may be the same buffer as last_state (the state advanced in place);
 *                    it must not overlap any other argument.
 * All other arguments, the workspace size and the errors are those of ssm_scan_fwd.  With
 * seqlen 0, last_state receives a copy of the initial state. */
SSMSCAN_API int ssm_scan_fwd_from(const float *initial_state, const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z, const float *delta_bias,
                      int flags, void *y, float *last_state, const ssm_dims *dims, void *workspace,
                      size_t workspace_bytes, void *stream);

/* The scan of a batch of sequences of different lengths, continued from a given state: the
 * recurrent form runs one token at a time over each sequence's own tokens only
 * (shakilmahmud.com section 3), so a batch padded to seqlen tokens is scanned sequence by
 * sequence up to its length, as separate calls of ssm_scan_fwd_from would.
 *   seq_lens       : [batch] int32 in device memory, 4-byte aligned: sequence b has
 *                    seq_lens[b] tokens (values outside [0, seqlen] are taken as 0 or
 *                    seqlen; they are read on the device, so the host never synchronises)
 *   y              : tokens t < seq_lens[b] are written; later tokens of y are left untouched
 *                    (no input past a sequence's length is read either)
 *   last_state     : the state after seq_lens[b] tokens (the initial state for length 0)
 * All other arguments (dims->seqlen is the padded length), the workspace size, the plans and
 * the errors are those of ssm_scan_fwd_from; seq_lens NULL returns SSM_ERR_NULL. */
SSMSCAN_API int ssm_scan_fwd_varlen(const float *initial_state, const int32_t *seq_lens, const void *u,
                                    const void *delta, const float *A, const void *B, const void *C,
                                    const float *D, const void *z, const float *delta_bias, int flags, void *y,
                                    float *last_state, const ssm_dims *dims, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Bytes of device workspace ssm_scan_bwd needs: the checkpointed states, one per 8
 * tokens (batch * ceil(seqlen / 8) * dim * dstate fp32, 256-byte aligned), followed, for
 * shapes the library runs under the split schedule (see ssm_plan_info), by that schedule's
 * hand-over scratch (states, flags and progress counters of the checkpoint pass and of the
 * reverse walk).
 * Depends on the current device's CU count.
 * Returns 0 for an invalid or empty problem. */
SSMSCAN_API size_t ssm_scan_bwd_workspace_bytes(const ssm_dims *dims);

/* Gradients of ssm_scan_fwd_from (and so of ssm_scan_fwd, initial_state NULL) with respect
 * to every input, given dy = dLoss/dy and dlast_state = dLoss/d(last_state): the backward
 * pass, recomputing the states from checkpoints instead of storing them
 * (azimuth.plus/paper/mamba, hardware-aware algorithm section).
 *   inputs          : exactly those of the forward call (same shapes, dtypes, NULLs);
 *                     flags may hold SSM_SCAN_SOFTPLUS, SSM_SCAN_EXACT_ZOH (the gradients
 *                     of the exact zero-order-hold scan; with SSM_SCAN_CHECKPOINTS the
 *                     forward call must have had it too) and SSM_SCAN_CHECKPOINTS
 *   dy              : [batch][seqlen][dim] (io_dtype)
 *   dlast_state     : [batch][dim][dstate] fp32, or NULL (= 0)
 *   du, ddelta      : [batch][seqlen][dim] (io_dtype) outputs; ddelta is the gradient with
 *                     respect to the delta input (through delta_bias and softplus)
 *   dz              : [batch][seqlen][dim] (io_dtype) output, required when z is given
 *   dA              : [dim][dstate] fp32 output
 *   dB, dC          : [batch][seqlen][dstate] fp32 outputs (summed over channels)
 *   dD, ddelta_bias : [dim] fp32 outputs, or NULL (not wanted)
 *   dinitial_state  : [batch][dim][dstate] fp32 output, or NULL (not wanted)
 *   workspace       : at least ssm_scan_bwd_workspace_bytes(dims) bytes, 16-byte aligned;
 *                     with SSM_SCAN_CHECKPOINTS it must hold the checkpoints a forward call
 *                     with that flag stored there (same inputs, initial state and dims;
 *                     not checked), and the checkpoint pass is skipped
 * dims->chunk_len is ignored.  dA, dB, dC, dD and ddelta_bias are sums over many
 * workgroups, accumulated with atomic adds after the library has zeroed them: their last
 * bits may differ from run to run.  Outputs must not overlap inputs or each other.
 * Returns SSM_OK or a negative ssm_status (validation before any launch). */
SSMSCAN_API int ssm_scan_bwd(const float *initial_state, const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *z, const float *delta_bias,
                 int flags, const void *dy, const float *dlast_state, void *du, void *ddelta,
                 float *dA, float *dB, float *dC, float *dD, void *dz, float *ddelta_bias,
                 float *dinitial_state, const ssm_dims *dims, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Gradients of ssm_scan_fwd_varlen (sequences of different lengths in one batch): sequence b's
 * gradients are those of the scan of its first seq_lens[b] tokens (clamped to [0, L]), with
 * dlast_state[b] applied to the state after that many tokens (shakilmahmud.com section 3,
 * recurrent form).
 *   seq_lens : [batch] int32 device array (4-byte aligned), the lengths the forward used
 *   du, ddelta, dz : written for every token; zero past each sequence's length (those inputs
 *                    reach no output), whatever dy holds there
 *   dB, dC   : zero past each length; dA, dD, ddelta_bias : sums over the real tokens only
 *   dinitial_state : dlast_state[b] itself for a length of 0
 * Everything else (flags, checkpoints from a training forward_varlen with
 * SSM_SCAN_CHECKPOINTS, workspace) as ssm_scan_bwd.  Returns SSM_OK or a negative ssm_status. */
SSMSCAN_API int ssm_scan_bwd_varlen(const float *initial_state, const int32_t *seq_lens, const void *u,
                const void *delta, const float *A, const void *B, const void *C, const float *D, const void *z,
                const float *delta_bias, int flags, const void *dy, const float *dlast_state, void *du,
                void *ddelta, float *dA, float *dB, float *dC, float *dD, void *dz, float *ddelta_bias,
                float *dinitial_state, const ssm_dims *dims, void *workspace, size_t workspace_bytes,
                void *stream);

/* Bits of the `flags` argument of ssm_conv1d_fwd. */
#define SSM_CONV_SILU 1         /* apply SiLU to the convolution's output */

/* The causal depthwise convolution over time that feeds the scan in the block's main
 * branch, with SiLU: a short 1-D convolution of kernel size 4, then SiLU, before the
 * selective SSM (azimuth.plus/paper/mamba, block architecture section).
 *   out[b,t,d] = silu(bias[d] + sum_{k < width} w[d,k] * x[b, t - (width-1) + k, d])
 * (without SSM_CONV_SILU the pre-activation itself).
 *   x, out       : [batch][seqlen][dim] (io_dtype)
 *   w            : [dim][width] fp32; width 1 to 4 (the pages' kernel size is 4)
 *   bias         : [dim] fp32, or NULL (= 0)
 *   state_in     : [batch][width-1][dim] (io_dtype), the width-1 inputs before token 0,
 *                  oldest first, or NULL (= zeros: the start of a sequence)
 *   state_out    : [batch][width-1][dim] (io_dtype), receives the last width-1 inputs of
 *                  (state_in, x) -- the state that continues the sequence -- or NULL.  It may
 *                  be the state_in buffer (advanced in place; then one thread per channel group
 *                  walks the whole sequence, so use it for short calls such as a decode step);
 *                  it must not overlap any other argument.
 * dims->dstate and dims->chunk_len are ignored.  With seqlen 0, state_out receives state_in
 * (zeros without it).  Running a sequence in pieces, each from the previous piece's
 * state_out, gives the run over the whole sequence bitwise.  Unknown flag bits return
 * SSM_ERR_FLAGS; a width outside 1..4 returns SSM_ERR_SHAPE. */
SSMSCAN_API int ssm_conv1d_fwd(const void *x, const float *w, const float *bias, int width, const void *state_in,
                   int flags, void *out, void *state_out, const ssm_dims *dims, void *stream);

/* Gradients of ssm_conv1d_fwd given dout = dLoss/dout: the backward pass of the block's
 * convolution + SiLU (azimuth.plus/paper/mamba, block architecture section, for the forward;
 * the backward is its exact derivative).  With g[t] = dout[t] * silu'(pre[t]) (dout[t]
 * without SSM_CONV_SILU) and H = width - 1:
 *   dx[b,t,d]      = sum_k w[d,k] * g[b, t + H - k, d]      (g = 0 past the sequence's end)
 *   dw[d,k]        = sum over b, t of g[b,t,d] * x[b, t - H + k, d]
 *   dbias[d]       = sum over b, t of g[b,t,d]
 *   dstate_in[b,r,d] = sum_{k <= r} w[d,k] * g[b, r - k, d]   (the inputs before token 0)
 *   x, w, bias, width, state_in, flags : exactly those of the forward call
 *   dout, dx     : [batch][seqlen][dim] (io_dtype)
 *   dw           : [dim][width] fp32 output (required)
 *   dbias        : [dim] fp32 output, or NULL (not wanted)
 *   dstate_in    : [batch][width-1][dim] (io_dtype) output, or NULL (not wanted); given also
 *                  when state_in is NULL (then the gradient with respect to the zero history)
 * The forward's state_out is taken to carry no gradient.  dw and dbias are sums over
 * workgroups, accumulated with atomic adds after the library has zeroed them: their last
 * bits may differ from run to run.  Outputs must not overlap inputs or each other.
 * dims->dstate and dims->chunk_len are ignored; seqlen is at most 2^30.  Unknown flag bits
 * return SSM_ERR_FLAGS; a width outside 1..4 returns SSM_ERR_SHAPE. */
SSMSCAN_API int ssm_conv1d_bwd(const void *x, const float *w, const float *bias, int width, const void *state_in,
                   int flags, const void *dout, void *dx, float *dw, float *dbias, void *dstate_in,
                   const ssm_dims *dims, void *stream);

/* The causal convolution + SiLU fused into the scan: the block's main branch from its
 * projected input x to y in one pass (azimuth.plus/paper/mamba, block architecture section:
 * 1-D convolution of kernel size 4, SiLU, selective SSM, times the SiLU gate).  Computes
 *   u = silu(conv_b + conv of x with conv_w)   (as ssm_conv1d_fwd, from a zero history)
 * inside the scan kernel and scans it exactly as ssm_scan_fwd would scan u, without
 * storing u unless u_out is given.  u stays fp32 inside (the two-call path rounds it to
 * io_dtype in between).
 *   x              : [batch][seqlen][dim] (io_dtype), the block's projected input
 *   conv_w, conv_b : [dim][4], [dim] fp32 (conv_b may be NULL);  conv_width must be 4
 *   u_out          : [batch][seqlen][dim] (io_dtype) receives u (for the backward pass), or NULL
 *   flags          : SSM_SCAN_SOFTPLUS and SSM_SCAN_CHECKPOINTS (the exact ZOH is not available
 *                    here: SSM_ERR_FLAGS).  With SSM_SCAN_CHECKPOINTS the backward's
 *                    checkpoints are stored as by ssm_scan_fwd, for ssm_scan_bwd called with
 *                    u = u_out; u is then scanned as rounded to io_dtype (the values u_out
 *                    holds), as the two-call path ssm_conv1d_fwd + ssm_scan_fwd does.
 * Every other argument, the workspace and the errors are those of ssm_scan_fwd. */
SSMSCAN_API int ssm_scan_fwd_conv(const void *x, const float *conv_w, const float *conv_b, int conv_width,
                      const void *delta, const float *A, const void *B, const void *C, const float *D,
                      const void *z, const float *delta_bias, int flags, void *y, float *last_state,
                      void *u_out, const ssm_dims *dims, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Sizes of Mamba-2's state space dual layer (ssm_ssd_fwd). */
typedef struct {
    int64_t batch;     /* sequences */
    int64_t seqlen;    /* tokens per sequence */
    int64_t nheads;    /* heads H */
    int64_t headdim;   /* channels per head P (32 or a multiple of 64) */
    int64_t ngroups;   /* groups G of the B / C projections; H % G == 0 */
    int64_t dstate;    /* states N (32, 64 or 128) */
    int32_t io_dtype;  /* SSM_IO_BF16, or SSM_IO_F32 (dstate 32 or 64) */
    int32_t reserved;  /* 0 */
} ssm_ssd_dims;

/* Mamba-2's state space dual layer (SSD): the selective scan with a scalar state matrix
 * per head, computed in its chunked matrix form on the matrix cores (the sequence map is a
 * 1-semiseparable matrix: mugbit.ir, Mamba-2 / structured state space duality).  Per head h
 * (channels h*P .. h*P+P-1, group g = h / (H/G)):
 *   dt_t     = softplus(dt[t,h] + dt_bias[h])  (SSM_SCAN_SOFTPLUS), else dt + dt_bias
 *   S_t      = exp(dt_t A[h]) S_{t-1} + dt_t x_t B_t[g]^T      (P x N state, from zero)
 *   y_t      = (S_t C_t[g] + D[h] x_t) * silu(z_t)              (z optional)
 *   x, z, y    : [batch][seqlen][nheads][headdim] (io_dtype)
 *   dt         : [batch][seqlen][nheads] (io_dtype)
 *   A, D, dt_bias : [nheads] fp32 (D and dt_bias may be NULL)
 *   B, C       : [batch][seqlen][ngroups][dstate] (io_dtype)
 *   last_state : [batch][nheads][headdim][dstate] fp32 output, or NULL
 * Supported: io_dtype SSM_IO_BF16 or SSM_IO_F32; headdim 32 or a multiple of 64 (a head of
 * 64 v channels runs as v independent 64-channel parts); dstate 32, 64 or 128 (32-wide heads
 * and states are padded to the 64-wide tiles with zeros, at the cost of 64-wide products;
 * dstate 128 takes 128-wide state tiles, one workgroup per CU, headdim a multiple of 64 and
 * bf16 I/O); nheads*headdim <= 2^24 (SSM_ERR_DTYPE / SSM_ERR_SHAPE otherwise); x, z, y, B, C
 * 16-byte aligned.  Products take bf16 operands with fp32 accumulation: the operands formed
 * in the kernel (the decay-weighted products and the state's copy) as high and low bf16
 * parts, and with fp32 I/O x, B and C as well (three products per pair: about 16 bits of
 * each operand; two workgroups per CU instead of three).  The state is carried in fp32.
 * Returns SSM_OK or a negative ssm_status. */
SSMSCAN_API int ssm_ssd_fwd(const void *x, const void *dt, const float *A, const void *B, const void *C,
                const float *D, const void *z, const float *dt_bias, int flags, void *y, float *last_state,
                const ssm_ssd_dims *dims, void *stream);

/* ssm_ssd_fwd continued from a given state (a prefill in pieces, or a decode state carried into
 * a new segment): S_{-1} = initial_state instead of zero.
 *   initial_state : [batch][nheads][headdim][dstate] fp32, or NULL (= zero); it may be the
 *                   last_state buffer (each element is read before it is overwritten)
 * Running a sequence in two calls, the second from the first's last_state, equals one call
 * (bitwise when the first piece's length is a multiple of the 64-token chunk).  With
 * seqlen = 0, last_state receives initial_state (or zeros).  Everything else as ssm_ssd_fwd. */
SSMSCAN_API int ssm_ssd_fwd_from(const float *initial_state, const void *x, const void *dt, const float *A,
                const void *B, const void *C, const float *D, const void *z, const float *dt_bias, int flags,
                void *y, float *last_state, const ssm_ssd_dims *dims, void *stream);

/* One recurrent (inference) step for `batch` independent sequences: the constant-memory
 * recurrent form (shakilmahmud.com section 3; urworte.de "Methodische Grundlagen").
 *   state          : [batch][dim][dstate] fp32, read and overwritten with the new state
 *   u, delta, z, y : [batch][dim] (io_dtype); delta is the already activated step size
 *                    (no bias, no softplus); z may be NULL
 *   B, C           : [batch][dstate] (io_dtype)
 *   A              : [dim][dstate] fp32;  D : [dim] fp32 or NULL
 * Repeating it over a sequence from a zero state reproduces ssm_scan_fwd with
 * flags = 0 and no delta_bias.  Returns SSM_OK or a negative ssm_status. */
SSMSCAN_API int ssm_step(float *state, const void *u, const void *delta, const float *A, const void *B,
             const void *C, const float *D, const void *z, void *y, const ssm_dims *dims,
             void *stream);

/* The recurrent step continuing a sequence that ssm_scan_fwd / ssm_scan_fwd_from produced with
 * activation flags (the prefill -> decode hand-over; recurrent form: shakilmahmud.com section 3;
 * the step size softplus(linear(x)): azimuth.plus/paper/mamba, selection section; the exact
 * zero-order hold: the same page, Theorem 1, and yapayzekasozluk.tr "Temel Matematiksel
 * Cerceve").  Arguments as ssm_step, except:
 *   delta      : [batch][dim] (io_dtype), the raw step-size input as ssm_scan_fwd takes it
 *   delta_bias : [dim] fp32 or NULL (4-byte aligned)
 *   flags      : SSM_SCAN_SOFTPLUS and / or SSM_SCAN_EXACT_ZOH, with the meaning they have for
 *                the scan; any other bit -> SSM_ERR_FLAGS (checkpoints belong to a scan)
 * The step size and the input term are formed with the scan kernel's arithmetic (the same
 * functions, in the same order): after a one-pass prefill by the scan (chunk_len = -1, or a
 * plan without the chunk carry) the steps continue the scan's state bitwise, and their outputs
 * equal the scan's up to the summation order of the readout.  The caller
 * owns every buffer; nothing is allocated; state is updated in place.  Returns SSM_OK or a
 * negative ssm_status (nothing is launched on an error). */
SSMSCAN_API int ssm_step_act(float *state, const void *u, const void *delta, const float *A, const void *B,
             const void *C, const float *D, const void *z, const float *delta_bias, int flags, void *y,
             const ssm_dims *dims, void *stream);

/* Message describing the last non-OK status returned on this thread ("" if none). */
SSMSCAN_API const char *ssm_last_error(void);

/* SSMSCAN_VERSION of the built library. */
SSMSCAN_API int ssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSMSCAN_H */

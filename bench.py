"""Benchmark of the selective scan (S6) forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3|c2|c4|c5] [--no-cpu]

One "step" is one ssm_scan_fwd call over the whole batch (for c5: one ssm_step over the
256 sequences).  Inputs are generated on the host, copied to HBM before the timed region,
and stay resident.  W untimed steps, then exactly K steps between two device
synchronisations; each step is also bracketed by HIP events on the launch stream, which
gives the kernel's average duration for the roofline.  (The decode steps are shorter than
the host's cost per call, so their K timed steps are captured as one HIP graph and the
events bracket its replay.)  Prints one JSON line.

The default workload is the B8 L2048 D5120 N16 bf16 layer scan (z gate, last_state).
The CPU baseline is the fp64 oracle on the host cores, on a channel sample of the same
workload sized to about 10-20 s of CPU work (the channel count comes from a timed probe).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# VALU issue capacity of MI355X: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz, in
# fp32 lane-operations per second (packed fp32 is not used).
VALU_PEAK_TLANEOPS = 256 * 64 * 2.4e9 / 1e12
# Unavoidable VALU issue slots per (token, channel, state): the multiplies delta*A and
# (delta u)*B, the state FMA and the readout FMA at one slot each, and exp2 at half rate.
SLOTS_PER_ELEMENT = 6
# state buffers the decode-step benchmark rotates over (4 x 84 MB > the 256 MB MALL)
ROTATE_STEP = 4

WORKLOADS = {
    "c2": "selective scan B2 L2048 D1536 N16, fp32 I/O, fp32 state",
    "c3": "selective scan B8 L2048 D5120 N16, bf16 I/O, fp32 state, SiLU(z) gate, D skip, last_state",
    "c4": "selective scan B1 L131072 D2048 N16, bf16 I/O, fp32 state, last_state",
    "c5": "recurrent step S256 D5120 N16, bf16 I/O, fp32 state in place",
    "c3_bwd": "selective scan backward B8 L2048 D5120 N16, bf16 I/O, fp32 state, SiLU(z) gate, D skip",
    "c3_train": "selective scan training step (forward with the backward's checkpoints + backward) B8 L2048 "
                "D5120 N16, bf16 I/O, fp32 state, SiLU(z) gate, D skip, last_state",
    "c3_zoh": "selective scan with the exact zero-order-hold input term B8 L2048 D5120 N16, bf16 I/O, "
              "fp32 state, SiLU(z) gate, D skip, last_state",
    "c3_conv": "causal depthwise conv1d (width 4) + SiLU B8 L2048 D5120, bf16 I/O, conv state out",
    "c3_conv_bwd": "causal depthwise conv1d (width 4) + SiLU backward (dx, dw, dbias, dstate) B8 L2048 D5120, "
                   "bf16 I/O",
    "c3_block_train": "block training step: conv1d (width 4) + SiLU fused into the selective scan storing the "
                      "backward's checkpoints and u, then the scan's backward and the convolution's backward, "
                      "B8 L2048 D5120 N16, bf16 I/O, fp32 state, SiLU(z) gate, D skip, last_state",
    "c3_block": "conv1d (width 4) + SiLU fused into the selective scan B8 L2048 D5120 N16, bf16 I/O, fp32 state, "
                "SiLU(z) gate, D skip, last_state",
}
WORKLOADS["ssd"] = ("Mamba-2 SSD layer B8 L2048 H80 P64 N64 G1 (model width 5120), bf16 I/O, fp32 state, "
                    "SiLU(z) gate, D skip, last_state")
WORKLOADS["ssd_f32"] = ("Mamba-2 SSD layer B8 L2048 H80 P64 N64 G1 (model width 5120), fp32 I/O, fp32 state, "
                        "SiLU(z) gate, D skip, last_state")


def host_threads() -> int:
    """Threads the CPU baseline may use: the cores this process is allowed to run on,
    capped by OMP_NUM_THREADS when that is set (the host's CPU share)."""
    n = max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def ssd_alg_bytes(bsz, L, H, P, G, N, es=2):
    """x, z read and y written; dt per head; B, C per group (es bytes each: 2 for bf16, 4 for
    fp32 I/O); A, D, dt_bias; the final state (fp32)."""
    return bsz * L * H * P * es * 3 + bsz * L * H * es + bsz * L * G * N * es * 2 + H * 12 + bsz * H * P * N * 4


def cpu_baseline_ssd(c, alg_bytes_full, target_s=20.0, threads=None):
    """The fp64 oracle's SSD layer on a sample of heads (heads are independent)."""
    from oracle import oracle
    oracle.build(force=False)
    threads = threads or host_threads()

    def run(sel):
        oracle.ssd(c.values("x")[:, :, sel], c.values("dt")[:, :, sel], c.A[sel], c.values("B"), c.values("C"),
                   D=c.Dskip[sel], z=c.values("z")[:, :, sel], dt_bias=c.dt_bias[sel], softplus=True,
                   threads=threads)
    t = time.perf_counter()
    run(np.array([0]))
    per_h = time.perf_counter() - t
    k = int(min(c.H, max(1, target_s / max(per_h, 1e-9))))
    sel = np.unique(np.linspace(0, c.H - 1, k).astype(np.int64))
    t = time.perf_counter()
    run(sel)
    dt = time.perf_counter() - t
    return {"value": round(alg_bytes_full * len(sel) / c.H / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(sel)} of {c.H} heads x all {c.bsz} sequences x {c.L} tokens (fp64 oracle)"}


# The fused convolution adds, per (token, channel), 4 FMAs and SiLU (multiply, exp2 at half
# rate, add, reciprocal at half rate): 10 issue slots.
SLOTS_PER_CHTOK_CONV = 10
# The exact zero-order-hold input term adds, per (token, channel, state), one evaluation of
# (exp(delta A) - 1) / A counted as a transcendental (2 slots) and its multiply (1 slot).
SLOTS_PER_ELEMENT_ZOH = SLOTS_PER_ELEMENT + 3
# VALU issue slots per (token, channel, state) of the backward: the recomputed step (delta*A,
# exp2 = 2, (delta u)*B, state FMA, readout FMA for the gate gradient) and the adjoint step
# (lambda FMA, delta*A and exp2 = 3 for the decay, decay * h_{t-1}, lambda*delta, dA FMA,
# A*(decay h) + B*u = 2, d delta FMA, du FMA, the dB and dC terms, the carried adjoint).
SLOTS_PER_ELEMENT_BWD = 20
METRIC = "selective-scan HBM GB/s (% of peak) + channel-tokens/s, B8 L2048 D5120 N16 bf16"


def scan_alg_bytes(bsz, L, D, N, io_bytes, gate, skip, bias, last_state):
    """Bytes the method must move per call: u, delta, (z), y per element; B, C per token;
    A, D, delta_bias per channel; last_state per (sequence, channel, state)."""
    per_el = io_bytes * (3 + (1 if gate else 0))
    b = bsz * L * D * per_el
    b += 2 * bsz * L * N * io_bytes
    b += D * N * 4 + D * 4 * ((1 if skip else 0) + (1 if bias else 0))
    if last_state:
        b += bsz * D * N * 4
    return b


def step_alg_bytes(S, D, N, io_bytes, gate, skip):
    """state read + write, u, delta, (z), y per (sequence, channel), B, C per sequence, A, D."""
    return S * D * (2 * N * 4 + io_bytes * (3 + (1 if gate else 0))) + 2 * S * N * io_bytes + D * N * 4 + \
        (D * 4 if skip else 0)


def scan_bwd_alg_bytes(bsz, L, D, N, io_bytes):
    """Bytes the backward must move: u, delta, z, dy read and du, ddelta, dz written per
    element; B, C read and dB, dC (fp32) written per token; A, dA, D, dD, bias, dbias."""
    return (bsz * L * D * io_bytes * 7 + bsz * L * N * (2 * io_bytes + 2 * 4) + D * N * 4 * 2 + D * 4 * 4)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_32_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        c = json.load(f)
    if c.get("kernel_source_digest") != kernel_source_digest():
        return None
    return c.get("hbm_bytes_per_launch")


def sized_sample(run, n_total, target_s, probe_n=16):
    """Indices of a sample of n_total independent items (channels, heads) sized to about
    target_s seconds of run(sel), and the time it took: a probe of probe_n items estimates the
    time per item; a sample that ran in under 0.6 of the target (the probe overstates the cost
    of a larger, better-threaded sample) is enlarged by its own measured rate, at most twice."""
    probe = np.unique(np.linspace(0, n_total - 1, min(probe_n, n_total)).astype(np.int64))
    t = time.perf_counter()
    run(probe)
    per = (time.perf_counter() - t) / len(probe)
    k = int(min(n_total, max(len(probe), target_s / max(per, 1e-9))))
    for _ in range(3):
        sel = np.unique(np.linspace(0, n_total - 1, k).astype(np.int64))
        t = time.perf_counter()
        run(sel)
        dt = time.perf_counter() - t
        if dt >= 0.6 * target_s or len(sel) >= n_total:
            break
        k = int(min(n_total, len(sel) * target_s / max(dt, 1e-9)))
    return sel, dt


def cpu_baseline_scan(case, alg_bytes_full, target_s=12.0, target_1core_s=8.0, exact_zoh=False):
    """Time the fp64 oracle on channel samples of the workload: on all the host cores this
    process may use (OpenMP over channels), and on one core.  Channels are independent, so
    each rate is scaled to the whole workload by the sampled fraction."""
    from oracle import oracle
    oracle.build(force=False)
    threads = host_threads()
    D = case.D

    def timed(threads_, budget):
        return sized_sample(lambda sel: oracle.scan_case(case, channels=sel, threads=threads_, exact_zoh=exact_zoh),
                            D, budget)

    sel, dt = timed(threads, target_s)
    sel1, dt1 = timed(1, target_1core_s)
    frac, frac1 = len(sel) / D, len(sel1) / D
    return {"value": round(alg_bytes_full * frac / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "channel_tokens_per_s": round(case.bsz * case.L * len(sel) / dt, 1), "seconds": round(dt, 2),
            "sample": f"{len(sel)} of {D} channels x all {case.bsz} sequences x {case.L} tokens "
                      f"(fp64 oracle, OpenMP over channels, {threads} threads)",
            "single_core": {"value": round(alg_bytes_full * frac1 / dt1 / 1e9, 5), "unit": "GB/s", "cores": 1,
                            "channel_tokens_per_s": round(case.bsz * case.L * len(sel1) / dt1, 1),
                            "seconds": round(dt1, 2),
                            "sample": f"{len(sel1)} of {D} channels x all {case.bsz} sequences x {case.L} tokens"},
            "cpu_model": host_cpu_model()}


def cpu_baseline_bwd(case, alg_bytes_full, target_s=20.0, with_forward=False, threads=None):
    """The fp64 oracle's backward (after its forward, with_forward) on a channel sample of the
    workload (per-channel work is independent; the cross-channel dB / dC sums then cover the
    sample only)."""
    from oracle import oracle
    oracle.build(force=False)
    threads = threads or host_threads()
    rng = np.random.default_rng(12)
    dyv = rng.standard_normal((case.bsz, case.L, 16))

    def run(sel):
        zv = case.values("z")
        if with_forward:
            oracle.scan_case(case, channels=sel, threads=threads)
        oracle.scan_bwd(case.values("u")[:, :, sel], case.values("delta")[:, :, sel], case.A[sel], case.values("B"),
                        case.values("C"), np.resize(dyv, (case.bsz, case.L, len(sel))), D=case.Dskip[sel],
                        z=None if zv is None else zv[:, :, sel], delta_bias=case.delta_bias[sel],
                        softplus=case.softplus, threads=threads)
    sel, dt = sized_sample(run, case.D, target_s)
    return {"value": round(alg_bytes_full * len(sel) / case.D / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(sel)} of {case.D} channels x all {case.bsz} sequences x {case.L} tokens "
                      f"(fp64 oracle {'forward + ' if with_forward else ''}backward, OpenMP over channels)"}


def conv_alg_bytes(bsz, L, D, width, io_bytes):
    """x read and out written per element, the state rows written, w and bias read."""
    return bsz * L * D * io_bytes * 2 + bsz * (width - 1) * D * io_bytes + D * (width + 1) * 4


def conv_bwd_alg_bytes(bsz, L, D, width, io_bytes):
    """x and dout read and dx written per element, the state rows read and their gradient
    written, w and bias read, dw and dbias written."""
    return bsz * L * D * io_bytes * 3 + bsz * (width - 1) * D * io_bytes * 2 + D * (width + 1) * 4 * 2


def cpu_baseline_conv_bwd(case, dout, alg_bytes_full, target_s=20.0):
    """The fp64 oracle's convolution backward on a channel sample of the workload (channels
    are independent; single-threaded)."""
    from oracle import oracle
    oracle.build(force=False)
    g = inputs_bf16_f64(dout)

    def run(sel):
        oracle.conv1d_bwd(case.values("x")[:, :, sel], case.w[sel], g[:, :, sel], bias=case.bias[sel],
                          state=case.values("state")[:, :, sel], silu=True)
    probe = np.arange(32)
    t = time.perf_counter()
    run(probe)
    per_ch = (time.perf_counter() - t) / len(probe)
    k = int(min(case.D, max(32, target_s / max(per_ch, 1e-9))))
    sel = np.unique(np.linspace(0, case.D - 1, k).astype(np.int64))
    t = time.perf_counter()
    run(sel)
    dt = time.perf_counter() - t
    return {"value": round(alg_bytes_full * len(sel) / case.D / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(sel)} of {case.D} channels x all {case.bsz} sequences x {case.L} tokens "
                      f"(fp64 oracle backward)"}


def inputs_bf16_f64(bits):
    from selective_state_space_32_amd import inputs
    return inputs.bf16_to_f32(bits).astype(np.float64)


def cpu_baseline_conv(case, alg_bytes_full, target_s=20.0):
    """The fp64 oracle's convolution on a channel sample of the workload (channels are
    independent; single-threaded)."""
    from oracle import oracle
    oracle.build(force=False)

    def run(sel):
        oracle.conv1d(case.values("x")[:, :, sel], case.w[sel], bias=case.bias[sel],
                      state=None if case.state is None else case.values("state")[:, :, sel], silu=True)
    probe = np.arange(64)
    t = time.perf_counter()
    run(probe)
    per_ch = (time.perf_counter() - t) / len(probe)
    k = int(min(case.D, max(64, target_s / max(per_ch, 1e-9))))
    sel = np.unique(np.linspace(0, case.D - 1, k).astype(np.int64))
    t = time.perf_counter()
    run(sel)
    dt = time.perf_counter() - t
    return {"value": round(alg_bytes_full * len(sel) / case.D / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(sel)} of {case.D} channels x all {case.bsz} sequences x {case.L} tokens (fp64 oracle)"}


def cpu_baseline_block(case, cc, alg_bytes_full, target_s=20.0, threads=None):
    """The fp64 oracle's convolution followed by its scan, on a channel sample."""
    from oracle import oracle
    oracle.build(force=False)
    threads = threads or host_threads()

    def run(sel):
        u, _ = oracle.conv1d(cc.values("x")[:, :, sel], cc.w[sel], bias=cc.bias[sel], silu=True)
        oracle.scan(u, case.values("delta")[:, :, sel], case.A[sel], case.values("B"), case.values("C"),
                    D=case.Dskip[sel], z=case.values("z")[:, :, sel], delta_bias=case.delta_bias[sel],
                    softplus=case.softplus, threads=threads)
    probe = np.arange(16)
    t = time.perf_counter()
    run(probe)
    per_ch = (time.perf_counter() - t) / len(probe)
    k = int(min(case.D, max(16, target_s / max(per_ch, 1e-9))))
    sel = np.unique(np.linspace(0, case.D - 1, k).astype(np.int64))
    t = time.perf_counter()
    run(sel)
    dt = time.perf_counter() - t
    return {"value": round(alg_bytes_full * len(sel) / case.D / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(sel)} of {case.D} channels x all {case.bsz} sequences x {case.L} tokens "
                      f"(fp64 oracle convolution, then scan)"}


def cpu_baseline_block_train(case, cc, alg_bytes_full, target_s=20.0, threads=None):
    """The fp64 oracle's block training step on a channel sample: convolution, scan, the
    scan's backward, the convolution's backward."""
    from oracle import oracle
    oracle.build(force=False)
    threads = threads or host_threads()
    rng = np.random.default_rng(13)
    dyv = rng.standard_normal((case.bsz, case.L, 16))

    def run(sel):
        u, _ = oracle.conv1d(cc.values("x")[:, :, sel], cc.w[sel], bias=cc.bias[sel], silu=True)
        zs = case.values("z")[:, :, sel]
        args = (u, case.values("delta")[:, :, sel], case.A[sel], case.values("B"), case.values("C"))
        kw = dict(D=case.Dskip[sel], z=zs, delta_bias=case.delta_bias[sel], softplus=case.softplus)
        oracle.scan(*args, threads=threads, **kw)
        g = oracle.scan_bwd(*args, np.resize(dyv, (case.bsz, case.L, len(sel))), threads=threads, **kw)
        oracle.conv1d_bwd(cc.values("x")[:, :, sel], cc.w[sel], g["du"], bias=cc.bias[sel], silu=True)
    probe = np.arange(16)
    t = time.perf_counter()
    run(probe)
    per_ch = (time.perf_counter() - t) / len(probe)
    k = int(min(case.D, max(16, target_s / max(per_ch, 1e-9))))
    sel = np.unique(np.linspace(0, case.D - 1, k).astype(np.int64))
    t = time.perf_counter()
    run(sel)
    dt = time.perf_counter() - t
    return {"value": round(alg_bytes_full * len(sel) / case.D / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{len(sel)} of {case.D} channels x all {case.bsz} sequences x {case.L} tokens "
                      f"(fp64 oracle convolution, scan, scan backward, convolution backward)"}


def cpu_baseline_step(case, alg_bytes_step, target_s=20.0, threads=None):
    from oracle import oracle
    oracle.build(force=False)
    threads = threads or host_threads()
    st = case.state0.astype(np.float64)
    done = 0
    t = time.perf_counter()
    while time.perf_counter() - t < target_s and done < case.steps:
        k = done
        _, st = oracle.step(st, case.values("u")[k], case.values("delta")[k], case.A, case.values("B")[k],
                            case.values("C")[k], D=case.Dskip, z=case.values("z")[k], threads=threads)
        done += 1
    dt = time.perf_counter() - t
    return {"value": round(alg_bytes_step * done / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2), "sample": f"{done} of {case.steps} steps over all {case.S} sequences"}


def with_one_core(leg, target_s=12.0, target_1core_s=6.0):
    """A CPU-baseline leg on all the host cores this process may use, then on one core (a
    shorter sample); the one-core rate and the CPU model go into the result."""
    r = leg(target_s=target_s)
    one = leg(target_s=target_1core_s, threads=1)
    r["single_core"] = {k: one[k] for k in ("value", "unit", "cores", "seconds", "sample") if k in one}
    r["cpu_model"] = host_cpu_model()
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the scan, run a plain device copy of MIB MiB (the reference kernel "
                         "for scaling HBM byte counters) and print its size")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": max(1, args.steps)}))
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the scan shards "
              "with no communication across sequences and channels, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_32_amd import inputs, ssmscan

    dev = "cuda"
    wl = args.workload
    if wl in ("c3_conv", "c3_conv_bwd"):
        case = inputs.conv_case(8, 2048, 5120, 4, "bf16", state=True, seed=185, name=wl)
    elif wl in ("ssd", "ssd_f32"):
        case = inputs.ssd_case(8, 2048, 80, 64, 1, 64, seed=230, name=wl, io="f32" if wl == "ssd_f32" else "bf16")
    else:
        case = inputs.config_case("c3" if wl in ("c3_bwd", "c3_train", "c3_zoh", "c3_block", "c3_block_train")
                                  else wl)
    io_bytes = 2 if getattr(case, "io", "bf16") == "bf16" else 4

    def td(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    stream = torch.cuda.current_stream()
    if wl == "c5":
        S, D, N = case.S, case.D, case.N
        A, Dv = td(case.A), td(case.Dskip)
        st = td(case.state0).clone()
        # R state buffers of 84 MB each, more than the 256 MB MALL together: steps that rotate
        # over them read each state cold from HBM; steps on one buffer find it in the MALL
        rot_states = [st] + [td(case.state0).clone() for _ in range(ROTATE_STEP - 1)]
        ins = [(td(case.u[k]), td(case.delta[k]), td(case.B[k]), td(case.C[k]), td(case.z[k]))
               for k in range(case.steps)]
        y = torch.empty((S, D), dtype=torch.bfloat16, device=dev)
        alg = step_alg_bytes(S, D, N, io_bytes, True, True)
        chtok = S * D
        elements = S * D * N

        # each step's call checked and marshalled once, outside the timed region
        calls = [ssmscan.step_call(st, u, dl, A, Bk, Ck, D=Dv, z=z, y=y) for (u, dl, Bk, Ck, z) in ins]

        def one(i):
            calls[i % case.steps]()
        plan = "one step kernel per call"
    elif wl in ("ssd", "ssd_f32"):
        c = case
        sx, sdt, sB, sC, sz = (td(a) for a in (c.x, c.dt, c.B, c.C, c.z))
        sA, sD, sbias = td(c.A), td(c.Dskip), td(c.dt_bias)
        ys = torch.empty_like(sx)
        lss = torch.empty((c.bsz, c.H, c.P, c.N), dtype=torch.float32, device=dev)
        alg = ssd_alg_bytes(c.bsz, c.L, c.H, c.P, c.G, c.N, 4 if c.io == "f32" else 2)
        chtok = c.bsz * c.L * c.H * c.P
        elements = chtok * c.N

        def one(i):
            ssmscan.ssd_fwd(sx, sdt, sA, sB, sC, D=sD, z=sz, dt_bias=sbias, y=ys, last_state=lss)
        plan = ("one workgroup per (sequence, head), chunks of 64 tokens, four 64x64x64 bf16 MFMA products per chunk"
                + (" (fp32 x, B, C as bf16 high + low parts: three products per pair; two workgroups per CU)"
                   if c.io == "f32" else ""))
    elif wl == "c3_conv":
        bsz, L, D, width = case.bsz, case.L, case.D, case.width
        x, st_in = td(case.x), td(case.state)
        out = torch.empty_like(x)
        st_out = torch.empty_like(st_in)
        # a second input / output set (168 MB each): steps alternating over the two sets read
        # x cold from HBM (336 MB of other traffic between two reads of one x)
        rot_conv = [(x, out), (x.clone(), torch.empty_like(x))]
        alg = conv_alg_bytes(bsz, L, D, width, io_bytes)
        chtok = bsz * L * D
        elements = chtok
        td_w, td_b = td(case.w), td(case.bias)
        call = ssmscan.conv1d_call(x, td_w, td_b, st_in, silu=True, out=out, state_out=st_out)

        def one(i):
            call()
        plan = "one kernel, runs of 32 tokens x 4 channels per thread"
    elif wl == "c3_conv_bwd":
        bsz, L, D, width = case.bsz, case.L, case.D, case.width
        x, st_in = td(case.x), td(case.state)
        dout_bits = inputs.bf16_bits(np.random.default_rng(186).standard_normal((bsz, L, D), dtype=np.float32))
        dout = td(dout_bits)
        alg = conv_bwd_alg_bytes(bsz, L, D, width, io_bytes)
        chtok = bsz * L * D
        elements = chtok
        td_w, td_b = td(case.w), td(case.bias)
        dx = torch.empty_like(x)
        call, _grads = ssmscan.conv1d_bwd_call(dout, x, td_w, td_b, st_in, silu=True, dx=dx)
        rot_conv = [(x, dout, dx), (x.clone(), dout.clone(), torch.empty_like(dx))]

        def one(i):
            call()
        plan = ("one fill launch zeroing dw and dbias, then one kernel: a wave walks a run of 64 tokens, "
                "2 channels per lane, 4 runs per workgroup, dw / dbias reduced in LDS and added atomically")
    elif wl == "c3_bwd":
        t = {k: td(getattr(case, f)) for k, f in (("u", "u"), ("delta", "delta"), ("A", "A"), ("B", "B"),
                                                   ("C", "C"), ("D", "Dskip"), ("z", "z"), ("bias", "delta_bias"))}
        bsz, L, D, N = case.bsz, case.L, case.D, case.N
        dy = td(inputs.bf16_bits(np.random.default_rng(13).standard_normal((bsz, L, D), dtype=np.float32)))
        ws = torch.empty(max(1, ssmscan.bwd_workspace_bytes(bsz, L, D, N, dy.dtype)), dtype=torch.uint8, device=dev)
        grads = ssmscan.scan_bwd(dy, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                 delta_bias=t["bias"], softplus=case.softplus, workspace=ws)
        alg = scan_bwd_alg_bytes(bsz, L, D, N, io_bytes)
        chtok = bsz * L * D
        elements = chtok * N

        def one(i):
            ssmscan.scan_bwd(dy, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             delta_bias=t["bias"], softplus=case.softplus, workspace=ws, out=grads)
        pinfo = ssmscan.plan_info(bsz, L, D, N, dy.dtype)
        plan = ("one fill launch, checkpoint pass (state every 8 tokens) + backward kernel"
                + (f", both under the split schedule ({pinfo['split_tiles']} of {bsz * ((D + 63) // 64)} tiles as "
                   f"two token halves, {pinfo['workgroups']} workgroups)" if pinfo["split_tiles"] else ""))
    elif wl == "c3_train":
        t = {k: td(getattr(case, f)) for k, f in (("u", "u"), ("delta", "delta"), ("A", "A"), ("B", "B"),
                                                   ("C", "C"), ("D", "Dskip"), ("z", "z"), ("bias", "delta_bias"))}
        bsz, L, D, N = case.bsz, case.L, case.D, case.N
        dy = td(inputs.bf16_bits(np.random.default_rng(13).standard_normal((bsz, L, D), dtype=np.float32)))
        y = torch.empty((bsz, L, D), dtype=dy.dtype, device=dev)
        ls = torch.empty((bsz, D, N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, ssmscan.bwd_workspace_bytes(bsz, L, D, N, dy.dtype) +
                             ssmscan.workspace_bytes(bsz, L, D, N, dy.dtype)), dtype=torch.uint8, device=dev)
        fwd = ssmscan.scan_fwd_call(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                    delta_bias=t["bias"], softplus=case.softplus, y=y, last_state=ls, workspace=ws,
                                    save_checkpoints=True)
        fwd()
        grads = ssmscan.scan_bwd(dy, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                 delta_bias=t["bias"], softplus=case.softplus, checkpoints=ws)
        alg = scan_alg_bytes(bsz, L, D, N, io_bytes, True, True, True, True) + scan_bwd_alg_bytes(bsz, L, D, N,
                                                                                                 io_bytes)
        chtok = bsz * L * D
        elements = chtok * N

        def one(i):
            fwd()
            ssmscan.scan_bwd(dy, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             delta_bias=t["bias"], softplus=case.softplus, checkpoints=ws, out=grads)
        pinfo = ssmscan.plan_info(bsz, L, D, N, dy.dtype)
        plan = ("forward storing the backward's checkpoints (state every 8 tokens) + backward kernel from them"
                + (f", both under the split schedule ({pinfo['split_tiles']} tiles as two token halves)"
                   if pinfo["split_tiles"] else ""))
    elif wl == "c3_block_train":
        t = {k: td(getattr(case, f)) for k, f in (("delta", "delta"), ("A", "A"), ("B", "B"), ("C", "C"),
                                                   ("D", "Dskip"), ("z", "z"), ("bias", "delta_bias"))}
        bsz, L, D, N = case.bsz, case.L, case.D, case.N
        cc = inputs.conv_case(bsz, L, D, 4, case.io, seed=4, name="c3_block_train")
        x, cw, cb = td(cc.x), td(cc.w), td(cc.bias)
        dy = td(inputs.bf16_bits(np.random.default_rng(13).standard_normal((bsz, L, D), dtype=np.float32)))
        y = torch.empty((bsz, L, D), dtype=dy.dtype, device=dev)
        u = torch.empty_like(y)
        ls = torch.empty((bsz, D, N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, ssmscan.bwd_workspace_bytes(bsz, L, D, N, dy.dtype) +
                             ssmscan.workspace_bytes(bsz, L, D, N, dy.dtype)), dtype=torch.uint8, device=dev)
        kw = dict(D=t["D"], z=t["z"], delta_bias=t["bias"], softplus=case.softplus)
        fwd = ssmscan.scan_fwd_conv_call(x, cw, cb, t["delta"], t["A"], t["B"], t["C"], y=y, last_state=ls,
                                         u_out=u, workspace=ws, save_checkpoints=True, **kw)
        fwd()
        grads = ssmscan.scan_bwd(dy, u, t["delta"], t["A"], t["B"], t["C"], checkpoints=ws, **kw)
        dx = torch.empty_like(x)
        cbwd, _cgrads = ssmscan.conv1d_bwd_call(grads["du"], x, cw, cb, silu=True, dx=dx)
        alg = (scan_alg_bytes(bsz, L, D, N, io_bytes, True, True, True, True) + D * 5 * 4 + bsz * L * D * io_bytes
               + scan_bwd_alg_bytes(bsz, L, D, N, io_bytes) + conv_bwd_alg_bytes(bsz, L, D, 4, io_bytes))
        chtok = bsz * L * D
        elements = chtok * N

        def one(i):
            fwd()
            ssmscan.scan_bwd(dy, u, t["delta"], t["A"], t["B"], t["C"], checkpoints=ws, out=grads, **kw)
            cbwd()
        plan = ("fused convolution + scan storing u and the backward's checkpoints, scan backward from them, "
                "convolution backward")
    else:
        t = {k: td(getattr(case, f)) for k, f in (("u", "u"), ("delta", "delta"), ("A", "A"), ("B", "B"),
                                                   ("C", "C"), ("D", "Dskip"), ("z", "z"), ("bias", "delta_bias"))}
        bsz, L, D, N = case.bsz, case.L, case.D, case.N
        dtype = t["u"].dtype
        y = torch.empty((bsz, L, D), dtype=dtype, device=dev)
        ls = torch.empty((bsz, D, N), dtype=torch.float32, device=dev)
        nchunk, clen = ssmscan.scan_plan(bsz, L, D, N, dtype)
        ws = torch.empty(max(1, ssmscan.workspace_bytes(bsz, L, D, N, dtype)), dtype=torch.uint8, device=dev)
        alg = scan_alg_bytes(bsz, L, D, N, io_bytes, case.z is not None, case.Dskip is not None,
                             case.delta_bias is not None, True)
        chtok = bsz * L * D
        elements = chtok * N

        if wl == "c3_block":
            # the block's projected input x in place of u, width-4 convolution weights
            cc = inputs.conv_case(bsz, L, D, 4, case.io, seed=4, name="c3_block")
            call = ssmscan.scan_fwd_conv_call(td(cc.x), td(cc.w), td(cc.bias), t["delta"], t["A"], t["B"], t["C"],
                                              D=t["D"], z=t["z"], delta_bias=t["bias"], softplus=case.softplus, y=y,
                                              last_state=ls, workspace=ws)
            alg += D * 5 * 4   # the convolution's taps and bias
        else:
            call = ssmscan.scan_fwd_call(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                         delta_bias=t["bias"], softplus=case.softplus, y=y, last_state=ls,
                                         workspace=ws, exact_zoh=wl == "c3_zoh")

        def one(i):
            call()
        pinfo = ssmscan.plan_info(bsz, L, D, N, dtype)
        if pinfo["split_tiles"] > 0:
            plan = (f"one pass, split schedule on {pinfo['cu_count']} CUs: {pinfo['workgroups'] - 2 * pinfo['split_tiles']}"
                    f" whole tiles + {pinfo['split_tiles']} tiles as two token halves (from token "
                    f"{pinfo['split_at']}), {pinfo['workgroups']} workgroups")
        elif nchunk == 1:
            plan = "single pass"
        else:
            plan = f"{nchunk} chunks of {clen} tokens (summary + carry + scan)"
        if wl == "c3_zoh":
            plan += ", exact zero-order-hold input term"
        if wl == "c3_block":
            plan += ", convolution + SiLU in the scan's preparation"
    torch.cuda.synchronize()

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    resident = None
    if wl in ("c5", "c3_conv", "c3_conv_bwd"):
        # A decode step (~35 us) or the convolution (~65 us) is short next to the host's cost
        # per call: the K timed steps are captured once as a HIP graph (the library allocates
        # and synchronises nothing, so its launches capture as they are) and replayed as one
        # submission.  Two graphs: the steps on one buffer set (whose data the 256 MB MALL
        # partly keeps between steps) and the steps rotating over buffer sets larger than the
        # MALL together (every step reads its inputs from HBM); the rotating one is `value`.
        def step_on(i, rot, cap):
            if wl == "c5":
                u, dl, Bk, Ck, z = ins[i % case.steps]
                ssmscan.step(rot_states[i % ROTATE_STEP] if rot else st, u, dl, A, Bk, Ck, D=Dv, z=z, y=y)
            elif wl == "c3_conv_bwd":
                xx, dd, gx = rot_conv[i % 2] if rot else (x, dout, dx)
                ssmscan.conv1d_bwd(dd, xx, td_w, td_b, st_in, silu=True, dx=gx, stream=cap)
            else:
                xx, oo = rot_conv[i % 2] if rot else (x, out)
                ssmscan.conv1d(xx, td_w, td_b, st_in, silu=True, out=oo, state_out=st_out, stream=cap)

        def graph_run(rot):
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            with torch.cuda.graph(graph, stream=cap):
                for i in range(args.steps):
                    step_on(i, rot, cap)
            torch.cuda.synchronize()
            graph.replay()   # one untimed replay
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e-3 / args.steps

        _, res_s = graph_run(False)
        wall, rot_s = graph_run(True)
        per = np.full(args.steps, rot_s)  # seconds per step
        resident = {"kernel_us_mean": round(res_s * 1e6, 3), "kernel_gbps": round(alg / res_s / 1e9, 2),
                    "note": "the same K steps on one buffer set: part of the data stays in the 256 MB MALL "
                            "between steps, so this rate is not an HBM rate"}
        plan += (f"; the timed steps replayed as one HIP graph, rotating over "
                 f"{ROTATE_STEP if wl == 'c5' else 2} buffer sets larger than the MALL together")
    else:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            one(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3  # seconds per launch
    ms_per_step = wall / args.steps * 1e3
    kern_s = float(np.mean(per))

    step_s = wall / args.steps
    gbps = alg / step_s / 1e9          # whole-job throughput over the timed region
    kern_gbps = alg / kern_s / 1e9     # the kernel's own rate (event-timed launches)
    slots = {"c3_bwd": SLOTS_PER_ELEMENT_BWD, "c3_zoh": SLOTS_PER_ELEMENT_ZOH,
             "c3_train": SLOTS_PER_ELEMENT + SLOTS_PER_ELEMENT_BWD,
             "c3_block_train": SLOTS_PER_ELEMENT + SLOTS_PER_ELEMENT_BWD}.get(wl, SLOTS_PER_ELEMENT)
    work_ops = elements * slots + (chtok * SLOTS_PER_CHTOK_CONV if wl in ("c3_block", "c3_block_train") else 0)
    lane_ops = work_ops / kern_s / 1e12
    traffic = counter_traffic(wl)
    if wl in ("c5", "c3_conv", "c3_conv_bwd", "ssd", "ssd_f32"):
        roof = {"bound": "hbm", "achieved": round(kern_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(kern_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "alu", "achieved": round(lane_ops, 3), "peak": round(VALU_PEAK_TLANEOPS, 3),
                "unit": "T fp32 VALU lane-ops/s", "frac": round(lane_ops / VALU_PEAK_TLANEOPS, 4),
                "traffic": traffic,
                "hbm": {"achieved": round(kern_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(kern_gbps / HBM_PEAK_GBPS, 4)},
                "work": f"{slots} VALU issue slots per (token, channel, state) x {elements} per launch"
                        + (f" + {SLOTS_PER_CHTOK_CONV} per (token, channel) x {chtok} for the convolution"
                           if wl in ("c3_block", "c3_block_train") else "")
                        + (" (the convolution's backward, bound by HBM, is not counted)" if wl == "c3_block_train"
                           else "")}

    cpu = None
    if not args.no_cpu:
        try:
            if wl in ("c3_conv", "c3_conv_bwd"):   # (single-threaded oracle: one core already)
                cpu = (cpu_baseline_conv(case, alg) if wl == "c3_conv" else cpu_baseline_conv_bwd(case, dout_bits, alg))
                cpu["cpu_model"] = host_cpu_model()
            elif wl in ("c2", "c3", "c4", "c3_zoh"):
                cpu = cpu_baseline_scan(case, alg, exact_zoh=wl == "c3_zoh")
            else:
                leg = {"c5": lambda **k: cpu_baseline_step(case, alg, **k),
                       "c3_bwd": lambda **k: cpu_baseline_bwd(case, alg, **k),
                       "c3_train": lambda **k: cpu_baseline_bwd(case, alg, with_forward=True, **k),
                       "ssd": lambda **k: cpu_baseline_ssd(case, alg, **k),
                       "ssd_f32": lambda **k: cpu_baseline_ssd(case, alg, **k),
                       "c3_block": lambda **k: cpu_baseline_block(case, cc, alg, **k),
                       "c3_block_train": lambda **k: cpu_baseline_block_train(case, cc, alg, **k)}[wl]
                cpu = with_one_core(leg)
        except Exception as e:  # the GPU figures stand without it
            cpu = {"error": repr(e)}

    out = {
        "metric": METRIC if wl == "c3" else f"{WORKLOADS[wl]}: HBM GB/s (% of peak) + channel-tokens/s",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[wl], "io_dtype": getattr(case, "io", "bf16"), "state_dtype": "f32",
                   "plan": plan,
                   "channel_tokens_per_step": chtok, "alg_bytes_per_step": alg},
        "hbm_pct_of_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "channel_tokens_per_s": round(chtok / step_s, 1),
        "kernel_gbps": round(kern_gbps, 2),
        "kernel_us_mean": round(kern_s * 1e6, 3),
        "kernel_us_p10_p50_p90": [round(float(np.percentile(per, q)) * 1e6, 3) for q in (10, 50, 90)],
        "roofline": roof,
        "cpu_baseline": cpu,
        **({"mall_resident": resident} if resident else {}),
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""TEST INFRASTRUCTURE ONLY: Python entry to the fp64 CPU oracle (ssm_oracle.c).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may use
this module; the GPU library never does.  Inputs are any float arrays (the exact fp32
values of fp32 or bf16-rounded tensors); they are widened to fp64 without rounding and
the C definition is run on them.  See ssm_oracle.c for what is computed and where the
pages state it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
# SSM_ORACLE_LIBRARY may name another build of the same source (the sanitized one, see build)
_SANITIZED = os.environ.get("SSM_ORACLE_LIBRARY", "")
_LIBPATH = _SANITIZED or os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra"]
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False, out: str = "") -> str:
    """Compile ssm_oracle.c into liboracle.so with gcc (fp64, no FMA contraction).  sanitize:
    an AddressSanitizer + UBSan build at `out` instead (run Python with gcc's libasan
    preloaded, ASAN_OPTIONS=detect_leaks=0 and SSM_ORACLE_LIBRARY=<out>)."""
    global _lib
    if sanitize:
        out = out or os.path.join(os.path.dirname(_HERE), "_build", "liboracle_asan.so")
        os.makedirs(os.path.dirname(out), exist_ok=True)
        subprocess.run(["gcc", *_CFLAGS, *_SAN_FLAGS, _SRC, "-o", out, "-lm"], check=True)
        return out
    if _SANITIZED:   # a sanitized build named by the environment is used as it is
        return _LIBPATH
    if force or not os.path.exists(_LIBPATH):
        tmp = _LIBPATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIBPATH)
        _lib = None
    return _LIBPATH


def _load():
    global _lib
    if _lib is None:
        if not _SANITIZED and (not os.path.exists(_LIBPATH) or os.path.getmtime(_LIBPATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIBPATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.ssm_oracle_scan.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P, ctypes.c_int,
                                        P, P, ctypes.c_int]
        lib.ssm_oracle_scan.restype = ctypes.c_int
        lib.ssm_oracle_scan_from.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int,
                                             P, P, ctypes.c_int]
        lib.ssm_oracle_scan_from.restype = ctypes.c_int
        lib.ssm_oracle_scan_bwd.argtypes = [I64, I64, I64, I64] + [P] * 9 + [ctypes.c_int] + [P] * 11 + \
            [ctypes.c_int]
        lib.ssm_oracle_scan_bwd.restype = ctypes.c_int
        lib.ssm_oracle_step.argtypes = [I64, I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.ssm_oracle_step.restype = ctypes.c_int
        lib.ssm_oracle_conv1d.argtypes = [I64, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P]
        lib.ssm_oracle_conv1d.restype = ctypes.c_int
        lib.ssm_oracle_conv1d_bwd.argtypes = [I64, I64, I64, I64, P, P, P, P, ctypes.c_int, P, P, P, P, P]
        lib.ssm_oracle_conv1d_bwd.restype = ctypes.c_int
        lib.ssm_oracle_ssd.argtypes = [I64] * 6 + [P] * 9 + [ctypes.c_int, P, P, ctypes.c_int]
        lib.ssm_oracle_ssd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a, shape=None) -> Optional[np.ndarray]:
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"shape {a.shape} != {tuple(shape)}")
    return a


def _ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


def scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus: bool = True,
         threads: Optional[int] = None, h0=None, exact_zoh: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 selective scan from h = 0, or from the state h0 (bsz, Dch, N) if given.
    exact_zoh: input term (exp(delta A) - 1) / A * B * u instead of delta * B * u.

    u, delta, z: (bsz, L, Dch); B, C: (bsz, L, N); A: (Dch, N); D, delta_bias: (Dch,).
    Returns (y (bsz, L, Dch), last_state (bsz, Dch, N)), both float64.
    """
    u = _f64(u)
    bsz, L, Dch = u.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (bsz, L, Dch))
    A = _f64(A, (Dch, N))
    B = _f64(B, (bsz, L, N))
    C = _f64(C, (bsz, L, N))
    D = _f64(D, (Dch,))
    z = _f64(z, (bsz, L, Dch))
    delta_bias = _f64(delta_bias, (Dch,))
    y = np.empty((bsz, L, Dch), dtype=np.float64)
    last = np.empty((bsz, Dch, N), dtype=np.float64)
    h0 = _f64(h0, (bsz, Dch, N))
    rc = _load().ssm_oracle_scan_from(bsz, L, Dch, N, _ptr(h0), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                      _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                      int(bool(softplus)) | (2 if exact_zoh else 0),
                                      _ptr(y), _ptr(last), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle scan rejected N=%d" % N)
    return y, last


def scan_varlen(u, delta, A, B, C, seq_lens, D=None, z=None, delta_bias=None, softplus: bool = True,
                threads: Optional[int] = None, h0=None, exact_zoh: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """The scan of sequences of different lengths: sequence b over its first seq_lens[b] tokens
    (clamped to [0, L]) only, each from h0[b] (or zero), exactly as the scan of that sequence
    alone (the recurrent form, shakilmahmud.com section 3).  Returns (y, last_state): y
    (bsz, L, Dch) with NaN at the tokens past each length (never computed), last_state the
    state after each sequence's own length."""
    u = _f64(u)
    bsz, L, Dch = u.shape
    A = _f64(A)
    N = A.shape[1]
    y = np.full((bsz, L, Dch), np.nan)
    last = np.empty((bsz, Dch, N))
    for b in range(bsz):
        lb = int(min(max(int(seq_lens[b]), 0), L))
        hb = None if h0 is None else np.asarray(h0, np.float64)[b:b + 1]
        if lb == 0:
            last[b] = 0.0 if hb is None else hb[0]
            continue
        sl = (slice(b, b + 1), slice(0, lb))
        yb, lsb = scan(u[sl], np.asarray(delta)[sl], A, np.asarray(B)[sl], np.asarray(C)[sl], D=D,
                       z=None if z is None else np.asarray(z)[sl], delta_bias=delta_bias, softplus=softplus,
                       threads=threads, h0=hb, exact_zoh=exact_zoh)
        y[b, :lb] = yb[0]
        last[b] = lsb[0]
    return y, last


def scan_bwd_varlen(u, delta, A, B, C, dy, seq_lens, D=None, z=None, delta_bias=None, softplus: bool = True,
                    h0=None, dlast=None, threads: Optional[int] = None, exact_zoh: bool = False) -> dict:
    """Gradients of scan_varlen: sequence b is the scan of its first seq_lens[b] tokens
    (clamped to [0, L]) alone, so its gradients are scan_bwd of that prefix, with dlast[b]
    applied to the state after its own length; the inputs past a length do not reach any
    output, so their gradients (du, ddelta, dz, dB, dC) are zero.  dA, dD, ddelta_bias are sums
    over the sequences; dh0 (always returned) is the gradient of each sequence's initial state
    (dlast[b] itself for a length of 0)."""
    u = _f64(u)
    bsz, L, Dch = u.shape
    A = _f64(A)
    N = A.shape[1]
    out = dict(du=np.zeros((bsz, L, Dch)), ddelta=np.zeros((bsz, L, Dch)), dA=np.zeros((Dch, N)),
               dB=np.zeros((bsz, L, N)), dC=np.zeros((bsz, L, N)), dh0=np.zeros((bsz, Dch, N)))
    if D is not None:
        out["dD"] = np.zeros(Dch)
    if z is not None:
        out["dz"] = np.zeros((bsz, L, Dch))
    if delta_bias is not None:
        out["ddelta_bias"] = np.zeros(Dch)
    for b in range(bsz):
        lb = int(min(max(int(seq_lens[b]), 0), L))
        dl_b = None if dlast is None else np.asarray(dlast, np.float64)[b:b + 1]
        if lb == 0:
            if dl_b is not None:
                out["dh0"][b] = dl_b[0]
            continue
        sl = (slice(b, b + 1), slice(0, lb))
        h0_b = np.zeros((1, Dch, N)) if h0 is None else np.asarray(h0, np.float64)[b:b + 1]
        g = scan_bwd(u[sl], np.asarray(delta)[sl], A, np.asarray(B)[sl], np.asarray(C)[sl], np.asarray(dy)[sl],
                     D=D, z=None if z is None else np.asarray(z)[sl], delta_bias=delta_bias, softplus=softplus,
                     h0=h0_b, dlast=dl_b, threads=threads, exact_zoh=exact_zoh)
        for k in ("du", "ddelta", "dB", "dC") + (("dz",) if z is not None else ()):
            out[k][b, :lb] = g[k][0]
        for k in ("dA",) + (("dD",) if D is not None else ()) + (("ddelta_bias",) if delta_bias is not None else ()):
            out[k] += g[k]
        out["dh0"][b] = g["dh0"][0]
    return out


def step(state, u, delta, A, B, C, D=None, z=None,
         threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 single-token step.  state: (S, Dch, N); u, delta, z: (S, Dch); B, C: (S, N).
    delta is already activated.  Returns (y (S, Dch), new_state (S, Dch, N))."""
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    S, Dch, N = st.shape
    u = _f64(u, (S, Dch))
    delta = _f64(delta, (S, Dch))
    A = _f64(A, (Dch, N))
    B = _f64(B, (S, N))
    C = _f64(C, (S, N))
    D = _f64(D, (Dch,))
    z = _f64(z, (S, Dch))
    y = np.empty((S, Dch), dtype=np.float64)
    rc = _load().ssm_oracle_step(S, Dch, N, _ptr(st), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                                 int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle step rejected N=%d" % N)
    return y, st


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus: bool = True, h0=None,
             dlast=None, threads: Optional[int] = None, exact_zoh: bool = False) -> dict:
    """fp64 gradients of the scan (from h0, or zero; with the exact-ZOH input term if asked)
    given dy = dLoss/dy and dlast = dLoss/d(last_state).  Returns a dict with du, ddelta
    (w.r.t. the delta input), dA, dB, dC, and dD, dz, ddelta_bias, dh0 for the optional
    inputs that are given."""
    u = _f64(u)
    bsz, L, Dch = u.shape
    A = _f64(A)
    N = A.shape[1]
    args = dict(delta=_f64(delta, (bsz, L, Dch)), B=_f64(B, (bsz, L, N)), C=_f64(C, (bsz, L, N)),
                D=_f64(D, (Dch,)), z=_f64(z, (bsz, L, Dch)), delta_bias=_f64(delta_bias, (Dch,)),
                h0=_f64(h0, (bsz, Dch, N)), dy=_f64(dy, (bsz, L, Dch)), dlast=_f64(dlast, (bsz, Dch, N)))
    out = dict(du=np.empty((bsz, L, Dch)), ddelta=np.empty((bsz, L, Dch)), dA=np.empty((Dch, N)),
               dB=np.empty((bsz, L, N)), dC=np.empty((bsz, L, N)))
    if D is not None:
        out["dD"] = np.empty(Dch)
    if z is not None:
        out["dz"] = np.empty((bsz, L, Dch))
    if delta_bias is not None:
        out["ddelta_bias"] = np.empty(Dch)
    if h0 is not None:
        out["dh0"] = np.empty((bsz, Dch, N))
    rc = _load().ssm_oracle_scan_bwd(
        bsz, L, Dch, N, _ptr(args["h0"]), _ptr(u), _ptr(args["delta"]), _ptr(A), _ptr(args["B"]), _ptr(args["C"]),
        _ptr(args["D"]), _ptr(args["z"]), _ptr(args["delta_bias"]), int(bool(softplus)) | (2 if exact_zoh else 0),
        _ptr(args["dy"]),
        _ptr(args["dlast"]), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
        _ptr(out["dC"]), _ptr(out.get("dD")), _ptr(out.get("dz")), _ptr(out.get("ddelta_bias")),
        _ptr(out.get("dh0")), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle backward failed (N=%d)" % N)
    return out


def scan_case(case, channels=None, threads: Optional[int] = None, h0=None, exact_zoh: bool = False):
    """Run the oracle on a generated ScanCase (from the package's input module).

    channels: optional index array of channels d to evaluate (all batches); the oracle
    then runs on those channel columns only -- channels are independent, so each
    sampled output is exactly the full-problem value.  h0: optional initial state
    (bsz, Dch, N) of the whole problem.  exact_zoh: the exact zero-order-hold input term.
    Returns (y, last_state) restricted to the sampled channels.
    """
    sel = slice(None) if channels is None else np.asarray(channels)
    u = case.values("u")[:, :, sel]
    dl = case.values("delta")[:, :, sel]
    z = case.values("z")
    z = None if z is None else z[:, :, sel]
    A = case.A[sel]
    D = None if case.Dskip is None else case.Dskip[sel]
    bias = None if case.delta_bias is None else case.delta_bias[sel]
    if h0 is not None:
        h0 = np.asarray(h0)[:, sel]
    return scan(u, dl, A, case.values("B"), case.values("C"), D=D, z=z, delta_bias=bias,
                softplus=case.softplus, threads=threads, h0=h0, exact_zoh=exact_zoh)


def conv1d(x, w, bias=None, state=None, silu: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 causal depthwise convolution over time, then SiLU (if silu).

    x: (bsz, L, Dch); w: (Dch, width), tap k multiplying x[t - (width-1) + k]; bias: (Dch,);
    state: (bsz, width-1, Dch), the inputs before token 0 (None = zeros).
    Returns (out (bsz, L, Dch), state_out (bsz, width-1, Dch)), both float64.
    """
    x = _f64(x)
    bsz, L, Dch = x.shape
    w = _f64(w)
    width = w.shape[1]
    w = _f64(w, (Dch, width))
    bias = _f64(bias, (Dch,))
    state = _f64(state, (bsz, width - 1, Dch))
    out = np.empty((bsz, L, Dch), dtype=np.float64)
    st = np.empty((bsz, width - 1, Dch), dtype=np.float64)
    rc = _load().ssm_oracle_conv1d(bsz, L, Dch, width, _ptr(x), _ptr(w), _ptr(bias), _ptr(state), int(bool(silu)),
                                   _ptr(out), _ptr(st))
    if rc != 0:
        raise ValueError("oracle conv1d rejected width=%d" % width)
    return out, st


def conv1d_bwd(x, w, dout, bias=None, state=None, silu: bool = True) -> dict:
    """fp64 gradients of conv1d given dout = dLoss/dout (state_out carries none).

    Returns a dict with dx (bsz, L, Dch), dw (Dch, width), and dbias (Dch,) and dstate
    (bsz, width-1, Dch) when bias / state are given (dstate: the gradient with respect to
    the inputs before token 0, also when they are the implicit zeros -- pass a zero state).
    """
    x = _f64(x)
    bsz, L, Dch = x.shape
    w = _f64(w)
    width = w.shape[1]
    w = _f64(w, (Dch, width))
    bias = _f64(bias, (Dch,))
    state = _f64(state, (bsz, width - 1, Dch))
    dout = _f64(dout, (bsz, L, Dch))
    out = dict(dx=np.empty((bsz, L, Dch)), dw=np.empty((Dch, width)))
    if bias is not None:
        out["dbias"] = np.empty(Dch)
    if state is not None:
        out["dstate"] = np.empty((bsz, width - 1, Dch))
    rc = _load().ssm_oracle_conv1d_bwd(bsz, L, Dch, width, _ptr(x), _ptr(w), _ptr(bias), _ptr(state),
                                       int(bool(silu)), _ptr(dout), _ptr(out["dx"]), _ptr(out["dw"]),
                                       _ptr(out.get("dbias")), _ptr(out.get("dstate")))
    if rc != 0:
        raise ValueError("oracle conv1d_bwd rejected width=%d" % width)
    return out


def ssd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus: bool = True, h0=None,
        threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 Mamba-2 SSD layer.  x, z: (bsz, L, H, P); dt: (bsz, L, H); A, D, dt_bias: (H,);
    B, C: (bsz, L, G, N); h0: (bsz, H, P, N).  Returns (y (bsz, L, H, P), last_state
    (bsz, H, P, N)), float64."""
    x = _f64(x)
    bsz, L, H, P = x.shape
    B = _f64(B)
    G, N = B.shape[2], B.shape[3]
    B = _f64(B, (bsz, L, G, N))
    C = _f64(C, (bsz, L, G, N))
    dt = _f64(dt, (bsz, L, H))
    A = _f64(A, (H,))
    D = _f64(D, (H,))
    z = _f64(z, (bsz, L, H, P))
    dt_bias = _f64(dt_bias, (H,))
    h0 = _f64(h0, (bsz, H, P, N))
    y = np.empty((bsz, L, H, P), dtype=np.float64)
    last = np.empty((bsz, H, P, N), dtype=np.float64)
    rc = _load().ssm_oracle_ssd(bsz, L, H, P, G, N, _ptr(h0), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(z), _ptr(dt_bias), int(bool(softplus)), _ptr(y), _ptr(last),
                                int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle ssd rejected N=%d G=%d H=%d" % (N, G, H))
    return y, last

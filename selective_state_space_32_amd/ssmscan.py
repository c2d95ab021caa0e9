"""Thin ctypes binding of libssmscan.so taking torch tensors.

Argument marshalling only: shapes and dtypes are checked, outputs and the workspace are
allocated with torch on the tensors' device, and the C entry points (include/ssmscan.h)
are called on torch's current stream.  Every step of the computation runs in the HIP
kernels of libssmscan.so; if the library is missing this module raises on import.
"""
from __future__ import annotations

import ctypes
import os
from typing import Callable, Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SSMSCAN_LIBRARY may name another build of the same library (the sanitized host build)
LIBPATH = os.environ.get("SSMSCAN_LIBRARY") or os.path.join(_PKG, "libssmscan.so")

SSM_IO_F32 = 0
SSM_IO_BF16 = 1

STATUS = {0: "SSM_OK", -1: "SSM_ERR_NULL", -2: "SSM_ERR_SHAPE", -3: "SSM_ERR_DTYPE", -4: "SSM_ERR_ALIGN",
          -5: "SSM_ERR_UNSUPPORTED_N", -6: "SSM_ERR_WORKSPACE", -7: "SSM_ERR_HIP", -8: "SSM_ERR_FLAGS"}


class ssm_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("chunk_len", ctypes.c_int32)]


class ssm_ssd_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ssm_plan_info(ctypes.Structure):
    _fields_ = [("cu_count", ctypes.c_int32), ("nchunk", ctypes.c_int64), ("chunk_len", ctypes.c_int64),
                ("split_tiles", ctypes.c_int64), ("split_at", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t)]


class SSMError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBPATH):
        raise ImportError(f"{LIBPATH} is not built; run `python -m selective_state_space_32_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIBPATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(ssm_dims)
    lib.ssm_version.restype = ctypes.c_int
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_scan_workspace_bytes.argtypes = [D]
    lib.ssm_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_scan_plan.argtypes = [D, ctypes.POINTER(ctypes.c_int64)]
    lib.ssm_scan_plan.restype = ctypes.c_int64
    lib.ssm_scan_plan_info.argtypes = [D, ctypes.c_int, ctypes.POINTER(ssm_plan_info)]
    lib.ssm_scan_plan_info.restype = ctypes.c_int
    lib.ssm_scan_fwd.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, P, P, D, P, ctypes.c_size_t, P]
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_fwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_int, P, P, D, P, ctypes.c_size_t, P]
    lib.ssm_scan_fwd_varlen.restype = ctypes.c_int
    lib.ssm_scan_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, P, P, D, P]
    lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssm_scan_fwd_from.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_int, P, P, D, P, ctypes.c_size_t, P]
    lib.ssm_scan_fwd_from.restype = ctypes.c_int
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [D]
    lib.ssm_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_scan_bwd.argtypes = [P] * 9 + [ctypes.c_int] + [P] * 11 + [D, P, ctypes.c_size_t, P]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_scan_bwd_varlen.argtypes = [P, P] + [P] * 8 + [ctypes.c_int] + [P] * 11 + [D, P, ctypes.c_size_t, P]
    lib.ssm_scan_bwd_varlen.restype = ctypes.c_int
    lib.ssm_step.argtypes = [P, P, P, P, P, P, P, P, P, D, P]
    lib.ssm_step.restype = ctypes.c_int
    lib.ssm_step_act.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_int, P, D, P]
    lib.ssm_step_act.restype = ctypes.c_int
    lib.ssm_conv1d_fwd.argtypes = [P, P, P, ctypes.c_int, P, ctypes.c_int, P, P, D, P]
    lib.ssm_conv1d_fwd.restype = ctypes.c_int
    lib.ssm_conv1d_bwd.argtypes = [P, P, P, ctypes.c_int, P, ctypes.c_int, P, P, P, P, P, D, P]
    lib.ssm_conv1d_bwd.restype = ctypes.c_int
    lib.ssm_scan_fwd_conv.argtypes = [P, P, P, ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_int, P, P, P, D, P,
                                      ctypes.c_size_t, P]
    lib.ssm_scan_fwd_conv.restype = ctypes.c_int
    lib.ssm_ssd_fwd.argtypes = [P] * 8 + [ctypes.c_int, P, P, ctypes.POINTER(ssm_ssd_dims), P]
    lib.ssm_ssd_fwd.restype = ctypes.c_int
    lib.ssm_ssd_fwd_from.argtypes = [P] * 9 + [ctypes.c_int, P, P, ctypes.POINTER(ssm_ssd_dims), P]
    lib.ssm_ssd_fwd_from.restype = ctypes.c_int
    return lib


lib = _load()


def last_error() -> str:
    return lib.ssm_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise SSMError(rc, last_error())


def _io_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return SSM_IO_F32
    if dt == torch.bfloat16:
        return SSM_IO_BF16
    raise TypeError(f"I/O tensors must be float32 or bfloat16, got {dt}")


def make_dims(batch: int, seqlen: int, dim: int, dstate: int, io_dtype, chunk_len: int = 0) -> ssm_dims:
    code = io_dtype if isinstance(io_dtype, int) else _io_code(io_dtype)
    return ssm_dims(int(batch), int(seqlen), int(dim), int(dstate), int(code), int(chunk_len))


def workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int, io_dtype, chunk_len: int = 0) -> int:
    d = make_dims(batch, seqlen, dim, dstate, io_dtype, chunk_len)
    return int(lib.ssm_scan_workspace_bytes(ctypes.byref(d)))


def bwd_workspace_bytes(batch: int, seqlen: int, dim: int, dstate: int, io_dtype) -> int:
    d = make_dims(batch, seqlen, dim, dstate, io_dtype)
    return int(lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d)))


def scan_plan(batch: int, seqlen: int, dim: int, dstate: int, io_dtype, chunk_len: int = 0) -> Tuple[int, int]:
    """(number of chunks per sequence, chunk length) the library will use."""
    d = make_dims(batch, seqlen, dim, dstate, io_dtype, chunk_len)
    cl = ctypes.c_int64(0)
    n = int(lib.ssm_scan_plan(ctypes.byref(d), ctypes.byref(cl)))
    if n < 0:
        raise SSMError(n, last_error())
    return n, int(cl.value)


def plan_info(batch: int, seqlen: int, dim: int, dstate: int, io_dtype, chunk_len: int = 0,
              cu_count: int = 0) -> dict:
    """The scan's schedule on a device with cu_count CUs (0: the current device), as a dict of
    the ssm_plan_info fields."""
    d = make_dims(batch, seqlen, dim, dstate, io_dtype, chunk_len)
    out = ssm_plan_info()
    _check(lib.ssm_scan_plan_info(ctypes.byref(d), int(cu_count), ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in ssm_plan_info._fields_}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream_handle(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


SCAN_SOFTPLUS = 1      # flag bits of the scan entry points (include/ssmscan.h)
SCAN_EXACT_ZOH = 2
SCAN_CHECKPOINTS = 4


def _scan_args(u, delta, A, B, C, D, z, delta_bias, softplus, y, last_state, return_last_state, chunk_len,
               workspace, stream, initial_state=None, exact_zoh=False, save_checkpoints=False):
    if u.dim() != 3:
        raise ValueError("u must be (batch, L, dim)")
    bsz, L, dim = u.shape
    N = A.shape[-1]
    dev, io = u.device, u.dtype
    _io_code(io)
    _need(u, "u", (bsz, L, dim), io, dev)
    _need(delta, "delta", (bsz, L, dim), io, dev)
    _need(A, "A", (dim, N), torch.float32, dev)
    _need(B, "B", (bsz, L, N), io, dev)
    _need(C, "C", (bsz, L, N), io, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (bsz, L, dim), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if y is None:
        y = torch.empty((bsz, L, dim), dtype=io, device=dev)
    else:
        _need(y, "y", (bsz, L, dim), io, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", (bsz, dim, N), torch.float32, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((bsz, dim, N), dtype=torch.float32, device=dev)
    elif last_state is not None:
        _need(last_state, "last_state", (bsz, dim, N), torch.float32, dev)
    dims = make_dims(bsz, L, dim, N, io, chunk_len)
    need = int(lib.ssm_scan_workspace_bytes(ctypes.byref(dims)))
    if save_checkpoints:   # the backward pass's checkpoints first, then the plan's carry area
        need += int(lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            (SCAN_SOFTPLUS if softplus else 0) | (SCAN_EXACT_ZOH if exact_zoh else 0) |
            (SCAN_CHECKPOINTS if save_checkpoints else 0), _ptr(y),
            _ptr(last_state), ctypes.byref(dims), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if initial_state is not None:
        args = (_ptr(initial_state),) + args
    # the tensors and the dims struct the pointers refer to, kept alive with the arguments
    keep = (u, delta, A, B, C, D, z, delta_bias, y, last_state, workspace, dims, initial_state)
    return args, keep, y, last_state, workspace


def scan_fwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
             delta_bias: Optional[torch.Tensor] = None, softplus: bool = True, *,
             y: Optional[torch.Tensor] = None, last_state: Optional[torch.Tensor] = None,
             return_last_state: bool = True, chunk_len: int = 0,
             workspace: Optional[torch.Tensor] = None, stream=None, exact_zoh: bool = False,
             save_checkpoints: bool = False):
    """Selective scan forward from a zero state (ssm_scan_fwd).

    u, delta, z: (batch, L, dim); B, C: (batch, L, N), all of one dtype (float32 or bfloat16);
    A: (dim, N) float32; D, delta_bias: (dim,) float32 or None.  exact_zoh: the exact
    zero-order-hold input term (exp(delta A) - 1) / A * B * u instead of delta * B * u.
    Returns (y, last_state) -- last_state (batch, dim, N) float32, or None if not asked for.
    save_checkpoints (a training forward): also store the states the backward pass needs in
    the workspace and return (y, last_state, workspace); pass that workspace to scan_bwd as
    `checkpoints` to skip its recompute pass.
    """
    args, _keep, y, last_state, ws = _scan_args(u, delta, A, B, C, D, z, delta_bias, softplus, y, last_state,
                                                return_last_state, chunk_len, workspace, stream,
                                                exact_zoh=exact_zoh, save_checkpoints=save_checkpoints)
    _check(lib.ssm_scan_fwd(*args))
    return (y, last_state, ws) if save_checkpoints else (y, last_state)


def scan_fwd_noalloc(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                     D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                     delta_bias: Optional[torch.Tensor] = None, softplus: bool = True, *,
                     y: torch.Tensor, last_state: Optional[torch.Tensor] = None, chunk_len: int = 0,
                     stream=None, exact_zoh: bool = False):
    """ssm_scan_fwd_noalloc: the scan of scan_fwd with the library's own device scratch.  Nothing
    is allocated here or in the library: y (and last_state, if wanted) are given by the caller.
    Returns (y, last_state)."""
    if u.dim() != 3:
        raise ValueError("u must be (batch, L, dim)")
    bsz, L, dim = u.shape
    N = A.shape[-1]
    dev, io = u.device, u.dtype
    _io_code(io)
    for t, name, shape, dt in ((u, "u", (bsz, L, dim), io), (delta, "delta", (bsz, L, dim), io),
                               (A, "A", (dim, N), torch.float32), (B, "B", (bsz, L, N), io),
                               (C, "C", (bsz, L, N), io), (y, "y", (bsz, L, dim), io)):
        _need(t, name, shape, dt, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (bsz, L, dim), io, dev)
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if last_state is not None:
        _need(last_state, "last_state", (bsz, dim, N), torch.float32, dev)
    dims = make_dims(bsz, L, dim, N, io, chunk_len)
    _check(lib.ssm_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                    _ptr(delta_bias),
                                    (SCAN_SOFTPLUS if softplus else 0) | (SCAN_EXACT_ZOH if exact_zoh else 0),
                                    _ptr(y), _ptr(last_state), ctypes.byref(dims), _stream_handle(stream)))
    return y, last_state


def scan_fwd_call(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                  D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                  delta_bias: Optional[torch.Tensor] = None, softplus: bool = True, *,
                  y: Optional[torch.Tensor] = None, last_state: Optional[torch.Tensor] = None,
                  return_last_state: bool = True, chunk_len: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  exact_zoh: bool = False, save_checkpoints: bool = False) -> Callable[[], None]:
    """The scan_fwd call checked and marshalled once: returns a function that enqueues the
    same call again (same tensors, the stream given or current now), for loops that repeat
    it.  Outputs go to the y / last_state tensors passed in (or allocated here and kept);
    with save_checkpoints, the checkpoints go to `workspace` (which must then be given)."""
    if save_checkpoints and workspace is None:
        raise ValueError("save_checkpoints needs the workspace that scan_bwd will read")
    args, keep, _y, _ls, _ws = _scan_args(u, delta, A, B, C, D, z, delta_bias, softplus, y, last_state,
                                          return_last_state, chunk_len, workspace, stream, exact_zoh=exact_zoh,
                                          save_checkpoints=save_checkpoints)

    def call(_args=args, _keep=keep):
        _check(lib.ssm_scan_fwd(*_args))
    return call


def scan_fwd_from(initial_state: torch.Tensor, u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                  B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                  z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                  softplus: bool = True, *, y: Optional[torch.Tensor] = None,
                  last_state: Optional[torch.Tensor] = None, return_last_state: bool = True,
                  chunk_len: int = 0, workspace: Optional[torch.Tensor] = None, stream=None,
                  exact_zoh: bool = False, save_checkpoints: bool = False):
    """The scan continued from initial_state (batch, dim, N) float32 (ssm_scan_fwd_from).
    last_state may be initial_state itself (the state advanced in place).  Otherwise as
    scan_fwd."""
    args, _keep, y, last_state, ws = _scan_args(u, delta, A, B, C, D, z, delta_bias, softplus, y, last_state,
                                                return_last_state, chunk_len, workspace, stream, initial_state,
                                                exact_zoh=exact_zoh, save_checkpoints=save_checkpoints)
    _check(lib.ssm_scan_fwd_from(*args))
    return (y, last_state, ws) if save_checkpoints else (y, last_state)


def scan_fwd_varlen(seq_lens: torch.Tensor, u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                    B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                    z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                    softplus: bool = True, *, initial_state: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None, last_state: Optional[torch.Tensor] = None,
                    return_last_state: bool = True, chunk_len: int = 0, workspace: Optional[torch.Tensor] = None,
                    stream=None, exact_zoh: bool = False, save_checkpoints: bool = False):
    """Scan of sequences of different lengths (ssm_scan_fwd_varlen): seq_lens (batch,) int32 on
    the device; sequence b's tokens t < seq_lens[b] are scanned (from initial_state, or zero)
    and written to y, the later tokens of y are left as they are.  Returns (y, last_state),
    last_state being the state after each sequence's own length; with save_checkpoints (a
    training forward) also the workspace holding the backward's checkpoints, for
    scan_bwd(..., seq_lens=..., checkpoints=ws)."""
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or seq_lens.shape[0] != u.shape[0]:
        raise ValueError("seq_lens must be an int32 tensor of shape (batch,)")
    if seq_lens.device != u.device:
        raise ValueError("seq_lens must be on the device of u")
    args, _keep, y, last_state, ws = _scan_args(u, delta, A, B, C, D, z, delta_bias, softplus, y, last_state,
                                                return_last_state, chunk_len, workspace, stream,
                                                initial_state=initial_state, exact_zoh=exact_zoh,
                                                save_checkpoints=save_checkpoints)
    if initial_state is None:
        args = (None,) + args
    _check(lib.ssm_scan_fwd_varlen(args[0], _ptr(seq_lens), *args[1:]))
    return (y, last_state, ws) if save_checkpoints else (y, last_state)


def scan_bwd(dy: torch.Tensor, u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
             C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
             delta_bias: Optional[torch.Tensor] = None, softplus: bool = True, *,
             initial_state: Optional[torch.Tensor] = None, dlast_state: Optional[torch.Tensor] = None,
             want_initial_state_grad: bool = False, workspace: Optional[torch.Tensor] = None,
             out: Optional[dict] = None, stream=None, checkpoints: Optional[torch.Tensor] = None,
             exact_zoh: bool = False, seq_lens: Optional[torch.Tensor] = None) -> dict:
    """Gradients of the scan (ssm_scan_bwd; of the exact zero-order-hold scan with exact_zoh;
    of scan_fwd_varlen with seq_lens, an int32 (batch,) tensor on the device: ssm_scan_bwd_varlen)
    given dy (batch, L, dim) and optionally
    dlast_state (batch, dim, N).  The forward inputs are passed as to scan_fwd / scan_fwd_from.
    Returns a dict: du, ddelta, dz (if z), dA, dB, dC (float32), dD (if D), ddelta_bias
    (if delta_bias), dinitial_state (if asked for).  `out`: such a dict from an earlier call
    with the same shapes, whose tensors are written again instead of new ones.
    `checkpoints`: the workspace a scan_fwd(..., save_checkpoints=True) call on the same
    inputs returned; its checkpoints are used instead of a recompute pass."""
    if checkpoints is not None:
        if workspace is not None:
            raise ValueError("give either workspace or checkpoints")
        workspace = checkpoints
    if u.dim() != 3:
        raise ValueError("u must be (batch, L, dim)")
    bsz, L, dim = u.shape
    N = A.shape[-1]
    dev, io = u.device, u.dtype
    _io_code(io)
    for t, name, shape, dt in ((u, "u", (bsz, L, dim), io), (delta, "delta", (bsz, L, dim), io),
                               (A, "A", (dim, N), torch.float32), (B, "B", (bsz, L, N), io),
                               (C, "C", (bsz, L, N), io), (dy, "dy", (bsz, L, dim), io)):
        _need(t, name, shape, dt, dev)
    for t, name, shape, dt in ((D, "D", (dim,), torch.float32), (z, "z", (bsz, L, dim), io),
                               (delta_bias, "delta_bias", (dim,), torch.float32),
                               (initial_state, "initial_state", (bsz, dim, N), torch.float32),
                               (dlast_state, "dlast_state", (bsz, dim, N), torch.float32)):
        if t is not None:
            _need(t, name, shape, dt, dev)
    if out is not None:
        g = out
    else:
        g = _bwd_outputs(bsz, L, dim, N, io, dev, z is not None, D is not None, delta_bias is not None,
                         want_initial_state_grad)
    dims = make_dims(bsz, L, dim, N, io)
    need = int(lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(dims)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(softplus)) | (SCAN_CHECKPOINTS if checkpoints is not None else 0)
            | (SCAN_EXACT_ZOH if exact_zoh else 0),
            _ptr(dy), _ptr(dlast_state), _ptr(g["du"]),
            _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")),
            _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")), _ptr(g.get("dinitial_state")),
            ctypes.byref(dims), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_handle(stream))
    if seq_lens is not None:
        if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or seq_lens.shape[0] != bsz:
            raise ValueError("seq_lens must be an int32 tensor of shape (batch,)")
        if seq_lens.device != dev:
            raise ValueError("seq_lens must be on the device of u")
        rc = lib.ssm_scan_bwd_varlen(_ptr(initial_state), _ptr(seq_lens), *args)
    else:
        rc = lib.ssm_scan_bwd(_ptr(initial_state), *args)
    _check(rc)
    return g


def _bwd_outputs(bsz, L, dim, N, io, dev, gate, skip, bias, want_h0):
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(du=torch.empty((bsz, L, dim), dtype=io, device=dev), ddelta=torch.empty((bsz, L, dim), dtype=io, device=dev),
             dA=torch.empty((dim, N), **f32), dB=torch.empty((bsz, L, N), **f32), dC=torch.empty((bsz, L, N), **f32))
    if gate:
        g["dz"] = torch.empty((bsz, L, dim), dtype=io, device=dev)
    if skip:
        g["dD"] = torch.empty((dim,), **f32)
    if bias:
        g["ddelta_bias"] = torch.empty((dim,), **f32)
    if want_h0:
        g["dinitial_state"] = torch.empty((bsz, dim, N), **f32)
    return g


def _step_args(state, u, delta, A, B, C, D, z, y, stream, act=None):
    """Arguments of ssm_step, or (act = (delta_bias, flags)) of ssm_step_act."""
    S, dim, N = state.shape
    dev, io = u.device, u.dtype
    _io_code(io)
    _need(state, "state", (S, dim, N), torch.float32, dev)
    _need(u, "u", (S, dim), io, dev)
    _need(delta, "delta", (S, dim), io, dev)
    _need(A, "A", (dim, N), torch.float32, dev)
    _need(B, "B", (S, N), io, dev)
    _need(C, "C", (S, N), io, dev)
    if D is not None:
        _need(D, "D", (dim,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (S, dim), io, dev)
    if y is None:
        y = torch.empty((S, dim), dtype=io, device=dev)
    else:
        _need(y, "y", (S, dim), io, dev)
    dims = make_dims(S, 1, dim, N, io)
    if act is None:
        args = (_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                ctypes.byref(dims), _stream_handle(stream))
        keep = (state, u, delta, A, B, C, D, z, y, dims)
    else:
        bias, flags = act
        if bias is not None:
            _need(bias, "delta_bias", (dim,), torch.float32, dev)
        args = (_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(bias),
                int(flags), _ptr(y), ctypes.byref(dims), _stream_handle(stream))
        keep = (state, u, delta, A, B, C, D, z, bias, y, dims)
    return args, keep, y


def step(state: torch.Tensor, u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
         C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None, *,
         delta_bias: Optional[torch.Tensor] = None, softplus: bool = False, exact_zoh: bool = False,
         y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One recurrent step; `state` (S, dim, N) float32 is updated in place.

    u, delta, z: (S, dim); B, C: (S, N) of one dtype.  Without delta_bias, softplus and
    exact_zoh, delta is the activated step size (ssm_step); with any of them delta is the raw
    input and the step size and input term are formed as the scan forms them (ssm_step_act).
    Returns y (S, dim)."""
    if delta_bias is None and not softplus and not exact_zoh:
        args, _keep, y = _step_args(state, u, delta, A, B, C, D, z, y, stream)
        _check(lib.ssm_step(*args))
        return y
    flags = (SCAN_SOFTPLUS if softplus else 0) | (SCAN_EXACT_ZOH if exact_zoh else 0)
    args, _keep, y = _step_args(state, u, delta, A, B, C, D, z, y, stream, act=(delta_bias, flags))
    _check(lib.ssm_step_act(*args))
    return y


def step_call(state: torch.Tensor, u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
              C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None, *,
              y: Optional[torch.Tensor] = None, stream=None) -> Callable[[], None]:
    """The step call checked and marshalled once (see scan_fwd_call)."""
    args, keep, _y = _step_args(state, u, delta, A, B, C, D, z, y, stream)

    def call(_args=args, _keep=keep):
        _check(lib.ssm_step(*_args))
    return call


CONV_SILU = 1   # flag bit of ssm_conv1d_fwd (include/ssmscan.h)


def _conv_args(x, w, bias, state, silu, out, state_out, return_state, stream):
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, dim)")
    bsz, L, dim = x.shape
    if w.dim() != 2 or w.shape[0] != dim:
        raise ValueError("w must be (dim, width)")
    width = int(w.shape[1])
    dev, io = x.device, x.dtype
    _io_code(io)
    _need(w, "w", (dim, width), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (dim,), torch.float32, dev)
    if state is not None:
        _need(state, "state", (bsz, width - 1, dim), io, dev)
    if out is None:
        out = torch.empty((bsz, L, dim), dtype=io, device=dev)
    else:
        _need(out, "out", (bsz, L, dim), io, dev)
    if state_out is None and return_state:
        state_out = torch.empty((bsz, width - 1, dim), dtype=io, device=dev)
    elif state_out is not None:
        _need(state_out, "state_out", (bsz, width - 1, dim), io, dev)
    dims = make_dims(bsz, L, dim, 1, io)
    args = (_ptr(x), _ptr(w), _ptr(bias), width, _ptr(state), CONV_SILU if silu else 0, _ptr(out), _ptr(state_out),
            ctypes.byref(dims), _stream_handle(stream))
    keep = (x, w, bias, state, out, state_out, dims)
    return args, keep, out, state_out


def conv1d(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
           state: Optional[torch.Tensor] = None, silu: bool = True, *, out: Optional[torch.Tensor] = None,
           state_out: Optional[torch.Tensor] = None, return_state: bool = True, stream=None):
    """Causal depthwise convolution over time, then SiLU (ssm_conv1d_fwd).

    x: (batch, L, dim) float32 or bfloat16; w: (dim, width) float32, width 1..4; bias: (dim,)
    float32; state: (batch, width-1, dim) of x's dtype, the inputs before token 0 (None = zeros).
    Returns (out (batch, L, dim), state_out (batch, width-1, dim) or None); state_out may be
    `state` itself (advanced in place)."""
    args, _keep, out, state_out = _conv_args(x, w, bias, state, silu, out, state_out, return_state, stream)
    _check(lib.ssm_conv1d_fwd(*args))
    return out, state_out


def conv1d_call(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
                state: Optional[torch.Tensor] = None, silu: bool = True, *, out: Optional[torch.Tensor] = None,
                state_out: Optional[torch.Tensor] = None, return_state: bool = True,
                stream=None) -> Callable[[], None]:
    """The conv1d call checked and marshalled once (see scan_fwd_call)."""
    args, keep, _o, _s = _conv_args(x, w, bias, state, silu, out, state_out, return_state, stream)

    def call(_args=args, _keep=keep):
        _check(lib.ssm_conv1d_fwd(*_args))
    return call


def _conv_bwd_args(dout, x, w, bias, state, silu, want_state_grad, dx, stream):
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, dim)")
    bsz, L, dim = x.shape
    if w.dim() != 2 or w.shape[0] != dim:
        raise ValueError("w must be (dim, width)")
    width = int(w.shape[1])
    dev, io = x.device, x.dtype
    _io_code(io)
    _need(w, "w", (dim, width), torch.float32, dev)
    _need(dout, "dout", (bsz, L, dim), io, dev)
    if bias is not None:
        _need(bias, "bias", (dim,), torch.float32, dev)
    if state is not None:
        _need(state, "state", (bsz, width - 1, dim), io, dev)
    if dx is None:
        dx = torch.empty((bsz, L, dim), dtype=io, device=dev)
    else:
        _need(dx, "dx", (bsz, L, dim), io, dev)
    g = dict(dx=dx, dw=torch.empty((dim, width), dtype=torch.float32, device=dev))
    if bias is not None:
        g["dbias"] = torch.empty((dim,), dtype=torch.float32, device=dev)
    if want_state_grad:
        g["dstate"] = torch.empty((bsz, width - 1, dim), dtype=io, device=dev)
    dims = make_dims(bsz, L, dim, 1, io)
    args = (_ptr(x), _ptr(w), _ptr(bias), width, _ptr(state), CONV_SILU if silu else 0, _ptr(dout), _ptr(dx),
            _ptr(g["dw"]), _ptr(g.get("dbias")), _ptr(g.get("dstate")), ctypes.byref(dims), _stream_handle(stream))
    keep = (x, w, bias, state, dout, g, dims)
    return args, keep, g


def conv1d_bwd(dout: torch.Tensor, x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
               state: Optional[torch.Tensor] = None, silu: bool = True, *, want_state_grad: Optional[bool] = None,
               dx: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of conv1d (ssm_conv1d_bwd) given dout = dLoss/dout.

    The inputs are those of the forward call.  Returns a dict with dx (batch, L, dim) of x's
    dtype, dw (dim, width) float32, dbias (dim,) float32 when bias is given, and dstate
    (batch, width-1, dim) of x's dtype when want_state_grad (default: when state is given)."""
    if want_state_grad is None:
        want_state_grad = state is not None
    args, _keep, g = _conv_bwd_args(dout, x, w, bias, state, silu, want_state_grad, dx, stream)
    _check(lib.ssm_conv1d_bwd(*args))
    return g


def conv1d_bwd_call(dout: torch.Tensor, x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    state: Optional[torch.Tensor] = None, silu: bool = True, *,
                    want_state_grad: Optional[bool] = None, dx: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[Callable[[], None], dict]:
    """The conv1d_bwd call checked and marshalled once (see scan_fwd_call); returns the call
    and the dict of gradient tensors it writes."""
    if want_state_grad is None:
        want_state_grad = state is not None
    args, keep, g = _conv_bwd_args(dout, x, w, bias, state, silu, want_state_grad, dx, stream)

    def call(_args=args, _keep=keep):
        _check(lib.ssm_conv1d_bwd(*_args))
    return call, g


def _scan_conv_args(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, softplus, y, last_state,
                    return_last_state, u_out, chunk_len, workspace, stream, save_checkpoints=False):
    if conv_w.dim() != 2 or conv_w.shape[0] != x.shape[-1]:
        raise ValueError("conv_w must be (dim, width)")
    bsz, L, dim = x.shape
    _need(conv_w, "conv_w", (dim, conv_w.shape[1]), torch.float32, x.device)
    if conv_b is not None:
        _need(conv_b, "conv_b", (dim,), torch.float32, x.device)
    if u_out is not None:
        _need(u_out, "u_out", (bsz, L, dim), x.dtype, x.device)
    args, keep, y, last_state, ws = _scan_args(x, delta, A, B, C, D, z, delta_bias, softplus, y, last_state,
                                               return_last_state, chunk_len, workspace, stream,
                                               save_checkpoints=save_checkpoints)
    # ssm_scan_fwd's arguments with x in place of u, the convolution's before delta, u_out after last_state
    args = (args[0], _ptr(conv_w), _ptr(conv_b), int(conv_w.shape[1])) + args[1:11] + (_ptr(u_out),) + args[11:]
    return args, keep + (conv_w, conv_b, u_out), y, last_state, ws


def scan_fwd_conv(x: torch.Tensor, conv_w: torch.Tensor, conv_b: Optional[torch.Tensor], delta: torch.Tensor,
                  A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                  z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                  softplus: bool = True, *, y: Optional[torch.Tensor] = None,
                  last_state: Optional[torch.Tensor] = None, return_last_state: bool = True,
                  u_out: Optional[torch.Tensor] = None, chunk_len: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None, save_checkpoints: bool = False):
    """Causal convolution (width 4) + SiLU fused into the scan (ssm_scan_fwd_conv): x is the
    block's projected input, conv_w (dim, 4), conv_b (dim,) float32; u_out (optional) receives
    the convolution's output.  Otherwise as scan_fwd (save_checkpoints: also the backward's
    checkpoints, for scan_bwd with u = u_out).  Returns (y, last_state), or
    (y, last_state, workspace) with save_checkpoints."""
    args, _keep, y, last_state, ws = _scan_conv_args(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, softplus,
                                                     y, last_state, return_last_state, u_out, chunk_len, workspace,
                                                     stream, save_checkpoints=save_checkpoints)
    _check(lib.ssm_scan_fwd_conv(*args))
    return (y, last_state, ws) if save_checkpoints else (y, last_state)


def scan_fwd_conv_call(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, *,
                       y=None, last_state=None, return_last_state=True, u_out=None, chunk_len=0, workspace=None,
                       stream=None, save_checkpoints=False) -> Callable[[], None]:
    """The scan_fwd_conv call checked and marshalled once (see scan_fwd_call); with
    save_checkpoints the checkpoints go to `workspace` (which must then be given)."""
    if save_checkpoints and workspace is None:
        raise ValueError("save_checkpoints needs the workspace that scan_bwd will read")
    args, keep, _y, _ls, _ws = _scan_conv_args(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, softplus, y,
                                               last_state, return_last_state, u_out, chunk_len, workspace, stream,
                                               save_checkpoints=save_checkpoints)

    def call(_args=args, _keep=keep):
        _check(lib.ssm_scan_fwd_conv(*_args))
    return call


def ssd_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
            D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
            dt_bias: Optional[torch.Tensor] = None, softplus: bool = True, *, y: Optional[torch.Tensor] = None,
            last_state: Optional[torch.Tensor] = None, return_last_state: bool = True,
            initial_state: Optional[torch.Tensor] = None, stream=None):
    """Mamba-2's SSD layer (ssm_ssd_fwd; ssm_ssd_fwd_from with initial_state).  x, z:
    (batch, L, H, P); dt: (batch, L, H); B, C: (batch, L, G, N) -- all bfloat16, or all float32
    (dstate 32 or 64); A, D, dt_bias: (H,) float32; initial_state: (batch, H, P, N) float32 (may
    be last_state).  Returns (y (batch, L, H, P) in x's dtype, last_state (batch, H, P, N) float32
    or None)."""
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    bf = x.dtype
    io = _io_code(bf)
    _need(x, "x", (bsz, L, H, P), bf, dev)
    _need(dt, "dt", (bsz, L, H), bf, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (bsz, L, G, N), bf, dev)
    _need(C, "C", (bsz, L, G, N), bf, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (bsz, L, H, P), bf, dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", (H,), torch.float32, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", (bsz, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty((bsz, L, H, P), dtype=bf, device=dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((bsz, H, P, N), dtype=torch.float32, device=dev)
    dims = ssm_ssd_dims(bsz, L, H, P, G, N, io, 0)
    _check(lib.ssm_ssd_fwd_from(_ptr(initial_state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(z), _ptr(dt_bias), 1 if softplus else 0, _ptr(y), _ptr(last_state),
                                ctypes.byref(dims), _stream_handle(stream)))
    return y, last_state

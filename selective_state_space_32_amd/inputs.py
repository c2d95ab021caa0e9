"""Seeded synthetic inputs for the selective state-space scan and its recurrent step.

This module holds random draws, the value-distribution recipes of the workloads and
dtype rounding (fp32 -> bf16, round-to-nearest-even) -- nothing of the scan's own
arithmetic.  It is the one piece shared by the fp64 oracle's tests and the HIP path:
both receive exactly the arrays built here.

Workloads (shapes, distributions) follow the five synthetic configurations the build
is measured on.  All draws use ``numpy.random.default_rng(seed)`` (PCG64) in this fixed
order: A, D, delta_bias, u, delta_in, B, C, z, state0.  Draws are fp32; tensors whose
I/O dtype is bf16 are then rounded to bf16.  A, D and delta_bias stay fp32 always.

Notation follows the Mamba page (azimuth.plus/paper/mamba, "selection" section):
u is the input x_t, delta the step size, B_t / C_t the input-dependent projections
(one N-vector per token, shared by all channels of a sequence) and A the fixed
diagonal state matrix, here one real value per (channel, state).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "ScanCase", "StepCase", "ConvCase", "SsdCase", "scan_case", "step_case",
    "conv_case", "ssd_case",
    "config_case", "CONFIGS",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN/Inf keep their top half (truncation).  For finite inputs the rounding add cannot
    overflow 32 bits (the largest finite pattern is 0xFF7FFFFF)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    out = (r >> np.uint32(16)).astype(np.uint16)
    bad = ~np.isfinite(x)
    if bad.any():
        out[bad] = (b[bad] >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exact fp32 values they encode."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _io(x: np.ndarray, io: str) -> np.ndarray:
    return bf16_bits(x) if io == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


@dataclasses.dataclass
class ScanCase:
    """Inputs of one scan call.  Layouts (row-major, innermost last):
    u, delta, z: [bsz][L][D]; B, C: [bsz][L][N]; A: [D][N]; D, delta_bias: [D].
    io == "bf16": u, delta, z, B, C hold uint16 bf16 bit patterns; else float32."""
    name: str
    io: str
    bsz: int
    L: int
    D: int
    N: int
    u: np.ndarray
    delta: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    Dskip: Optional[np.ndarray]
    z: Optional[np.ndarray]
    delta_bias: Optional[np.ndarray]
    softplus: bool
    seed: int

    def values(self, field: str) -> Optional[np.ndarray]:
        """The float32 values a tensor holds (exact for bf16 tensors)."""
        a = getattr(self, field)
        if a is None:
            return None
        return bf16_to_f32(a) if a.dtype == np.uint16 else a

    @property
    def chtok(self) -> int:
        return self.bsz * self.L * self.D

    def digest(self) -> str:
        h = hashlib.sha256()
        for f in ("u", "delta", "A", "B", "C", "Dskip", "z", "delta_bias"):
            a = getattr(self, f)
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()[:16]


@dataclasses.dataclass
class StepCase:
    """Inputs of `steps` consecutive single-token steps over S sequences.
    state0: [S][D][N] fp32; u, delta, z: [steps][S][D]; B, C: [steps][S][N] (bf16 bits
    or float32 per io).  delta is already activated (positive step sizes)."""
    name: str
    io: str
    S: int
    D: int
    N: int
    steps: int
    state0: np.ndarray
    u: np.ndarray
    delta: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    Dskip: Optional[np.ndarray]
    z: Optional[np.ndarray]
    seed: int

    def values(self, field: str) -> Optional[np.ndarray]:
        a = getattr(self, field)
        if a is None:
            return None
        return bf16_to_f32(a) if a.dtype == np.uint16 else a


def _draw_A(rng, D, N, a_init):
    if a_init == "s4d":        # A[d, n] = -(n + 1)
        return np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)).copy()
    if a_init == "lognormal":  # A = -exp(N(log 4, 0.5)), sd 0.5
        return (-np.exp(rng.normal(np.log(4.0), 0.5, size=(D, N)))).astype(np.float32)
    raise ValueError(a_init)


def _draw_bias(rng, D, bias):
    if bias is None:
        return None
    if isinstance(bias, (int, float)):
        return np.full(D, float(bias), dtype=np.float32)
    lo, hi = {"wide": (1e-3, 0.1), "long": (1e-3, 0.0166)}[bias]
    # inverse of softplus applied to a uniform target step size: the recipe that
    # makes softplus(bias) ~ U[lo, hi]
    return np.log(np.expm1(rng.uniform(lo, hi, size=D))).astype(np.float32)


def scan_case(bsz: int, L: int, D: int, N: int, io: str = "f32", *, a_init: str = "lognormal",
              bias="wide", delta_scale: float = 0.5, softplus: bool = True, gate: bool = False,
              skip: bool = True, lti: bool = False, seed: int = 0, name: str = "") -> ScanCase:
    """Build one scan input set.

    a_init: "s4d" (A = -(n+1)) or "lognormal" (A = -exp(N(log 4, 0.5))).
    bias:   None, a constant, "wide" (softplus(bias) ~ U[1e-3, 0.1]) or "long"
            (~ U[1e-3, 0.0166], mean step about 0.01).
    delta_in = delta_scale * N(0, 1).  lti=True repeats t=0's delta_in, B and C over t.
    """
    if io not in ("f32", "bf16"):
        raise ValueError(io)
    rng = np.random.default_rng(seed)
    A = _draw_A(rng, D, N, a_init)
    Dskip = rng.standard_normal(D, dtype=np.float32) if skip else None
    delta_bias = _draw_bias(rng, D, bias)
    u = rng.standard_normal((bsz, L, D), dtype=np.float32)
    delta_in = (np.float32(delta_scale) * rng.standard_normal((bsz, L, D), dtype=np.float32))
    Bm = rng.standard_normal((bsz, L, N), dtype=np.float32)
    Cm = rng.standard_normal((bsz, L, N), dtype=np.float32)
    z = rng.standard_normal((bsz, L, D), dtype=np.float32) if gate else None
    if lti:
        delta_in[:] = delta_in[:, :1, :]
        Bm[:] = Bm[:, :1, :]
        Cm[:] = Cm[:, :1, :]
    return ScanCase(name=name or f"scan_b{bsz}_l{L}_d{D}_n{N}_{io}", io=io, bsz=bsz, L=L, D=D, N=N,
                    u=_io(u, io), delta=_io(delta_in, io), A=A, B=_io(Bm, io), C=_io(Cm, io),
                    Dskip=Dskip, z=None if z is None else _io(z, io), delta_bias=delta_bias,
                    softplus=softplus, seed=seed)


def step_case(S: int, D: int, N: int, steps: int, io: str = "bf16", *, gate: bool = True,
              skip: bool = True, state_sd: float = 0.1, seed: int = 5, name: str = "") -> StepCase:
    """Build `steps` consecutive single-token step inputs over S independent sequences.

    A, D and the step-size bias follow the B8/L2048/D5120 layer recipe; the per-step
    step size is the activated value softplus(0.5 N(0,1) + bias) (computed here in fp32
    with numpy's logaddexp as the distribution recipe, then rounded to the I/O dtype).
    """
    rng = np.random.default_rng(seed)
    A = _draw_A(rng, D, N, "lognormal")
    Dskip = rng.standard_normal(D, dtype=np.float32) if skip else None
    bias = _draw_bias(rng, D, "wide")
    u = rng.standard_normal((steps, S, D), dtype=np.float32)
    x = np.float32(0.5) * rng.standard_normal((steps, S, D), dtype=np.float32) + bias
    delta = np.logaddexp(np.float32(0.0), x).astype(np.float32)
    Bm = rng.standard_normal((steps, S, N), dtype=np.float32)
    Cm = rng.standard_normal((steps, S, N), dtype=np.float32)
    z = rng.standard_normal((steps, S, D), dtype=np.float32) if gate else None
    state0 = (np.float32(state_sd) * rng.standard_normal((S, D, N), dtype=np.float32))
    return StepCase(name=name or f"step_s{S}_d{D}_n{N}_x{steps}_{io}", io=io, S=S, D=D, N=N,
                    steps=steps, state0=state0, u=_io(u, io), delta=_io(delta, io), A=A,
                    B=_io(Bm, io), C=_io(Cm, io), Dskip=Dskip,
                    z=None if z is None else _io(z, io), seed=seed)


@dataclasses.dataclass
class ConvCase:
    """Inputs of one causal depthwise convolution call.  x: [bsz][L][D] (io); w: [D][width]
    fp32; bias: [D] fp32; state: [bsz][width-1][D] (io) or None."""
    name: str
    io: str
    bsz: int
    L: int
    D: int
    width: int
    x: np.ndarray
    w: np.ndarray
    bias: Optional[np.ndarray]
    state: Optional[np.ndarray]
    seed: int

    def values(self, field: str) -> Optional[np.ndarray]:
        a = getattr(self, field)
        if a is None:
            return None
        return bf16_to_f32(a) if a.dtype == np.uint16 else a


def conv_case(bsz: int, L: int, D: int, width: int = 4, io: str = "bf16", *, bias: bool = True,
              state: bool = False, seed: int = 0, name: str = "conv") -> ConvCase:
    """Draw order w, bias, x, state.  w and bias ~ U(-1/sqrt(width), 1/sqrt(width)) (the
    default uniform initialisation of a depthwise convolution, fan-in = width); x ~ N(0, 1)
    (the projected block input); state ~ N(0, 1) rows of earlier inputs."""
    rng = np.random.default_rng(seed)
    lim = 1.0 / np.sqrt(width)
    w = rng.uniform(-lim, lim, (D, width)).astype(np.float32)
    b = rng.uniform(-lim, lim, D).astype(np.float32) if bias else None
    x = _io(rng.standard_normal((bsz, L, D), dtype=np.float32), io)
    st = _io(rng.standard_normal((bsz, width - 1, D), dtype=np.float32), io) if state else None
    return ConvCase(name, io, bsz, L, D, width, x, w, b, st, seed)


@dataclasses.dataclass
class SsdCase:
    """Inputs of one SSD layer call.  x, z: [bsz][L][H][P] bf16 bits; dt: [bsz][L][H] bf16 bits;
    B, C: [bsz][L][G][N] bf16 bits; A, D, dt_bias: [H] fp32."""
    name: str
    bsz: int
    L: int
    H: int
    P: int
    G: int
    N: int
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    Dskip: Optional[np.ndarray]
    z: Optional[np.ndarray]
    dt_bias: Optional[np.ndarray]
    softplus: bool
    seed: int

    def values(self, field: str) -> Optional[np.ndarray]:
        a = getattr(self, field)
        if a is None:
            return None
        return bf16_to_f32(a) if a.dtype == np.uint16 else a

    @property
    def io(self) -> str:
        return "bf16" if self.x.dtype == np.uint16 else "f32"


def ssd_case(bsz: int, L: int, H: int, P: int = 64, G: int = 1, N: int = 64, *, gate: bool = True,
             skip: bool = True, seed: int = 0, name: str = "ssd", io: str = "bf16") -> SsdCase:
    """Draw order A, D, dt_bias, x, dt, B, C, z.  A = -exp(U[log 1, log 16]) per head; dt_bias =
    log(expm1(U[1e-3, 0.1])) (step sizes between 1e-3 and 0.1 at dt = 0); dt ~ 0.5 N(0, 1);
    x, B, C, z ~ N(0, 1); D ~ N(0, 1).  io "bf16": x, dt, B, C, z are the RNE rounding of the fp32
    draws (bit patterns); "f32": the fp32 draws themselves."""
    cast = bf16_bits if io == "bf16" else (lambda a: np.ascontiguousarray(a, dtype=np.float32))
    rng = np.random.default_rng(seed)
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), H))).astype(np.float32)
    Dskip = rng.standard_normal(H).astype(np.float32) if skip else None
    dt_bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, H))).astype(np.float32)
    x = cast(rng.standard_normal((bsz, L, H, P), dtype=np.float32))
    dt = cast((0.5 * rng.standard_normal((bsz, L, H))).astype(np.float32))
    B = cast(rng.standard_normal((bsz, L, G, N), dtype=np.float32))
    C = cast(rng.standard_normal((bsz, L, G, N), dtype=np.float32))
    z = cast(rng.standard_normal((bsz, L, H, P), dtype=np.float32)) if gate else None
    return SsdCase(name, bsz, L, H, P, G, N, x, dt, A, B, C, Dskip, z, dt_bias, True, seed)


# The five measured workloads (plus the LTI variant of the tiny one).
CONFIGS = {
    "c1": dict(kind="scan", bsz=1, L=256, D=16, N=4, io="f32", a_init="s4d", bias=-1.0,
               delta_scale=1.0, gate=False, seed=1),
    "c1_lti": dict(kind="scan", bsz=1, L=256, D=16, N=4, io="f32", a_init="s4d", bias=-1.0,
                   delta_scale=1.0, gate=False, lti=True, seed=11),
    "c2": dict(kind="scan", bsz=2, L=2048, D=1536, N=16, io="f32", a_init="lognormal",
               bias="wide", gate=False, seed=2),
    "c3": dict(kind="scan", bsz=8, L=2048, D=5120, N=16, io="bf16", a_init="lognormal",
               bias="wide", gate=True, seed=3),
    "c4": dict(kind="scan", bsz=1, L=131072, D=2048, N=16, io="bf16", a_init="lognormal",
               bias="long", gate=False, seed=4),
    "c5": dict(kind="step", S=256, D=5120, N=16, steps=64, io="bf16", gate=True, seed=5),
}

CONFIG_TITLES = {
    "c1": "tiny fp32 scan B1 L256 D16 N4",
    "c1_lti": "tiny fp32 LTI scan B1 L256 D16 N4",
    "c2": "fp32 layer scan B2 L2048 D1536 N16",
    "c3": "bf16 layer scan B8 L2048 D5120 N16 (z gate, last_state)",
    "c4": "bf16 long-context scan B1 L131072 D2048 N16",
    "c5": "bf16 recurrent decode S256 D5120 N16 x64 steps",
}


def config_case(name: str, **override):
    """One of the named workloads; keyword overrides replace recipe fields (e.g. L=...)."""
    spec = dict(CONFIGS[name])
    spec.update(override)
    kind = spec.pop("kind")
    if kind == "step":
        return step_case(name=name, **spec)
    return scan_case(name=name, **spec)

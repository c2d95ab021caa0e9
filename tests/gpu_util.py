"""Helpers for the GPU parity tests: moving generated cases to the device and the
tolerance metrics the outputs are checked with."""
from __future__ import annotations

import numpy as np


def to_dev(a, torch, device="cuda"):
    """numpy array (float32, or uint16 bf16 bit patterns) -> torch tensor on the device."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def case_tensors(case, torch, device="cuda"):
    g = lambda f: to_dev(getattr(case, f), torch, device)
    return dict(u=g("u"), delta=g("delta"), A=g("A"), B=g("B"), C=g("C"), D=g("Dskip"), z=g("z"),
                delta_bias=g("delta_bias"))


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (normal range; 0 for v == 0)."""
    v = np.abs(np.asarray(v, np.float64))
    out = np.zeros_like(v)
    nz = v > 0
    e = np.floor(np.log2(v[nz]))
    e = np.maximum(e, -126.0)
    out[nz] = np.exp2(e - 7.0)
    return out


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def y_error(y_gpu: np.ndarray, y_ref: np.ndarray, io: str) -> float:
    """Error of the GPU output relative to rms(y_ref).

    fp32 outputs: max |y_gpu - y_ref| / rms(y_ref).
    bf16 outputs: the kernel's final rounding to bf16 alone moves a value by up to half a
    bf16 spacing, which for the largest outputs exceeds the tolerance by itself; the error
    before that rounding is measured as max(|y_gpu - y_ref| - ulp(y_gpu)/2) / rms(y_ref)."""
    d = np.abs(y_gpu - y_ref)
    if io == "bf16":
        d = d - 0.5 * bf16_ulp(y_gpu)
    r = rms(y_ref)
    return float(np.max(d)) / r if r > 0 else float(np.max(d))


def bf16_pair_error(a: np.ndarray, b: np.ndarray) -> float:
    """Difference of two bf16 outputs computed from values that agree up to fp32 rounding,
    beyond the rounding of each to bf16: max(|a - b| - ulp(a)/2 - ulp(b)/2) / rms(b)."""
    d = np.abs(a - b) - 0.5 * bf16_ulp(a) - 0.5 * bf16_ulp(b)
    r = rms(b)
    m = float(np.max(d)) if d.size else 0.0
    return max(m, 0.0) / r if r > 0 else max(m, 0.0)


def raw_error(a: np.ndarray, ref: np.ndarray) -> float:
    r = rms(ref)
    d = float(np.max(np.abs(a - ref))) if a.size else 0.0
    return d / r if r > 0 else d


TOL = {"f32": 1e-4, "bf16": 3e-3}

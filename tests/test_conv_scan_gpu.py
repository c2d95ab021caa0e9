"""Parity of the convolution + SiLU fused into the scan (ssm_scan_fwd_conv, through the C
ABI) with the fp64 oracle's convolution followed by its scan, on the same seeded inputs:
y within the scan tolerances (1e-4 rms fp32, 3e-3 rms before the final rounding bf16),
last_state within the same factor, u_out within the convolution's."""
import numpy as np
import pytest

from selective_state_space_32_amd import inputs
from gpu_util import TOL, case_tensors, raw_error, to_dev, to_host_f64, y_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_32_amd import ssmscan  # noqa: E402


def make(bsz, L, D, N, io, seed, gate=True):
    """The scan's inputs from the scan recipe, with the projected block input x in place of u
    and width-4 convolution weights from the convolution recipe."""
    sc = inputs.scan_case(bsz, L, D, N, io, gate=gate, seed=seed)
    cc = inputs.conv_case(bsz, L, D, 4, io, seed=seed + 1)
    return sc, cc


def run_gpu(sc, cc, chunk_len=0, want_u=True):
    t = case_tensors(sc, torch)
    x = to_dev(cc.x, torch)
    u_out = torch.empty_like(x) if want_u else None
    y, ls = ssmscan.scan_fwd_conv(x, torch.from_numpy(cc.w).cuda(), torch.from_numpy(cc.bias).cuda(), t["delta"],
                                  t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                  softplus=sc.softplus, u_out=u_out, chunk_len=chunk_len)
    torch.cuda.synchronize()
    return to_host_f64(y), to_host_f64(ls), (None if u_out is None else to_host_f64(u_out))


def run_oracle(oracle_mod, sc, cc, channels=None):
    sel = slice(None) if channels is None else np.asarray(channels)
    u, _ = oracle_mod.conv1d(cc.values("x")[:, :, sel], cc.w[sel], bias=cc.bias[sel], silu=True)
    zv = sc.values("z")
    y, ls = oracle_mod.scan(u, sc.values("delta")[:, :, sel], sc.A[sel], sc.values("B"), sc.values("C"),
                            D=None if sc.Dskip is None else sc.Dskip[sel], z=None if zv is None else zv[:, :, sel],
                            delta_bias=None if sc.delta_bias is None else sc.delta_bias[sel], softplus=sc.softplus)
    return y, ls, u


def check(sc, got, ref, label):
    y, ls, u = got
    y_ref, ls_ref, u_ref = ref
    tol = TOL[sc.io]
    ey, es = y_error(y, y_ref, sc.io), raw_error(ls, ls_ref)
    eu = y_error(u, u_ref, sc.io) if u is not None else 0.0
    print(f"[conv+scan {label}] y {ey:.3e}  last_state {es:.3e}  u {eu:.3e}  tol {tol}", flush=True)
    assert np.all(np.isfinite(y))
    assert ey <= tol and es <= tol and eu <= tol, (label, ey, es, eu)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("chunk_len", [-1, 64])
def test_conv_scan_small(oracle_mod, io, N, chunk_len):
    """Several tiles, a ragged tail (L = 300) and a ragged channel tile (D = 202); one pass and
    the chunk carry (whose chunks start with rows of the previous chunk in the window)."""
    sc, cc = make(2, 300, 202, N, io, seed=190 + N)
    got = run_gpu(sc, cc, chunk_len=chunk_len)
    check(sc, got, run_oracle(oracle_mod, sc, cc), f"{io} N={N} chunk_len={chunk_len}")


def test_conv_scan_equals_two_calls_fp32():
    """With fp32 I/O the fused call is bitwise the convolution call followed by the scan call
    (the same arithmetic in the same order; u is fp32 either way)."""
    sc, cc = make(2, 500, 256, 16, "f32", seed=200)
    t = case_tensors(sc, torch)
    x = to_dev(cc.x, torch)
    w, b = torch.from_numpy(cc.w).cuda(), torch.from_numpy(cc.bias).cuda()
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=sc.softplus)
    y1, ls1 = ssmscan.scan_fwd_conv(x, w, b, t["delta"], t["A"], t["B"], t["C"], **kw)
    u, _ = ssmscan.conv1d(x, w, b)
    y2, ls2 = ssmscan.scan_fwd(u, t["delta"], t["A"], t["B"], t["C"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(ls1, ls2)


def test_conv_scan_without_u_out_or_gate(oracle_mod):
    sc, cc = make(3, 200, 128, 16, "bf16", seed=201, gate=False)
    got = run_gpu(sc, cc, want_u=False)
    check(sc, got, run_oracle(oracle_mod, sc, cc), "no u_out, no gate")


def test_conv_scan_layer_size_sampled(oracle_mod):
    """B8 L2048 D5120 N16 bf16 with gate (the layer workload, x in place of u), in the
    benchmark's launch configuration: sampled channels against the oracle's convolution and
    scan."""
    sc, cc = make(8, 2048, 5120, 16, "bf16", seed=3)
    got = run_gpu(sc, cc)
    sel = np.unique(np.linspace(0, 5119, 24).astype(np.int64))
    y, ls, u = got
    check(sc, (y[:, :, sel], ls[:, sel], u[:, :, sel]), run_oracle(oracle_mod, sc, cc, sel), "layer, sampled")

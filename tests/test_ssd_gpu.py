"""Parity of Mamba-2's SSD layer on the matrix cores (ssm_ssd_fwd, through the C ABI) with the
fp64 oracle on the same seeded inputs.  The products take bf16 operands (the decay-weighted
matrix M, the weighted B and the state's copy are rounded to bf16), so y is held to the bf16
tolerance of the scan (3e-3 rms before its own final rounding) and the state to 3e-3 rms."""
import numpy as np
import pytest

from selective_state_space_32_amd import inputs
from gpu_util import TOL, raw_error, to_dev, to_host_f64, y_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_32_amd import ssmscan  # noqa: E402


def run_gpu(c):
    dev = lambda a: None if a is None else to_dev(a, torch)   # noqa: E731
    f = lambda a: None if a is None else torch.from_numpy(a).cuda()   # noqa: E731
    y, ls = ssmscan.ssd_fwd(dev(c.x), dev(c.dt), f(c.A), dev(c.B), dev(c.C), D=f(c.Dskip), z=dev(c.z),
                            dt_bias=f(c.dt_bias), softplus=c.softplus)
    torch.cuda.synchronize()
    return to_host_f64(y), to_host_f64(ls)


def run_oracle(oracle_mod, c, heads=None):
    sel = slice(None) if heads is None else np.asarray(heads)
    zv = c.values("z")
    return oracle_mod.ssd(c.values("x")[:, :, sel], c.values("dt")[:, :, sel], c.A[sel], c.values("B"),
                          c.values("C"), D=None if c.Dskip is None else c.Dskip[sel],
                          z=None if zv is None else zv[:, :, sel],
                          dt_bias=None if c.dt_bias is None else c.dt_bias[sel], softplus=c.softplus)


def check(c, y, ls, y_ref, ls_ref, label):
    ey, es = y_error(y, y_ref, "bf16"), raw_error(ls, ls_ref)
    print(f"[ssd {label}] y err/rms {ey:.3e} (raw {raw_error(y, y_ref):.3e})  last_state {es:.3e}  "
          f"tol {TOL['bf16']}", flush=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(ls))
    assert ey <= TOL["bf16"] and es <= TOL["bf16"], (label, ey, es)


@pytest.mark.parametrize("L", [1, 63, 64, 200, 513])
@pytest.mark.parametrize("G", [1, 2])
def test_ssd_small(oracle_mod, L, G):
    """Chunks of 64 with ragged tails, one or two groups of B / C."""
    c = inputs.ssd_case(2, L, 4, G=G, seed=210 + L + G)
    y, ls = run_gpu(c)
    check(c, y, ls, *run_oracle(oracle_mod, c), f"L={L} G={G}")


@pytest.mark.parametrize("gate,skip", [(False, False), (True, False), (False, True)])
def test_ssd_optional_inputs(oracle_mod, gate, skip):
    c = inputs.ssd_case(1, 300, 3, G=3, gate=gate, skip=skip, seed=220)
    y, ls = run_gpu(c)
    check(c, y, ls, *run_oracle(oracle_mod, c), f"gate={gate} skip={skip}")


def test_ssd_layer_size_sampled(oracle_mod):
    """B8 L2048 H80 P64 N64 G1 (model width 5120, the layer size of the scan workloads), in the
    benchmark's launch configuration: sampled heads (all batches, tokens, channels)."""
    c = inputs.ssd_case(8, 2048, 80, G=1, seed=230)
    y, ls = run_gpu(c)
    heads = np.array([0, 17, 41, 79])
    y_ref, ls_ref = run_oracle(oracle_mod, c, heads)
    check(c, y[:, :, heads], ls[:, heads], y_ref, ls_ref, "layer, 4 heads")


def test_ssd_grid_beyond_one_round(oracle_mod):
    """1024 (sequence, head) workgroups -- more than the GPU holds at once -- with four groups of
    B / C and a ragged last chunk; the oracle on sampled heads, each with its own group."""
    c = inputs.ssd_case(4, 130, 256, G=4, seed=232)
    y, ls = run_gpu(c)
    H, G = 256, 4
    for h in (0, 63, 64, 200, 255):
        g = h // (H // G)
        xv, dtv, zv = c.values("x")[:, :, [h]], c.values("dt")[:, :, [h]], c.values("z")
        y_ref, ls_ref = oracle_mod.ssd(xv, dtv, c.A[[h]], c.values("B")[:, :, [g]], c.values("C")[:, :, [g]],
                                       D=None if c.Dskip is None else c.Dskip[[h]],
                                       z=None if zv is None else zv[:, :, [h]],
                                       dt_bias=None if c.dt_bias is None else c.dt_bias[[h]], softplus=c.softplus)
        check(c, y[:, :, [h]], ls[:, [h]], y_ref, ls_ref, f"1024 workgroups, head {h} (group {g})")


def test_ssd_deterministic():
    c = inputs.ssd_case(2, 700, 8, G=2, seed=231)
    y1, l1 = run_gpu(c)
    y2, l2 = run_gpu(c)
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)

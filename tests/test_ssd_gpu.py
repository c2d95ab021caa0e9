"""Parity of Mamba-2's SSD layer on the matrix cores (ssm_ssd_fwd, through the C ABI) with the
fp64 oracle on the same seeded inputs.  With bf16 I/O the products take bf16 operands (the formed
operands -- the decay-weighted matrix M, the weighted B and the state's copy -- as high and low
bf16 parts), so y is held to the bf16 tolerance of the scan (3e-3 rms before its own final
rounding) and the state to 3e-3 rms.  With fp32 I/O x, B and C are split into high and low parts
too (three products per pair, about 16 bits) and y and the state are held to 1e-3 rms (SSD_TOL)."""
import numpy as np
import pytest

from selective_state_space_32_amd import inputs
from gpu_util import TOL, raw_error, to_dev, to_host_f64, y_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_32_amd import ssmscan  # noqa: E402

# fp32 I/O: every product takes 16-bit operands (bf16 high + low parts, three of the four
# partial products), a relative error of at most 2^-15 per term; a 64-token chunk's outputs
# sum about 64 + 64 such terms, whose absolute sum is ~6x the rms of the result for these
# Gaussian inputs, and the maximum over a layer's outputs is ~5x the typical error: 2^-15 x 6 x
# 5 ~ 1e-3 of rms(y).  (Measured: 1e-4 to 5e-4; the scan's fp32 bound of 1e-4 would need
# 24-bit operands.)
SSD_TOL = {"bf16": TOL["bf16"], "f32": 1e-3}


def run_gpu(c, h0=None):
    dev = lambda a: None if a is None else to_dev(a, torch)   # noqa: E731
    f = lambda a: None if a is None else torch.from_numpy(a).cuda()   # noqa: E731
    y, ls = ssmscan.ssd_fwd(dev(c.x), dev(c.dt), f(c.A), dev(c.B), dev(c.C), D=f(c.Dskip), z=dev(c.z),
                            dt_bias=f(c.dt_bias), softplus=c.softplus,
                            initial_state=None if h0 is None else torch.from_numpy(h0.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    return to_host_f64(y), to_host_f64(ls)


def run_oracle(oracle_mod, c, heads=None, h0=None):
    sel = slice(None) if heads is None else np.asarray(heads)
    zv = c.values("z")
    return oracle_mod.ssd(c.values("x")[:, :, sel], c.values("dt")[:, :, sel], c.A[sel], c.values("B"),
                          c.values("C"), D=None if c.Dskip is None else c.Dskip[sel],
                          z=None if zv is None else zv[:, :, sel],
                          dt_bias=None if c.dt_bias is None else c.dt_bias[sel], softplus=c.softplus,
                          h0=None if h0 is None else np.asarray(h0, np.float64)[:, sel])


def check(c, y, ls, y_ref, ls_ref, label):
    """The I/O type's tolerance for y and for the state: 3e-3 rms with bf16 I/O (y before its
    final rounding), 1e-4 rms with fp32 I/O."""
    io = c.io
    tol = SSD_TOL[io]
    ey, es = y_error(y, y_ref, io), raw_error(ls, ls_ref)
    print(f"[ssd {io} {label}] y err/rms {ey:.3e} (raw {raw_error(y, y_ref):.3e})  last_state {es:.3e}  "
          f"tol {tol}", flush=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(ls))
    assert ey <= tol and es <= tol, (label, ey, es)


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


def _h0(c, seed):
    """An initial state of the size a layer carries: N(0, 0.5), rounded to fp32."""
    return (0.5 * np.random.default_rng(seed).standard_normal((c.bsz, c.H, c.P, c.N))).astype(np.float32)


@pytest.mark.parametrize("L", [1, 64, 200])
def test_ssd_from_state(oracle_mod, L):
    """ssm_ssd_fwd_from: the layer continued from a given state, against the oracle from it."""
    c = inputs.ssd_case(2, L, 4, G=2, seed=240 + L)
    h0 = _h0(c, 241 + L)
    y, ls = run_gpu(c, h0)
    check(c, y, ls, *run_oracle(oracle_mod, c, h0=h0), f"from a state L={L}")


def test_ssd_pieces_equal_whole():
    """A sequence in two calls, the second from the first's last_state: the first piece a whole
    number of 64-token chunks, so every chunk and every state copy is the same as in one call
    (bitwise); in place (initial_state = last_state) as well."""
    c = inputs.ssd_case(2, 320, 3, G=1, seed=250)
    dev = lambda a: to_dev(a, torch)   # noqa: E731
    f = lambda a: torch.from_numpy(a).cuda()   # noqa: E731
    x, dt, B, C, z = dev(c.x), dev(c.dt), dev(c.B), dev(c.C), dev(c.z)
    kw = dict(D=f(c.Dskip), dt_bias=f(c.dt_bias), softplus=c.softplus)
    y0, ls0 = ssmscan.ssd_fwd(x, dt, f(c.A), B, C, z=z, **kw)
    cut = 128
    part = lambda t, a, b: t[:, a:b].contiguous()   # noqa: E731
    y1, ls1 = ssmscan.ssd_fwd(part(x, 0, cut), part(dt, 0, cut), f(c.A), part(B, 0, cut), part(C, 0, cut),
                              z=part(z, 0, cut), **kw)
    y2, ls2 = ssmscan.ssd_fwd(part(x, cut, c.L), part(dt, cut, c.L), f(c.A), part(B, cut, c.L),
                              part(C, cut, c.L), z=part(z, cut, c.L), initial_state=ls1, last_state=ls1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], 1), y0) and torch.equal(ls2, ls0)


def test_ssd_from_state_zero_length():
    """No tokens: last_state is the initial state."""
    c = inputs.ssd_case(1, 1, 2, G=1, seed=260)
    h0 = torch.from_numpy(_h0(c, 261)).cuda()
    e = torch.empty((1, 0, c.H, c.P), dtype=torch.bfloat16, device="cuda")
    f = lambda a: torch.from_numpy(a).cuda()   # noqa: E731
    _, ls = ssmscan.ssd_fwd(e, torch.empty((1, 0, c.H), dtype=torch.bfloat16, device="cuda"), f(c.A),
                            torch.empty((1, 0, 1, c.N), dtype=torch.bfloat16, device="cuda"),
                            torch.empty((1, 0, 1, c.N), dtype=torch.bfloat16, device="cuda"), initial_state=h0)
    torch.cuda.synchronize()
    assert torch.equal(ls, h0)


@pytest.mark.parametrize("P,N", [(32, 64), (64, 32), (32, 32), (128, 64), (128, 32), (192, 64), (64, 128),
                                 (128, 128)])
@pytest.mark.parametrize("L", [77, 200])
def test_ssd_head_and_state_sizes(oracle_mod, P, N, L):
    """headdim 32 / 128 / 192 and dstate 32: heads of several 64-channel parts, and 32-wide
    heads or states padded to the 64-wide tiles; two groups, gate, skip, from a state."""
    c = inputs.ssd_case(2, L, 4, P=P, G=2, N=N, seed=270 + P + N + L)
    h0 = _h0(c, 271 + P + N)
    y, ls = run_gpu(c, h0)
    assert y.shape == (2, L, 4, P) and ls.shape == (2, 4, P, N)
    check(c, y, ls, *run_oracle(oracle_mod, c, h0=h0), f"P={P} N={N} L={L}")


@pytest.mark.parametrize("L", [1, 64, 200, 513])
@pytest.mark.parametrize("G", [1, 2])
def test_ssd_dstate_128(oracle_mod, L, G):
    """dstate 128 (128-wide state tiles): chunks with ragged tails, one or two groups, gate and
    skip, from a given state."""
    c = inputs.ssd_case(2, L, 4, P=64, G=G, N=128, seed=300 + L + G)
    h0 = _h0(c, 301 + L)
    y, ls = run_gpu(c, h0)
    check(c, y, ls, *run_oracle(oracle_mod, c, h0=h0), f"N=128 L={L} G={G}")
    y0, ls0 = run_gpu(c)
    check(c, y0, ls0, *run_oracle(oracle_mod, c), f"N=128 L={L} G={G} from zero")


def test_ssd_dstate_128_pieces_equal_whole():
    """dstate 128 in two calls through the state equals one call bitwise (first piece two
    whole chunks)."""
    c = inputs.ssd_case(1, 256, 3, P=128, G=1, N=128, seed=310)
    dev = lambda a: to_dev(a, torch)   # noqa: E731
    f = lambda a: torch.from_numpy(a).cuda()   # noqa: E731
    x, dt, B, C, z = dev(c.x), dev(c.dt), dev(c.B), dev(c.C), dev(c.z)
    kw = dict(D=f(c.Dskip), dt_bias=f(c.dt_bias), softplus=c.softplus)
    y0, ls0 = ssmscan.ssd_fwd(x, dt, f(c.A), B, C, z=z, **kw)
    part = lambda t, a, b: t[:, a:b].contiguous()   # noqa: E731
    y1, ls1 = ssmscan.ssd_fwd(part(x, 0, 128), part(dt, 0, 128), f(c.A), part(B, 0, 128), part(C, 0, 128),
                              z=part(z, 0, 128), **kw)
    y2, ls2 = ssmscan.ssd_fwd(part(x, 128, 256), part(dt, 128, 256), f(c.A), part(B, 128, 256),
                              part(C, 128, 256), z=part(z, 128, 256), initial_state=ls1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], 1), y0) and torch.equal(ls2, ls0)


# --- fp32 I/O (dstate 32 or 64)

@pytest.mark.parametrize("L", [1, 63, 64, 200, 513])
@pytest.mark.parametrize("G", [1, 2])
def test_ssd_f32_small(oracle_mod, L, G):
    """fp32 x, dt, B, C, z and y: chunks of 64 with ragged tails, one or two groups."""
    c = inputs.ssd_case(2, L, 4, G=G, seed=410 + L + G, io="f32")
    y, ls = run_gpu(c)
    check(c, y, ls, *run_oracle(oracle_mod, c), f"L={L} G={G}")


@pytest.mark.parametrize("gate,skip", [(False, False), (True, False), (False, True)])
def test_ssd_f32_optional_inputs(oracle_mod, gate, skip):
    c = inputs.ssd_case(1, 300, 3, G=3, gate=gate, skip=skip, seed=420, io="f32")
    y, ls = run_gpu(c)
    check(c, y, ls, *run_oracle(oracle_mod, c), f"gate={gate} skip={skip}")


@pytest.mark.parametrize("P,N", [(32, 64), (64, 32), (32, 32), (128, 64), (192, 32)])
@pytest.mark.parametrize("L", [77, 200])
def test_ssd_f32_head_and_state_sizes(oracle_mod, P, N, L):
    """fp32 I/O with 32-wide heads or states (padded tiles) and heads of several 64-channel
    parts, from a given state."""
    c = inputs.ssd_case(2, L, 4, P=P, G=2, N=N, seed=430 + P + N + L, io="f32")
    h0 = _h0(c, 431 + P + N)
    y, ls = run_gpu(c, h0)
    assert y.shape == (2, L, 4, P) and ls.shape == (2, 4, P, N)
    check(c, y, ls, *run_oracle(oracle_mod, c, h0=h0), f"P={P} N={N} L={L}")


def test_ssd_f32_layer_size_sampled(oracle_mod):
    """B8 L2048 H80 P64 N64 G1 with fp32 I/O: sampled heads (all batches, tokens, channels)."""
    c = inputs.ssd_case(8, 2048, 80, G=1, seed=440, io="f32")
    y, ls = run_gpu(c)
    heads = np.array([0, 33, 79])
    y_ref, ls_ref = run_oracle(oracle_mod, c, heads)
    check(c, y[:, :, heads], ls[:, heads], y_ref, ls_ref, "layer, 3 heads")


def test_ssd_f32_pieces_equal_whole():
    """fp32 I/O in two calls through the state (in place) equals one call bitwise (first piece a
    whole number of chunks); repeated calls are bitwise the same."""
    c = inputs.ssd_case(2, 320, 3, G=1, seed=450, io="f32")
    dev = lambda a: to_dev(a, torch)   # noqa: E731
    f = lambda a: torch.from_numpy(a).cuda()   # noqa: E731
    x, dt, B, C, z = dev(c.x), dev(c.dt), dev(c.B), dev(c.C), dev(c.z)
    kw = dict(D=f(c.Dskip), dt_bias=f(c.dt_bias), softplus=c.softplus)
    y0, ls0 = ssmscan.ssd_fwd(x, dt, f(c.A), B, C, z=z, **kw)
    assert y0.dtype == torch.float32
    ya, lsa = ssmscan.ssd_fwd(x, dt, f(c.A), B, C, z=z, **kw)
    cut = 192
    part = lambda t, a, b: t[:, a:b].contiguous()   # noqa: E731
    y1, ls1 = ssmscan.ssd_fwd(part(x, 0, cut), part(dt, 0, cut), f(c.A), part(B, 0, cut), part(C, 0, cut),
                              z=part(z, 0, cut), **kw)
    y2, ls2 = ssmscan.ssd_fwd(part(x, cut, c.L), part(dt, cut, c.L), f(c.A), part(B, cut, c.L),
                              part(C, cut, c.L), z=part(z, cut, c.L), initial_state=ls1, last_state=ls1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(ya, y0) and torch.equal(lsa, ls0)
    assert torch.equal(torch.cat([y1, y2], 1), y0) and torch.equal(ls2, ls0)


def test_ssd_f32_agrees_with_bf16_inputs(oracle_mod):
    """The fp32 path on inputs that are bf16 values (exactly representable): its y agrees with
    the bf16 path's y to the bf16 output rounding, both against the oracle."""
    cb = inputs.ssd_case(2, 200, 4, G=2, seed=460)
    cf = inputs.SsdCase(**{**cb.__dict__, **{k: cb.values(k) for k in ("x", "dt", "B", "C", "z")}})
    assert cf.io == "f32"
    yb, lb = run_gpu(cb)
    yf, lf = run_gpu(cf)
    y_ref, ls_ref = run_oracle(oracle_mod, cb)
    check(cb, yb, lb, y_ref, ls_ref, "bf16 inputs, bf16 path")
    check(cf, yf, lf, y_ref, ls_ref, "bf16 inputs, fp32 path")

"""The training forward: ssm_scan_fwd(_from) with SSM_SCAN_CHECKPOINTS stores in its workspace
the states the backward pass needs, and ssm_scan_bwd with the same flag reads them there
instead of recomputing them in a pass of its own (both through the C ABI).

- The forward's own outputs do not change: y and last_state bitwise equal to the plain call.
- With a single-pass plan the stored states are the recompute pass's arithmetic exactly, so
  the per-element gradients (du, ddelta, dz) are bitwise those of the plain backward; the
  summed ones (atomic adds, last bits free) within 1e-6 of their rms.
- With a chunked plan the states at chunk starts come from the carry and differ by rounding:
  the fp32 gradients within 1e-5 of their rms of the plain backward; the bf16 ones, where a
  changed state can move an output across a rounding boundary, within 1e-5 of their rms after
  half a bf16 spacing of each side is taken off (both are roundings of values that agree to
  fp32 rounding: |a - b| - ulp(a)/2 - ulp(b)/2); and every gradient within the parity
  tolerance of the fp64 oracle.
"""
import numpy as np
import pytest

from selective_state_space_32_amd import inputs
from gpu_util import TOL, bf16_pair_error, case_tensors, raw_error, to_dev, to_host_f64, y_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_32_amd import ssmscan  # noqa: E402

IO_OUT = ("du", "ddelta", "dz")


def _run(case, seed, chunk_len, with_state):
    rng = np.random.default_rng(seed)
    bsz, L, D, N = case.bsz, case.L, case.D, case.N
    dy_f = rng.standard_normal((bsz, L, D), dtype=np.float32)
    dy = to_dev(inputs.bf16_bits(dy_f) if case.io == "bf16" else dy_f, torch)
    t = case_tensors(case, torch)
    h0 = torch.from_numpy((0.5 * rng.standard_normal((bsz, D, N))).astype(np.float32)).cuda() if with_state else None
    dlast = torch.from_numpy(rng.standard_normal((bsz, D, N)).astype(np.float32)).cuda() if with_state else None
    common = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=case.softplus)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"])
    # with checkpoints a forced chunk length is rounded up to a multiple of 8 tokens: the plain
    # forward it must equal bitwise runs that rounded length
    plain_len = (chunk_len + 7) // 8 * 8 if chunk_len > 0 else chunk_len
    if with_state:
        y0, ls0 = ssmscan.scan_fwd_from(h0, *args, chunk_len=plain_len, **common)
        y1, ls1, ws = ssmscan.scan_fwd_from(h0, *args, save_checkpoints=True, chunk_len=chunk_len, **common)
    else:
        y0, ls0 = ssmscan.scan_fwd(*args, chunk_len=plain_len, **common)
        y1, ls1, ws = ssmscan.scan_fwd(*args, save_checkpoints=True, chunk_len=chunk_len, **common)
    bwd = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=case.softplus, initial_state=h0,
               dlast_state=dlast, want_initial_state_grad=with_state)
    g0 = ssmscan.scan_bwd(dy, *args, **bwd)
    g1 = ssmscan.scan_bwd(dy, *args, checkpoints=ws, **bwd)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(ls0, ls1), "the forward's outputs changed with checkpoints"
    return ({k: to_host_f64(v) for k, v in g0.items()}, {k: to_host_f64(v) for k, v in g1.items()},
            to_host_f64(dy))


CASES = [
    # (label, case, chunk_len, initial state)
    ("bf16 gated, one pass", dict(bsz=2, L=300, D=128, N=16, io="bf16", gate=True), -1, False),
    ("f32 from a state, one pass", dict(bsz=1, L=257, D=64, N=16, io="f32"), -1, True),
    ("f32 N4, one pass", dict(bsz=2, L=100, D=72, N=4, io="f32"), -1, False),
    ("bf16 gated from a state, chunks of 64", dict(bsz=2, L=300, D=128, N=16, io="bf16", gate=True), 64, True),
    # chunk lengths that are not multiples of the checkpoint spacing (8 tokens): the library
    # rounds them up (20 -> 24, 100 -> 104) so that every chunk starts on a checkpoint
    ("bf16 gated, chunks of 20", dict(bsz=2, L=300, D=128, N=16, io="bf16", gate=True), 20, False),
    ("f32 from a state, chunks of 100", dict(bsz=1, L=257, D=64, N=16, io="f32"), 100, True),
]


@pytest.mark.parametrize("label,spec,chunk_len,with_state", CASES, ids=[c[0] for c in CASES])
def test_backward_from_forward_checkpoints(oracle_mod, label, spec, chunk_len, with_state):
    case = inputs.scan_case(seed=300 + spec["L"], name=label, **spec)
    g0, g1, dy = _run(case, 310 + spec["D"], chunk_len, with_state)
    assert sorted(g0) == sorted(g1)
    one_pass = chunk_len < 0
    for k in g0:
        e = raw_error(g1[k], g0[k])
        print(f"[{label}] {k}: vs the plain backward err/rms {e:.3e}", flush=True)
        assert np.all(np.isfinite(g1[k])), k
        if one_pass and k in IO_OUT:
            assert np.array_equal(g0[k], g1[k]), (label, k)
        elif one_pass:
            assert e <= 1e-6, (label, k, e)
        elif k in IO_OUT and case.io == "bf16":
            e2 = bf16_pair_error(g1[k], g0[k])
            print(f"[{label}] {k}: vs the plain backward, beyond half a bf16 spacing of each: {e2:.3e}", flush=True)
            assert e2 <= 1e-5, (label, k, e2)
        else:
            assert e <= 1e-5, (label, k, e)
    if not one_pass:   # the chunked plan's gradients against the fp64 oracle as well
        zv = case.values("z")
        rng = np.random.default_rng(310 + spec["D"])
        rng.standard_normal((case.bsz, case.L, case.D), dtype=np.float32)
        h0 = (0.5 * rng.standard_normal((case.bsz, case.D, case.N))).astype(np.float32) if with_state else None
        dlast = rng.standard_normal((case.bsz, case.D, case.N)).astype(np.float32) if with_state else None
        ref = oracle_mod.scan_bwd(case.values("u"), case.values("delta"), case.A, case.values("B"), case.values("C"),
                                  dy, D=case.Dskip, z=zv, delta_bias=case.delta_bias, softplus=case.softplus,
                                  h0=h0, dlast=dlast)
        names = {"dh0": "dinitial_state"}
        for k, r in ref.items():
            kg = names.get(k, k)
            e = y_error(g1[kg], r, case.io) if kg in IO_OUT else raw_error(g1[kg], r)
            print(f"[{label}] {kg}: vs the oracle err/rms {e:.3e} (tol {TOL[case.io]})", flush=True)
            assert e <= TOL[case.io], (label, kg, e)


@pytest.mark.parametrize("chunk_len", [-1, 64], ids=["one pass", "chunks of 64"])
def test_fused_conv_forward_checkpoints(oracle_mod, chunk_len):
    """The fused convolution's training forward: ssm_scan_fwd_conv with SSM_SCAN_CHECKPOINTS
    scans u rounded to bf16 (what u_out holds) -- in both passes of a chunked plan -- so its
    u_out equals the plain call's bitwise, its y and last_state match the oracle's scan of
    that stored u, and the backward from its checkpoints with u = u_out gives the plain
    backward's per-element gradients bitwise with one pass (the same states; with chunks, whose
    chunk-start states come from the carry, within 1e-5 of their rms beyond half a bf16 spacing
    of each side) and its sums within
    1e-6 (1e-5); through the convolution's backward, the block's input side matches the
    oracle."""
    case = inputs.scan_case(bsz=2, L=200, D=128, N=16, io="bf16", gate=True, seed=331, name="fused")
    cc = inputs.conv_case(2, 200, 128, 4, "bf16", state=False, seed=332)
    t = case_tensors(case, torch)
    x = to_dev(cc.x, torch)
    w = torch.from_numpy(cc.w).cuda()
    cb = torch.from_numpy(cc.bias).cuda()
    args = (t["delta"], t["A"], t["B"], t["C"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=case.softplus)
    u0, u1 = torch.empty_like(x), torch.empty_like(x)
    y0, ls0 = ssmscan.scan_fwd_conv(x, w, cb, *args, u_out=u0, chunk_len=chunk_len, **kw)
    y1, ls1, ws = ssmscan.scan_fwd_conv(x, w, cb, *args, u_out=u1, save_checkpoints=True, chunk_len=chunk_len, **kw)
    rng = np.random.default_rng(333)
    dy_f = rng.standard_normal((case.bsz, case.L, case.D), dtype=np.float32)
    dy = to_dev(inputs.bf16_bits(dy_f), torch)
    g0 = ssmscan.scan_bwd(dy, u0, *args, **kw)
    g1 = ssmscan.scan_bwd(dy, u1, *args, checkpoints=ws, **kw)
    gc = ssmscan.conv1d_bwd(g1["du"], x, w, cb)
    torch.cuda.synchronize()
    assert torch.equal(u0, u1)
    # y of the training forward is the scan of the bf16 u it stored (not of the fp32 u, which
    # differs by that rounding: up to 8 % of rms(y) here, where |y| reaches 35 times its rms)
    yref, lref = oracle_mod.scan(to_host_f64(u1), case.values("delta"), case.A, case.values("B"), case.values("C"),
                                 D=case.Dskip, z=case.values("z"), delta_bias=case.delta_bias, softplus=case.softplus)
    e = y_error(to_host_f64(y1), yref, "bf16")
    print(f"[fused ckpt] y vs the oracle on the stored u err/rms {e:.3e}", flush=True)
    assert e <= TOL["bf16"] and raw_error(to_host_f64(ls1), lref) <= TOL["bf16"]
    for k in g0:
        a, r = to_host_f64(g1[k]), to_host_f64(g0[k])
        e = raw_error(a, r)
        print(f"[fused ckpt] {k}: vs the plain backward err/rms {e:.3e}", flush=True)
        assert np.all(np.isfinite(a)), k
        if k in IO_OUT and chunk_len < 0:
            assert np.array_equal(a, r), k
        elif k in IO_OUT:
            assert bf16_pair_error(a, r) <= 1e-5, (k, bf16_pair_error(a, r))
        else:
            assert e <= (1e-6 if chunk_len < 0 else 1e-5), (k, e)
    # the block's input side against the oracle: the scan's backward at u = u_out, then the
    # convolution's backward of the du it gives
    uh = to_host_f64(u1)
    ref = oracle_mod.scan_bwd(uh, case.values("delta"), case.A, case.values("B"), case.values("C"),
                              to_host_f64(dy), D=case.Dskip, z=case.values("z"), delta_bias=case.delta_bias,
                              softplus=case.softplus)
    e = y_error(to_host_f64(g1["du"]), ref["du"], "bf16")
    print(f"[fused ckpt] du vs the oracle err/rms {e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    rc = oracle_mod.conv1d_bwd(cc.values("x"), cc.w, to_host_f64(g1["du"]), bias=cc.bias, silu=True)
    for k in ("dx", "dw", "dbias"):
        a = to_host_f64(gc[k])
        e = y_error(a, rc[k], "bf16") if k == "dx" else raw_error(a, rc[k])
        print(f"[fused ckpt] conv {k} vs the oracle err/rms {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (k, e)


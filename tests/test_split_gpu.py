"""The split schedule, the library's plan for dstate 16 with 2 to 2.5 channel tiles per CU
(the B8 D5120 layer on a 256-CU MI355X): part of the tiles run as two token halves, the
second started from the state the first hands over through the workspace, so that every CU
gets the same share of tokens.  The states are those of the one-pass plan, so every output
must be bitwise the same as with dims->chunk_len = -1 (one workgroup per tile, one pass), and
the oracle must agree on sampled channels.  The time-out path (a second half that gets no
hand-over computes its whole tile) is forced from the host with SSMSCAN_HANDOVER_WAIT_US=0.
"""
import os

import numpy as np
import pytest

from selective_state_space_32_amd import inputs
from gpu_util import TOL, case_tensors, raw_error, to_dev, to_host_f64, y_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_32_amd import ssmscan  # noqa: E402


def split_dim():
    """A channel count giving the batch of 8 between 2 and 2.5 tiles per CU on this device."""
    cus = ssmscan.plan_info(1, 256, 64, 16, 1)["cu_count"]
    return 64 * ((5 * cus) // 16), cus


def _case(L, io, gate, seed):
    D, _ = split_dim()
    return inputs.scan_case(8, L, D, 16, io, gate=gate, seed=seed, name=f"split {io} L{L}")


def _ckpt_bytes(case):
    """The checkpoints at the start of a training forward's workspace: the state before every
    8th token, fp32."""
    return case.bsz * ((case.L + 7) // 8) * case.D * 16 * 4


def _fwd(case, t, chunk_len, **kw):
    y, ls = ssmscan.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                             delta_bias=t["delta_bias"], softplus=case.softplus, chunk_len=chunk_len, **kw)
    return y, ls


@pytest.mark.parametrize("io,gate,L", [("bf16", True, 300), ("f32", False, 300), ("bf16", False, 2048)],
                         ids=["bf16 gated L300", "f32 L300", "bf16 L2048"])
def test_split_equals_one_pass(oracle_mod, io, gate, L):
    case = _case(L, io, gate, seed=500 + L)
    p = ssmscan.plan_info(case.bsz, case.L, case.D, 16, torch.bfloat16 if io == "bf16" else torch.float32)
    print(f"[{case.name}] plan {p}", flush=True)
    assert p["split_tiles"] > 0 and p["split_at"] == (L // 2 + 31) // 32 * 32
    t = case_tensors(case, torch)
    y0, ls0 = _fwd(case, t, -1)
    y1, ls1 = _fwd(case, t, 0)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1), "split schedule y differs from the one pass"
    assert torch.equal(ls0, ls1), "split schedule last_state differs from the one pass"
    # sampled channels of the split result against the oracle: the whole tiles (first), the
    # split tiles (last 128 * 64 channels of the batch's flat tile order) and channel edges
    D = case.D
    sel = np.unique(np.array([0, 1, 63, 64, D // 2, D - 65, D - 64, D - 2, D - 1]))
    y_ref, ls_ref = oracle_mod.scan_case(case, channels=sel)
    yh, lh = to_host_f64(y1), to_host_f64(ls1)
    e = y_error(yh[:, :, sel], y_ref, io)
    es = raw_error(lh[:, sel], ls_ref)
    print(f"[{case.name}] split vs oracle: y err/rms {e:.3e}, last_state {es:.3e} (tol {TOL[io]})", flush=True)
    assert e <= TOL[io] and es <= TOL[io]


def test_split_time_out_path_equals_one_pass(monkeypatch):
    """Every second half gives up waiting at once and computes its whole tile."""
    case = _case(300, "bf16", True, seed=520)
    t = case_tensors(case, torch)
    y0, ls0 = _fwd(case, t, -1)
    monkeypatch.setenv("SSMSCAN_HANDOVER_WAIT_US", "0")
    y1, ls1 = _fwd(case, t, 0)
    torch.cuda.synchronize()
    monkeypatch.delenv("SSMSCAN_HANDOVER_WAIT_US")
    assert torch.equal(y0, y1) and torch.equal(ls0, ls1)


def test_split_repeated_calls_reuse_workspace():
    """The hand-over flags are cleared by each call: three calls on one workspace agree."""
    case = _case(300, "bf16", True, seed=530)
    t = case_tensors(case, torch)
    ws = torch.empty(ssmscan.workspace_bytes(case.bsz, case.L, case.D, 16, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    outs = [_fwd(case, t, 0, workspace=ws) for _ in range(3)]
    y0, ls0 = _fwd(case, t, -1)
    torch.cuda.synchronize()
    for y, ls in outs:
        assert torch.equal(y, y0) and torch.equal(ls, ls0)


def test_split_from_a_state_and_in_place():
    """scan_fwd_from: from a separate initial state (split) and with the initial state being
    the last_state buffer (the library then takes the one pass) -- both equal the one pass."""
    case = _case(300, "bf16", True, seed=540)
    t = case_tensors(case, torch)
    rng = np.random.default_rng(541)
    h0 = torch.from_numpy((0.3 * rng.standard_normal((case.bsz, case.D, 16))).astype(np.float32)).cuda()
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=True)
    y0, ls0 = ssmscan.scan_fwd_from(h0, *args, chunk_len=-1, **kw)
    y1, ls1 = ssmscan.scan_fwd_from(h0, *args, chunk_len=0, **kw)
    st = h0.clone()
    y2, ls2 = ssmscan.scan_fwd_from(st, *args, chunk_len=0, last_state=st, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(ls0, ls1)
    assert torch.equal(y0, y2) and torch.equal(ls0, st)


def test_split_training_forward_checkpoints():
    """With SSM_SCAN_CHECKPOINTS the split forward stores the same checkpoints as the one pass
    (bitwise), and the backward from them gives the same per-element gradients."""
    case = _case(300, "bf16", True, seed=550)
    t = case_tensors(case, torch)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=True)
    y0, ls0, ws0 = ssmscan.scan_fwd(*args, chunk_len=-1, save_checkpoints=True, **kw)
    y1, ls1, ws1 = ssmscan.scan_fwd(*args, chunk_len=0, save_checkpoints=True, **kw)
    nck = _ckpt_bytes(case)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(ls0, ls1)
    assert torch.equal(ws0[:nck], ws1[:nck]), "checkpoints differ between the split and the one pass"
    dy = to_dev(inputs.bf16_bits(np.random.default_rng(551).standard_normal((case.bsz, case.L, case.D),
                                                                             dtype=np.float32)), torch)
    g0 = ssmscan.scan_bwd(dy, *args, checkpoints=ws0, **kw)
    g1 = ssmscan.scan_bwd(dy, *args, checkpoints=ws1, **kw)
    # the backward's own checkpoint pass, under the split schedule on this device
    g2 = ssmscan.scan_bwd(dy, *args, **kw)
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dz"):
        assert torch.equal(g0[k], g1[k]), k
        assert torch.equal(g0[k], g2[k]), k + " (checkpoint pass)"


@pytest.mark.parametrize("ckpt", [False, True], ids=["forward", "training forward"])
def test_split_fused_convolution(ckpt):
    """The convolution fused into the scan under the split schedule: the second halves take the
    three x rows before their first token from memory; y, u_out and last_state equal the one
    pass bitwise."""
    case = _case(300, "bf16", True, seed=560)
    cc = inputs.conv_case(case.bsz, case.L, case.D, 4, "bf16", state=False, seed=561)
    t = case_tensors(case, torch)
    x, w, cb = to_dev(cc.x, torch), torch.from_numpy(cc.w).cuda(), torch.from_numpy(cc.bias).cuda()
    args = (t["delta"], t["A"], t["B"], t["C"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=True)
    u0, u1 = torch.empty_like(x), torch.empty_like(x)
    r0 = ssmscan.scan_fwd_conv(x, w, cb, *args, u_out=u0, chunk_len=-1, save_checkpoints=ckpt, **kw)
    r1 = ssmscan.scan_fwd_conv(x, w, cb, *args, u_out=u1, chunk_len=0, save_checkpoints=ckpt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(r0[0], r1[0]) and torch.equal(r0[1], r1[1]) and torch.equal(u0, u1)
    if ckpt:
        nck = _ckpt_bytes(case)
        assert torch.equal(r0[2][:nck], r1[2][:nck])


@pytest.mark.parametrize("gate", [True, False], ids=["gated", "ungated"])
def test_split_backward_time_out_path(monkeypatch, gate):
    """The backward under the split schedule (checkpoint pass and reverse walk) with every
    second half giving up at once: the checkpoint pass's second halves compute whole tiles,
    the walk's form the adjoint at the split point themselves.  The per-element gradients and
    the initial state's gradient are bitwise those with the hand-overs; the sums over
    workgroups (atomic, in another order) agree to rounding."""
    case = _case(300, "bf16", gate, seed=570)
    t = case_tensors(case, torch)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=True)
    rng = np.random.default_rng(571)
    dy = to_dev(inputs.bf16_bits(rng.standard_normal((case.bsz, case.L, case.D), dtype=np.float32)), torch)
    dls = torch.from_numpy(rng.standard_normal((case.bsz, case.D, 16)).astype(np.float32)).cuda()
    g0 = ssmscan.scan_bwd(dy, *args, dlast_state=dls, want_initial_state_grad=True, **kw)
    torch.cuda.synchronize()
    monkeypatch.setenv("SSMSCAN_HANDOVER_WAIT_US", "0")
    g1 = ssmscan.scan_bwd(dy, *args, dlast_state=dls, want_initial_state_grad=True, **kw)
    torch.cuda.synchronize()
    monkeypatch.delenv("SSMSCAN_HANDOVER_WAIT_US")
    keys = ("du", "ddelta", "dinitial_state") + (("dz",) if gate else ())
    for k in keys:
        assert torch.equal(g0[k], g1[k]), k
    for k in ("dA", "dB", "dC", "dD", "ddelta_bias"):
        a, b = g0[k].double(), g1[k].double()
        e = float((a - b).abs().max() / a.abs().max().clamp_min(1e-30))
        assert e < 1e-5, f"{k}: {e:.3g}"

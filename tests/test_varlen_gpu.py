"""Sequences of different lengths in one batch (ssm_scan_fwd_varlen): sequence b is scanned
over its first seq_lens[b] tokens only, from its initial state, and its final state is the
state after that length.  Checked against the oracle's per-sequence scan on every plan the
library picks (one pass, chunked carry, split halves), with lengths 0, 1, ragged, a chunk
boundary and L; the outputs past each length must be left exactly as they were, and values
there (NaN here) must not reach anything."""
import numpy as np
import pytest

from selective_state_space_32_amd import inputs
from gpu_util import TOL, case_tensors, raw_error, to_dev, to_host_f64, y_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_32_amd import ssmscan  # noqa: E402

SENTINEL = 12288.0   # exact in bf16 and fp32


def _oracle(oracle_mod, case, lens, sel, h0=None):
    u = case.values("u")[:, :, sel]
    dl = case.values("delta")[:, :, sel]
    z = case.values("z")
    z = None if z is None else z[:, :, sel]
    D = None if case.Dskip is None else case.Dskip[sel]
    bias = None if case.delta_bias is None else case.delta_bias[sel]
    h = None if h0 is None else np.asarray(h0)[:, sel]
    return oracle_mod.scan_varlen(u, dl, case.A[sel], case.values("B"), case.values("C"), lens, D=D, z=z,
                                  delta_bias=bias, softplus=case.softplus, h0=h)


def _lens(bsz, L, pattern):
    if pattern == "ragged":
        base = [0, 1, L, L // 2 + 3, 64, L - 1, 17, 2 * L // 3]
    elif pattern == "full":
        base = [L]
    else:
        base = [0]
    return np.array([base[i % len(base)] for i in range(bsz)], np.int32)


def _run(case, t, lens, chunk_len, h0, poison):
    io = case.io
    dev_lens = torch.from_numpy(lens).cuda()
    if poison:
        # NaN in every input past each sequence's length: none of it may be read
        for k in ("u", "delta", "B", "C", "z"):
            if t[k] is None:
                continue
            v = t[k].clone()
            for b, lb in enumerate(lens):
                v[b, int(lb):] = float("nan")
            t = dict(t, **{k: v})
    y = torch.full_like(t["u"], SENTINEL)
    h0_t = None if h0 is None else torch.from_numpy(h0.astype(np.float32)).cuda()
    y, ls = ssmscan.scan_fwd_varlen(dev_lens, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                    delta_bias=t["delta_bias"], softplus=case.softplus, initial_state=h0_t,
                                    y=y, chunk_len=chunk_len)
    torch.cuda.synchronize()
    return to_host_f64(y), to_host_f64(ls)


def _check(oracle_mod, case, lens, y, ls, sel, h0):
    io = case.io
    y_ref, ls_ref = _oracle(oracle_mod, case, lens, sel, h0)
    ys = y[:, :, sel]
    tol = TOL[io]
    for b, lb in enumerate(lens):
        lb = int(lb)
        assert np.all(ys[b, lb:] == SENTINEL), f"sequence {b}: outputs past length {lb} were written"
        if lb:
            e = y_error(ys[b, :lb], y_ref[b, :lb], io)
            assert e < tol, f"sequence {b} (length {lb}): y error {e:.3g}"
    e = raw_error(ls[:, sel], ls_ref)
    assert e < tol, f"last_state error {e:.3g}"


CASES = [
    # (name, bsz, L, D, N, io, gate, chunk_len, h0)
    ("one pass f32 N16", 8, 300, 128, 16, "f32", True, -1, False),
    ("one pass bf16 N16 h0", 8, 300, 128, 16, "bf16", True, -1, True),
    ("carry f32 N16 chunk64", 8, 300, 256, 16, "f32", False, 64, False),
    ("carry bf16 N16 chunk96 h0", 8, 300, 256, 16, "bf16", True, 96, True),
    ("carry bf16 N4 chunk32", 8, 300, 192, 4, "bf16", True, 32, False),
    ("one pass f32 N8", 8, 131, 64, 8, "f32", False, -1, True),
    ("auto plan bf16 N16", 8, 520, 320, 16, "bf16", True, 0, False),
]


@pytest.mark.parametrize("name,bsz,L,D,N,io,gate,chunk_len,use_h0", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("pattern", ["ragged", "full", "empty"])
def test_varlen_matches_oracle(oracle_mod, name, bsz, L, D, N, io, gate, chunk_len, use_h0, pattern):
    case = inputs.scan_case(bsz, L, D, N, io, gate=gate, seed=700 + L + D + N, name=f"varlen {name}")
    lens = _lens(bsz, L, pattern)
    rng = np.random.default_rng(7)
    h0 = rng.standard_normal((bsz, D, N)) if use_h0 else None
    print(f"[{case.name} {pattern}] lens {lens.tolist()} chunk_len {chunk_len}", flush=True)
    t = case_tensors(case, torch)
    y, ls = _run(case, t, lens, chunk_len, h0, poison=(pattern == "ragged"))
    sel = np.unique(np.array([0, 1, D // 3, D // 2, D - 2, D - 1]))
    _check(oracle_mod, case, lens, y, ls, sel, h0)


def test_varlen_full_lengths_bitwise_scan(oracle_mod):
    """All lengths L: bitwise the plain scan (same plan, same arithmetic)."""
    case = inputs.scan_case(4, 300, 256, 16, "bf16", gate=True, seed=711, name="varlen = scan")
    t = case_tensors(case, torch)
    for chunk_len in (-1, 64, 0):
        lens = torch.full((4,), 300, dtype=torch.int32, device="cuda")
        y0, ls0 = ssmscan.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                   delta_bias=t["delta_bias"], softplus=True, chunk_len=chunk_len)
        y1, ls1 = ssmscan.scan_fwd_varlen(lens, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                          delta_bias=t["delta_bias"], softplus=True, chunk_len=chunk_len)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(ls0, ls1), f"chunk_len {chunk_len}"


def test_varlen_split_plan(oracle_mod):
    """The split plan (2 to 2.5 tiles per CU): the handover of a sequence whose length ends in
    either half, at the split point or before it."""
    cus = ssmscan.plan_info(1, 256, 64, 16, 1)["cu_count"]
    D = 64 * ((5 * cus) // 16)
    L = 300
    case = inputs.scan_case(8, L, D, 16, "bf16", gate=True, seed=733, name="varlen split")
    p = ssmscan.plan_info(8, L, D, 16, torch.bfloat16)
    print(f"[{case.name}] plan {p}", flush=True)
    assert p["split_tiles"] > 0
    mid = p["split_at"]
    lens = np.array([L, 0, mid, mid - 1, mid + 1, 1, L - 1, 37], np.int32)
    t = case_tensors(case, torch)
    y, ls = _run(case, t, lens, 0, None, poison=True)
    # whole tiles first in the flat tile order, the split ones last: sample both, and the edges
    sel = np.unique(np.array([0, 1, 63, 64, D // 2, D - 65, D - 64, D - 2, D - 1]))
    _check(oracle_mod, case, lens, y, ls, sel, None)


def test_varlen_rejects_bad_lengths_tensor():
    t = torch.zeros(2, 8, 64, device="cuda")
    A = -torch.ones(64, 16, device="cuda")
    Bm = torch.zeros(2, 8, 16, device="cuda")
    with pytest.raises(ValueError):
        ssmscan.scan_fwd_varlen(torch.zeros(2, dtype=torch.int64, device="cuda"), t, t, A, Bm, Bm)
    with pytest.raises(ValueError):
        ssmscan.scan_fwd_varlen(torch.zeros(3, dtype=torch.int32, device="cuda"), t, t, A, Bm, Bm)


# --- gradients (ssm_scan_bwd_varlen) -----------------------------------------------------------

from test_bwd_gpu import check_grads, _io_array, _values  # noqa: E402

BWD_CASES = [
    # (name, bsz, L, D, N, io, gate)
    ("bwd f32 N16", 8, 150, 128, 16, "f32", True),
    ("bwd bf16 N16", 8, 150, 128, 16, "bf16", True),
    ("bwd bf16 N4 ungated", 8, 97, 64, 4, "bf16", False),
]


def _bwd_run(oracle_mod, case, lens, seed, poison=False, channels=None, checkpoints=None):
    rng = np.random.default_rng(seed)
    bsz, L, D, N = case.bsz, case.L, case.D, case.N
    dy = _io_array(rng.standard_normal((bsz, L, D), dtype=np.float32), case.io)
    h0 = (0.5 * rng.standard_normal((bsz, D, N))).astype(np.float32)
    dlast = rng.standard_normal((bsz, D, N)).astype(np.float32)
    t = case_tensors(case, torch)
    dyt = to_dev(dy, torch)
    if poison:
        for k in ("u", "delta", "B", "C", "z"):
            if t[k] is None:
                continue
            v = t[k].clone()
            for b, lb in enumerate(lens):
                v[b, int(lb):] = float("nan")
            t[k] = v
        dyt = dyt.clone()
        for b, lb in enumerate(lens):
            dyt[b, int(lb):] = float("nan")
    g = ssmscan.scan_bwd(dyt, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                         delta_bias=t["delta_bias"], softplus=case.softplus, initial_state=torch.from_numpy(h0).cuda(),
                         dlast_state=torch.from_numpy(dlast).cuda(), want_initial_state_grad=True,
                         seq_lens=torch.from_numpy(np.asarray(lens, np.int32)).cuda(), checkpoints=checkpoints)
    torch.cuda.synchronize()
    got = {k: to_host_f64(v) for k, v in g.items()}
    sel = slice(None) if channels is None else np.asarray(channels)
    zv = case.values("z")
    ref = oracle_mod.scan_bwd_varlen(case.values("u")[:, :, sel], case.values("delta")[:, :, sel], case.A[sel],
                                     case.values("B"), case.values("C"), _values(dy, case.io)[:, :, sel], lens,
                                     D=None if case.Dskip is None else case.Dskip[sel],
                                     z=None if zv is None else zv[:, :, sel],
                                     delta_bias=None if case.delta_bias is None else case.delta_bias[sel],
                                     softplus=case.softplus, h0=h0[:, sel], dlast=dlast[:, sel])
    if channels is not None:
        got = {k: (v[:, :, sel] if v.ndim == 3 and k in ("du", "ddelta", "dz") else
                   v[sel] if k in ("dA", "dD", "ddelta_bias") else
                   v[:, sel] if k == "dinitial_state" else v)
               for k, v in got.items()}
        got.pop("dB"), got.pop("dC"), ref.pop("dB"), ref.pop("dC")
    return got, ref


@pytest.mark.parametrize("name,bsz,L,D,N,io,gate", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_varlen_bwd_matches_oracle(oracle_mod, name, bsz, L, D, N, io, gate):
    """Every gradient against the oracle's per-sequence backward, lengths 0, 1, ragged and L,
    with NaN past each length in the inputs and in dy; the gradients there are exactly zero."""
    case = inputs.scan_case(bsz, L, D, N, io, gate=gate, seed=800 + L + N, name=f"varlen {name}")
    lens = _lens(bsz, L, "ragged")
    print(f"[{case.name}] lens {lens.tolist()}", flush=True)
    got, ref = _bwd_run(oracle_mod, case, lens, seed=801, poison=True)
    for k in ("du", "ddelta", "dz", "dB", "dC"):
        if k in got:
            for b, lb in enumerate(lens):
                assert np.all(got[k][b, int(lb):] == 0.0), (k, b)
    check_grads(case, got, ref, "varlen")


def test_varlen_bwd_full_lengths_bitwise():
    """All lengths L: the per-element gradients of the plain backward bitwise."""
    case = inputs.scan_case(4, 300, 256, 16, "bf16", gate=True, seed=811, name="varlen bwd = bwd")
    t = case_tensors(case, torch)
    dy = to_dev(inputs.bf16_bits(np.random.default_rng(812).standard_normal((4, 300, 256), dtype=np.float32)),
                torch)
    args = (dy, t["u"], t["delta"], t["A"], t["B"], t["C"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=True)
    g0 = ssmscan.scan_bwd(*args, **kw)
    g1 = ssmscan.scan_bwd(*args, seq_lens=torch.full((4,), 300, dtype=torch.int32, device="cuda"), **kw)
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dz"):
        assert torch.equal(g0[k], g1[k]), k


def test_varlen_bwd_split_plan_and_checkpoints(oracle_mod):
    """The split schedule (checkpoint pass and walk), lengths around the split point, sampled
    channels against the oracle; and the same gradients from a training forward_varlen's
    checkpoints."""
    cus = ssmscan.plan_info(1, 256, 64, 16, 1)["cu_count"]
    D = 64 * ((5 * cus) // 16)
    L = 300
    case = inputs.scan_case(8, L, D, 16, "bf16", gate=True, seed=821, name="varlen bwd split")
    p = ssmscan.plan_info(8, L, D, 16, torch.bfloat16)
    assert p["split_tiles"] > 0
    mid = p["split_at"]
    lens = np.array([L, 0, mid, mid - 1, mid + 1, 1, L - 1, 37], np.int32)
    sel = np.unique(np.array([0, 1, 63, 64, D // 2, D - 65, D - 64, D - 2, D - 1]))
    got, ref = _bwd_run(oracle_mod, case, lens, seed=822, channels=sel)
    check_grads(case, got, ref, "varlen split")
    # from the training forward's checkpoints (forward_varlen with SSM_SCAN_CHECKPOINTS), from
    # the same initial state
    t = case_tensors(case, torch)
    rng = np.random.default_rng(822)
    _ = rng.standard_normal((8, L, D), dtype=np.float32)   # (dy, drawn first in _bwd_run)
    h0 = torch.from_numpy((0.5 * rng.standard_normal((8, D, 16))).astype(np.float32)).cuda()
    dl = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    _, _, ws = ssmscan.scan_fwd_varlen(dl, t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                       delta_bias=t["delta_bias"], softplus=True, initial_state=h0,
                                       save_checkpoints=True)
    got2, _ = _bwd_run(oracle_mod, case, lens, seed=822, channels=sel, checkpoints=ws)
    for k in ("du", "ddelta", "dz"):
        assert np.array_equal(got[k], got2[k]), k

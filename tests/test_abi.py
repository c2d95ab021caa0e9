"""The C-ABI library: it loads, exports every symbol include/ssmscan.h declares, and
rejects bad arguments before launching anything (no GPU needed: every call here fails
validation on the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssmscan.h")
LIB = os.environ.get("SSMSCAN_LIBRARY") or os.path.join(ROOT, "selective_state_space_32_amd", "libssmscan.so")


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"SSMSCAN_API\s+[\w\s\*]+?\b(ssm_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def b():
    if not os.path.exists(LIB):
        pytest.fail("libssmscan.so is not built (run __graft_entry__.build())")
    from selective_state_space_32_amd import ssmscan
    return ssmscan


def test_header_declares_the_entry_points():
    syms = set(declared_symbols())
    assert {"ssm_scan_fwd", "ssm_scan_fwd_from", "ssm_scan_bwd", "ssm_scan_bwd_workspace_bytes", "ssm_step",
            "ssm_conv1d_fwd", "ssm_conv1d_bwd", "ssm_scan_fwd_conv", "ssm_ssd_fwd", "ssm_ssd_fwd_from", "ssm_scan_bwd_varlen",
            "ssm_scan_workspace_bytes", "ssm_scan_plan", "ssm_last_error", "ssm_version", "ssm_step_act"} <= syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for s in declared_symbols():
        assert hasattr(lib, s), s


def test_version(b):
    import re
    hdr = open(os.path.join(ROOT, "include", "ssmscan.h")).read()
    assert b.lib.ssm_version() == int(re.search(r"#define SSMSCAN_VERSION (\d+)", hdr).group(1))


def _dims(b, **kw):
    base = dict(batch=2, seqlen=64, dim=128, dstate=16, io_dtype=1, chunk_len=0)
    base.update(kw)
    return b.ssm_dims(base["batch"], base["seqlen"], base["dim"], base["dstate"], base["io_dtype"], base["chunk_len"])


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def _scan(b, dims, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, y=FAKE, ws=FAKE, ws_bytes=None, z=None, ls=None):
    if ws_bytes is None:
        ws_bytes = b.lib.ssm_scan_workspace_bytes(ctypes.byref(dims))
    P = ctypes.c_void_p
    return b.lib.ssm_scan_fwd(P(u), P(delta), P(A), P(B), P(C), None, P(z) if z else None, None, 1, P(y),
                              P(ls) if ls else None, ctypes.byref(dims), P(ws), ws_bytes, None)


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "y"])
def test_null_pointer_rejected(b, field):
    rc = _scan(b, _dims(b), **{field: 0})
    assert rc == -1 and field in b.last_error() or rc == -1


def test_null_dims_rejected(b):
    P = ctypes.c_void_p
    rc = b.lib.ssm_scan_fwd(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, None, 1, P(FAKE), None, None,
                            P(FAKE), 1 << 20, None)
    assert rc == -1


@pytest.mark.parametrize("n", [0, 3, 5, 32, 64])
def test_unsupported_state_size(b, n):
    assert _scan(b, _dims(b, dstate=n)) == -5
    assert "dstate" in b.last_error()


def test_bad_dtype(b):
    assert _scan(b, _dims(b, io_dtype=7)) == -3


@pytest.mark.parametrize("kw", [dict(batch=-1), dict(seqlen=-5), dict(dim=-2), dict(chunk_len=-2),
                                dict(dim=(1 << 30) + 1), dict(batch=1 << 20, seqlen=1 << 20, dim=1 << 20)])
def test_bad_shape(b, kw):
    assert _scan(b, _dims(b, **kw)) == -2


def test_workspace_too_small(b):
    d = _dims(b, chunk_len=16)   # 4 chunks per sequence: carry states need workspace
    need = b.lib.ssm_scan_workspace_bytes(ctypes.byref(d))
    assert need >= 2 * 4 * 128 * 16 * 4
    assert _scan(b, d, ws_bytes=need - 1) == -6
    assert _scan(b, d, ws=0) == -6


def test_scan_from_validation(b):
    # a misaligned initial state is rejected before any launch; the other checks are the scan's
    P = ctypes.c_void_p
    d = _dims(b)
    ws = b.lib.ssm_scan_workspace_bytes(ctypes.byref(d))
    args = [P(FAKE)] * 5 + [None, None, None, 1, P(FAKE), None, ctypes.byref(d), P(FAKE), ws, None]
    assert b.lib.ssm_scan_fwd_from(P(FAKE + 2), *args) == -4
    assert "initial_state" in b.last_error()
    args[0] = P(0)
    assert b.lib.ssm_scan_fwd_from(P(FAKE), *args) == -1


def _bwd(b, dims, ws_bytes=None, **kw):
    P = ctypes.c_void_p
    names = ["h0", "u", "delta", "A", "B", "C", "D", "z", "bias", "softplus", "dy", "dlast", "du", "ddelta", "dA",
             "dB", "dC", "dD", "dz", "dbias", "dh0"]
    vals = dict(h0=None, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, softplus=1, dy=FAKE,
                dlast=None, du=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=None, dz=None, dbias=None, dh0=None)
    vals.update(kw)
    args = [vals[k] if k == "softplus" else (P(vals[k]) if vals[k] else None) for k in names]
    if ws_bytes is None:
        ws_bytes = b.lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(dims))
    return b.lib.ssm_scan_bwd(*args, ctypes.byref(dims), P(FAKE), ws_bytes, None)


def test_bwd_validation(b):
    # every rejection happens before any launch (the pointers are never dereferenced)
    d = _dims(b)
    assert b.lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d)) >= 2 * 4 * 128 * 16 * 4
    assert _bwd(b, d, dy=0) == -1
    assert _bwd(b, d, z=FAKE) == -1 and "dz" in b.last_error()
    assert _bwd(b, d, du=FAKE + 1) == -4
    assert _bwd(b, d, dh0=FAKE + 2) == -4
    assert _bwd(b, d, ws_bytes=16) == -6


def test_flags_validated(b):
    # unknown flag bits are rejected by the scan and by the backward
    P = ctypes.c_void_p
    d = _dims(b)
    ws = b.lib.ssm_scan_workspace_bytes(ctypes.byref(d))
    def fwd(flags, ws_bytes=ws):
        return b.lib.ssm_scan_fwd(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, None, flags, P(FAKE),
                                  None, ctypes.byref(d), P(FAKE), ws_bytes, None)
    for flags in (8, 1 << 20, -1):
        assert fwd(flags) == -8 and "flag" in b.last_error()
    # checkpoints for the backward (also with the exact ZOH): the workspace must hold them
    assert fwd(1 | 2 | 4) == -6
    assert fwd(1 | 4) == -6
    ckpt = b.lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d))
    assert fwd(1 | 4, ckpt + ws - 16) == -6
    # the backward takes softplus, the exact ZOH and checkpoints (rejected here for the workspace)
    assert _bwd(b, d, softplus=3, ws_bytes=16) == -6
    assert _bwd(b, d, softplus=2 | 4, ws_bytes=16) == -6
    assert _bwd(b, d, softplus=1 | 8) == -8 and "flag" in b.last_error()


def test_conv_validation(b):
    # every rejection happens before any launch
    P = ctypes.c_void_p
    d = _dims(b, dstate=3)           # dstate does not apply to the convolution

    def conv(width=4, flags=1, x=FAKE, out=FAKE, w=FAKE, si=None, so=None, dims=d):
        return b.lib.ssm_conv1d_fwd(P(x), P(w), None, width, P(si) if si else None, flags, P(out),
                                    P(so) if so else None, ctypes.byref(dims), None)
    assert conv(width=0) == -2 and conv(width=5) == -2
    assert conv(flags=2) == -8
    assert conv(x=FAKE + 1) == -4
    assert conv(w=0) == -1
    assert conv(out=0) == -1
    assert conv(dims=_dims(b, io_dtype=5)) == -3


def test_conv_bwd_validation(b):
    P = ctypes.c_void_p
    d = _dims(b, dstate=3)

    def call(width=4, flags=1, x=FAKE, dout=FAKE, dx=FAKE, w=FAKE, dw=FAKE, dims=d):
        return b.lib.ssm_conv1d_bwd(P(x), P(w), None, width, None, flags, P(dout), P(dx), P(dw), None, None,
                                    ctypes.byref(dims) if dims is not None else None, None)
    assert call(dims=None) == -1
    assert call(width=0) == -2 and call(width=5) == -2
    assert call(flags=2) == -8
    assert call(x=FAKE + 1) == -4 and call(dx=FAKE + 1) == -4 and call(dw=FAKE + 2) == -4
    assert call(w=0) == -1 and call(dw=0) == -1
    assert call(x=0) == -1 and call(dout=0) == -1 and call(dx=0) == -1
    assert call(dims=_dims(b, io_dtype=5)) == -3
    assert call(dims=_dims(b, seqlen=-1)) == -2


def test_conv_scan_validation(b):
    P = ctypes.c_void_p
    d = _dims(b)
    ws = b.lib.ssm_scan_workspace_bytes(ctypes.byref(d))

    def call(width=4, flags=1, x=FAKE, w=FAKE, dims=d):
        return b.lib.ssm_scan_fwd_conv(P(x), P(w), None, width, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, None,
                                       flags, P(FAKE), None, None, ctypes.byref(dims), P(FAKE), ws, None)
    assert call(width=3) == -2
    assert call(flags=3) == -8
    assert call(flags=1 | 4) == -6          # checkpoints accepted: the workspace must then hold them
    assert call(w=0) == -1
    assert call(x=FAKE + 1) == -4          # a bf16 x must be 2-byte aligned


def test_ssd_validation(b):
    P = ctypes.c_void_p

    def call(x=FAKE, io=1, hd=64, ds=64, H=8, G=2, flags=1):
        d = b.ssm_ssd_dims(2, 100, H, hd, G, ds, io, 0)
        return b.lib.ssm_ssd_fwd(P(x), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, None, flags, P(FAKE), None,
                                 ctypes.byref(d), None)
    assert call(io=7) == -3
    assert call(io=0, ds=128) == -2     # fp32 I/O: dstate 32 or 64
    assert call(hd=48) == -2 and call(hd=96) == -2 and call(ds=256) == -2 and call(ds=16) == -2
    assert call(hd=32, ds=128) == -2   # dstate 128 has no padded form for 32-wide heads
    assert call(G=3) == -2
    assert call(H=(1 << 18) + 1, G=1) == -2   # nheads*headdim above 2^24
    assert call(flags=3) == -8
    assert call(x=FAKE + 2) == -4


def test_misaligned_rejected(b):
    assert _scan(b, _dims(b), u=FAKE + 1) == -4
    assert _scan(b, _dims(b, io_dtype=0), y=FAKE + 2) == -4
    assert _scan(b, _dims(b, chunk_len=16), ws=FAKE + 8) == -4
    assert _scan(b, _dims(b), B=FAKE + 2) == -4    # bf16 B/C are read as 32-bit words


def test_step_validation(b):
    P = ctypes.c_void_p
    d = _dims(b, seqlen=1)
    args = [P(FAKE)] * 6 + [None, None, P(FAKE)]
    assert b.lib.ssm_step(None, *args[1:], ctypes.byref(d), None) == -1
    assert b.lib.ssm_step(P(FAKE + 4), *args[1:], ctypes.byref(d), None) == -4   # state needs 16 B
    assert b.lib.ssm_step(*args, ctypes.byref(_dims(b, dstate=6)), None) == -5


def test_step_act_validation(b):
    P = ctypes.c_void_p
    d = _dims(b, seqlen=1)
    rest = [P(FAKE)] * 5 + [None, None]   # u, delta, A, B, C, D, z

    def call(flags, bias=None, dims=d, state=P(FAKE)):
        return b.lib.ssm_step_act(state, *rest, bias, flags, P(FAKE), ctypes.byref(dims), None)
    assert call(4) == -8                      # checkpoints belong to a scan
    assert b"SSM_SCAN_EXACT_ZOH" in b.lib.ssm_last_error()
    assert call(8) == -8                      # unknown bit
    assert call(1, bias=P(FAKE + 2)) == -4    # delta_bias must be 4-byte aligned
    assert call(3, state=None) == -1
    assert call(1, state=P(FAKE + 4)) == -4   # state needs 16 bytes when dstate >= 4
    assert call(2, dims=_dims(b, dstate=6)) == -5


def test_empty_problems_are_noops(b):
    # zero batch or zero channels: nothing to do, no pointer is touched
    for kw in (dict(batch=0), dict(dim=0)):
        d = _dims(b, **kw)
        assert b.lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == 0
        assert _scan(b, d, u=0, delta=0, A=0, B=0, C=0, y=0, ws=0) == 0


def test_plan(b):
    # (with no GPU visible the library plans for 256 CUs)
    # the B8 L2048 D5120 layer has 640 channel tiles, all resident at once: one pass (the split
    # schedule, see test_plan_follows_the_cu_count)
    assert b.scan_plan(8, 2048, 5120, 16, 1) == (1, 2048)
    # more tiles than resident workgroups: still one grid pass (several rounds)
    assert b.scan_plan(16, 2048, 4096, 16, 1) == (1, 2048)
    # the long B1 L131072 D2048 sequence has 32 channel tiles: chunks of at most 512 tokens
    n, cl = b.scan_plan(1, 131072, 2048, 16, 1)
    assert cl <= 512 and cl % 32 == 0 and n * cl >= 131072 and (n - 1) * cl < 131072
    # B2 L2048 D1536 (48 tiles): one round of 768 work items
    assert b.scan_plan(2, 2048, 1536, 16, 0) == (16, 128)
    assert b.scan_plan(2, 300, 70, 4, 0, chunk_len=64) == (5, 64)
    assert b.scan_plan(2, 300, 70, 4, 0, chunk_len=-1) == (1, 300)
    assert b.scan_plan(1, 256, 16, 4, 0) == (1, 256)
    # a plain single pass needs no workspace; the split schedule holds its handed-over states
    # (128 tiles x 64 channels x 16 states fp32) and flags, the chunk carry its chunk states
    # split schedule: 128 handed-over states; 128 flags and 512 progress counters (2,560 B)
    assert b.workspace_bytes(8, 2048, 5120, 16, 1) == 128 * 64 * 16 * 4 + 2560
    assert b.workspace_bytes(16, 2048, 4096, 16, 1) == 0
    assert b.workspace_bytes(1, 131072, 2048, 16, 1) >= 256 * 2048 * 16 * 4
    assert b.workspace_bytes(1, 4096, 64, 16, 1, chunk_len=128) > b.workspace_bytes(1, 4096, 64, 16, 1, chunk_len=-1)


def test_plan_follows_the_cu_count(b):
    """ssm_scan_plan_info for devices of several CU counts (planning is host logic)."""
    # B8 L2048 D5120 N16 = 640 tiles.  256 CUs: 2.5 tiles per CU; 128 tiles run as two halves,
    # 512 + 2 x 128 = 768 workgroups = 3 per CU, each CU the work of 2.5 tiles
    p = b.plan_info(8, 2048, 5120, 16, 1, cu_count=256)
    assert p["cu_count"] == 256 and p["nchunk"] == 1 and p["chunk_len"] == 2048
    assert p["split_tiles"] == 128 and p["split_at"] == 1024 and p["workgroups"] == 768
    assert p["workspace_bytes"] == 128 * 64 * 16 * 4 + 2560
    # 304 CUs (2.1 tiles per CU): 3 x 304 - 640 = 272 tiles split, 912 workgroups
    p = b.plan_info(8, 2048, 5120, 16, 1, cu_count=304)
    assert p["split_tiles"] == 272 and p["workgroups"] == 912 and p["nchunk"] == 1
    # 200 CUs (3.2 tiles per CU): more than 2.5 per CU, a plain pass
    p = b.plan_info(8, 2048, 5120, 16, 1, cu_count=200)
    assert p["split_tiles"] == 0 and p["nchunk"] == 1 and p["workgroups"] == 640 and p["workspace_bytes"] == 0
    # 400 CUs (1.6 tiles per CU, L >= 512): the chunk carry, chunks of 512 tokens
    p = b.plan_info(8, 2048, 5120, 16, 1, cu_count=400)
    assert (p["nchunk"], p["chunk_len"], p["split_tiles"]) == (4, 512, 0) and p["workgroups"] == 2560
    # the small-batch carry follows the CU count too: B2 L2048 D1536 (48 tiles)
    assert (b.plan_info(2, 2048, 1536, 16, 0, cu_count=256)["nchunk"], b.plan_info(2, 2048, 1536, 16, 0,
            cu_count=256)["chunk_len"]) == (16, 128)
    p = b.plan_info(2, 2048, 1536, 16, 0, cu_count=64)
    assert (p["nchunk"], p["chunk_len"]) == (4, 512)
    # no split for another state size, a forced one pass, forced chunks or short sequences
    assert b.plan_info(8, 2048, 5120, 8, 1, cu_count=256)["split_tiles"] == 0
    assert b.plan_info(8, 2048, 5120, 16, 1, chunk_len=-1, cu_count=256)["split_tiles"] == 0
    assert b.plan_info(8, 2048, 5120, 16, 1, chunk_len=256, cu_count=256)["split_tiles"] == 0
    assert b.plan_info(8, 64, 5120, 16, 1, cu_count=256)["split_tiles"] == 0
    # an odd length: the second halves start on a 32-token boundary
    p = b.plan_info(8, 1001, 5120, 16, 0, cu_count=256)
    assert p["split_tiles"] == 128 and p["split_at"] == 512
    # cu_count <= 0 plans for the current device (256 without one)
    assert b.plan_info(8, 2048, 5120, 16, 1)["cu_count"] > 0


def test_noalloc_validation(b):
    """ssm_scan_fwd_noalloc refuses the checkpoints flag and plans needing more scratch than the
    library holds (64 MiB) before anything is launched."""
    P = ctypes.c_void_p

    def call(dims, flags=1):
        return b.lib.ssm_scan_fwd_noalloc(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, None, flags,
                                          P(FAKE), None, ctypes.byref(dims), None)
    assert call(_dims(b), flags=1 | 4) == -8               # SSM_ERR_FLAGS
    big = _dims(b, batch=1, seqlen=1 << 20, dim=4096, chunk_len=256)   # 4096 chunks x 4096 x 16 states
    assert b.lib.ssm_scan_workspace_bytes(ctypes.byref(big)) > 64 << 20
    assert call(big) == -6                                  # SSM_ERR_WORKSPACE
    assert "64" in b.last_error() or "67108864" in b.last_error()
    assert call(_dims(b, dstate=3)) == -5

"""ssm_scan_fwd_noalloc (the scan for callers that cannot allocate, its scratch in the
library's own device array) against ssm_scan_fwd on the same inputs and plan: bitwise equal
outputs, on two calls in a row whose second input is smaller (so the scratch holds the first
call's values when the second starts)."""
import numpy as np
import pytest

from selective_state_space_32_amd import inputs
from gpu_util import case_tensors

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from selective_state_space_32_amd import ssmscan  # noqa: E402


def _both(case, chunk_len=0):
    t = case_tensors(case, torch)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"])
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=case.softplus, chunk_len=chunk_len)
    y0, ls0 = ssmscan.scan_fwd(*args, **kw)
    y1 = torch.empty_like(y0)
    ls1 = torch.empty_like(ls0)
    ssmscan.scan_fwd_noalloc(*args, y=y1, last_state=ls1, **kw)
    torch.cuda.synchronize()
    return (y0, ls0), (y1, ls1)


@pytest.mark.parametrize("first,second", [
    # the chunk carry (scratch = chunk states), then a smaller carry
    (dict(bsz=1, L=8192, D=2048, N=16, io="bf16"), dict(bsz=2, L=1000, D=192, N=16, io="f32")),
    # the split schedule (scratch = handed-over states and flags), then a smaller split
    (dict(bsz=8, L=600, D=5120, N=16, io="bf16", gate=True), dict(bsz=8, L=300, D=5120, N=16, io="bf16")),
], ids=["carry then smaller carry", "split then smaller split"])
def test_noalloc_equals_scan_fwd_twice(first, second):
    for k, spec in enumerate((first, second)):
        case = inputs.scan_case(seed=700 + k, name=f"noalloc {k}", **spec)
        p = ssmscan.plan_info(case.bsz, case.L, case.D, case.N,
                              torch.bfloat16 if case.io == "bf16" else torch.float32)
        print(f"[noalloc call {k}] plan {p}", flush=True)
        assert p["workspace_bytes"] > 0
        (y0, ls0), (y1, ls1) = _both(case)
        assert torch.equal(y0, y1), k
        assert torch.equal(ls0, ls1), k


def test_noalloc_single_pass_and_flags():
    """A plan without scratch, and the exact ZOH, also through the no-allocation entry."""
    case = inputs.scan_case(bsz=2, L=257, D=96, N=8, io="f32", seed=720, name="noalloc small")
    t = case_tensors(case, torch)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"])
    for zoh in (False, True):
        kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], softplus=True, exact_zoh=zoh)
        y0, ls0 = ssmscan.scan_fwd(*args, **kw)
        y1, ls1 = torch.empty_like(y0), torch.empty_like(ls0)
        ssmscan.scan_fwd_noalloc(*args, y=y1, last_state=ls1, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(ls0, ls1), zoh

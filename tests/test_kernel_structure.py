"""Structure of the compiled persistent (chained) scan kernels, checked on the CPU.

The chained schedule claims work items from an atomic counter and broadcasts the claimed
index through LDS; the item loop contains workgroup barriers.  If the compiler cannot
prove the index uniform it may structurize the item loop as divergent control flow, so
that the claim ends up in an outer loop while the index read and the barriers sit in an
inner loop that can iterate without a new claim -- waves then fall out of step at the
barriers and the kernel stops making progress.  This test compiles the device code and
checks, for every chained kernel instantiation, that each read of the broadcast index
lies in the same loop as an atomic claim.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_32_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def loop_check(asm: str):
    """Yield (kernel name, ok, claim loops, index-read loops) per chained kernel."""
    for f in re.split(r"\n(?=_Z\S+:\s)", asm):
        name = f.split(":", 1)[0]
        if "scan_chunk_kernel" not in name or not re.search(r"Li2ELb[01]E", name):
            continue
        lines = f.split("\n")
        cur, loop_of = None, []
        for i, ln in enumerate(lines):
            m = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):\s*(;.*)?$", ln)
            if m:
                blk = m.group(1).lstrip(".L")
                c = m.group(2) or ""
                j = i + 1
                while j < len(lines) and re.match(r"^\s+;", lines[j]):
                    c += " " + lines[j]
                    j += 1
                if re.search(r"This (Inner )?Loop Header", c):
                    cur = blk
                else:
                    h = re.search(r"Header=(BB\d+_\d+)", c)
                    cur = h.group(1) if h else None
            loop_of.append(cur)
        claims = {loop_of[i] for i, l in enumerate(lines) if "global_atomic_add" in l}
        offs = [int(m.group(1)) for m in re.finditer(r"ds_read_b32 v\d+, v\d+ offset:(\d+)", f)]
        top = max(offs) if offs else None  # the index word sits above the LDS tiles
        reads = {loop_of[i] for i, l in enumerate(lines)
                 if top is not None and re.search(r"ds_read_b32 v\d+, v\d+ offset:%d\b" % top, l)}
        yield name, bool(claims) and reads <= (claims | {None}), claims, reads


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_chained_item_loop_is_uniform(tmp_path):
    out = tmp_path / "ssmscan.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, "ssmscan.hip")]
    subprocess.run(cmd, check=True, capture_output=True)
    res = list(loop_check(out.read_text()))
    assert len(res) >= 20, "expected a chained kernel per state size, I/O type and access width"
    bad = [(n[:70], c, r) for n, ok, c, r in res if not ok]
    assert not bad, bad

"""The grouped GEMM's per-step barrier waits count vector-memory instructions in issue order.

Each K step of `gemm_f8f4_kernel` issues its activation-tile loads into LDS (4 per wave, 5 in
wave 0) and then its weight-operand loads (NB per wave), and ends with
`s_waitcnt vmcnt(n) lgkmcnt(0); s_barrier`, n = 2 NB + 4: the next step's tile, issued one step
earlier, is complete once at most n newer loads are outstanding.  That holds only if the
compiled code keeps the order the source asks for.  This test compiles gemm.hip for gfx950
(on the CPU) and checks, for every kernel instantiation, that

* within each K step the loads into LDS come before the weight loads, and
* every barrier's vmcnt is at most the number of loads issued after the tile loads it waits for
  (the prologue's first step tile; else the previous segment's last run of tile loads), taking
  the 4 tile loads of waves other than 0 (the one-stage pipeline's first step waits for fewer
  loads than the steps after it),

so a compiler that reorders them fails here instead of racing on the GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

from fp4_routed_expert_moe_amd import build

KERNEL = re.compile(r"^(_ZN3moe16gemm_f8f4_kernel\S+):")
LOAD = re.compile(r"^\s*(buffer_load_\w+|global_load_\w+)\b(.*)$")
BARRIER_WAIT = re.compile(r"^\s*s_waitcnt vmcnt\((\d+)\) lgkmcnt\(0\)\s*$")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [build.hipcc(), *build.HIP_FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, "gemm.hip"),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def _kernels(lines):
    """kernel name -> its segments: [(loads between barriers, vmcnt of the closing barrier)]."""
    kernels, name, seg = {}, None, []
    for i, line in enumerate(lines):
        m = KERNEL.match(line)
        if m:
            name, seg = m.group(1), []
            kernels[name] = []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            name = None
            continue
        lm = LOAD.match(line)
        if lm:
            seg.append("D" if lm.group(2).rstrip().endswith(" lds") else "B")
        elif line.strip() == "s_barrier":
            wm = BARRIER_WAIT.match(lines[i - 1])
            kernels[name].append((seg, int(wm.group(1)) if wm else None))
            seg = []
    return kernels


def _runs(seg):
    out = []
    for t in seg:
        if out and out[-1][0] == t:
            out[-1][1] += 1
        else:
            out.append([t, 1])
    return out


def _newer(runs):
    """Loads in `runs` as a wave other than 0 issues them (a run of 5 tile loads is 4 there)."""
    return sum(c - (1 if t == "D" and c == 5 else 0) for t, c in runs)


def test_gemm_tile_loads_precede_weight_loads_and_barrier_counts_hold(gemm_asm):
    kernels = _kernels(gemm_asm)
    assert len(kernels) >= 5, sorted(kernels)
    for name, segs in kernels.items():
        checked = 0
        for k, (seg, n) in enumerate(segs):
            if n is None:  # the epilogue's barriers
                continue
            runs = _runs(seg)
            d_runs = [i for i, (t, _) in enumerate(runs) if t == "D"]
            if len(d_runs) >= 2:
                # the prologue: its first step's tile must be complete
                newer = _newer(runs[d_runs[0] + 1:])
            else:
                # one K step: its tile loads come first; the tile it waits for was the last run of
                # tile loads of the segment before (the prologue or the previous step)
                assert len(d_runs) == 1 and d_runs[0] == 0, (name, k, "".join(seg))
                prev = _runs(segs[k - 1][0])
                last_d = max(i for i, (t, _) in enumerate(prev) if t == "D")
                newer = _newer(prev[last_d + 1:]) + _newer(runs)
            assert n <= newer, (name, k, n, newer, "".join(seg))
            checked += 1
        assert checked >= 4, (name, checked)

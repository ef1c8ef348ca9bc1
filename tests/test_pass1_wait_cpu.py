"""The column pass's copies of the chi_q block into the LDS must have landed before the
workgroup barrier that precedes the correction, while the spectrum loads issued after
them may stay in flight.  The wait before that barrier is the compiler's own; this test
reads the gfx950 assembly of this build and checks that it covers every copy: with K
vector memory operations issued after the last copy and before the wait, a
``s_waitcnt vmcnt(c)`` covers the copies when c <= K (vector memory operations of one
wave complete in issue order)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "aberration_phase_variance_amd", "csrc")
VMEM = re.compile(r"^\s*(buffer_|global_|scratch_|flat_)(load|store|atomic)")


def _device_asm(tmp):
    from aberration_phase_variance_amd import build as B
    out = os.path.join(tmp, "kernels.s")
    cmd = [B.hipcc()] + [f for f in B.flags() if f not in ("-shared", "-fPIC")] + [
        "--cuda-device-only", "-S", os.path.join(CSRC, "ssb_kernels.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def _functions(asm, pattern):
    names = re.findall(r"^(_Z\w+):", asm, flags=re.M)
    for name in names:
        if re.search(pattern, name):
            start = asm.index(f"\n{name}:")
            end = asm.find(".Lfunc_end", start)
            yield name, asm[start:end].splitlines()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
def test_chi_copies_waited_for_before_barrier(tmp_path):
    """Every group of copies to the LDS (one per trial a workgroup handles) is covered by a
    wait before the next barrier; in the single-trial kernels the 16 spectrum loads issued
    after the copies are not waited for there (they stay in flight)."""
    asm = _device_asm(str(tmp_path))
    found = {1: 0, 8: 0}
    for name, lines in _functions(asm, r"k_pass1ILi512ELi8ELb[01]ELi[18]E"):
        tb = int(re.search(r"Lb[01]ELi(\d+)E", name).group(1))
        found[tb] += 1
        copies = [i for i, ln in enumerate(lines) if VMEM.match(ln) and ln.rstrip().endswith(" lds")]
        assert copies, name
        # the last copy of each group: a copy whose next copy (if any) lies past a barrier
        groups = []
        for idx, i in enumerate(copies):
            nxt = copies[idx + 1] if idx + 1 < len(copies) else None
            if nxt is None or any(lines[q].strip() == "s_barrier" for q in range(i, nxt)):
                groups.append(i)
        for g in groups:
            barrier = next(i for i in range(g, len(lines)) if lines[i].strip() == "s_barrier")
            issued = 0
            covered = False
            for ln in lines[g + 1:barrier]:
                if VMEM.match(ln):
                    issued += 1
                m = re.match(r"^\s*s_waitcnt\s+.*vmcnt\((\d+)\)", ln)
                if m and int(m.group(1)) <= issued:
                    covered = True
            assert covered, f"{name}: no wait covering the chi_q copies before the barrier ({issued} issued after)"
            if tb == 1:
                assert issued >= 16, name
    assert found == {1: 2, 8: 2}, found

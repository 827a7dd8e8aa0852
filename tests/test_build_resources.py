"""The streaming kernels schedule their vector-memory loads explicitly (exact
vmcnt waits); a register spill would add scratch traffic the waits do not count
and could copy a register whose load is still in flight.  This compiles the
library for gfx950 with resource-usage remarks and requires zero spills and zero
scratch for every kernel (no GPU needed); SGPR spills (kept in VGPR lanes) are allowed."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "block_diffusion_drafter_states_amd", "csrc", "dflash.hip")


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_register_spills_or_scratch(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-c", "-fPIC", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"),
           SRC, "-o", str(tmp_path / "dflash.o")]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    text = res.stderr
    names = re.findall(r"Function Name: (\S+)", text)
    spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", text)]
    sspills = [int(x) for x in re.findall(r"SGPRs Spill: (\d+)", text)]
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    assert len(names) >= 10 and len(names) == len(spills) == len(scratch) == len(sspills)
    # SGPR spills land in VGPR lanes (no memory traffic) and are allowed; VGPR spills and
    # any scratch use are not
    bad = [(n, v, sc) for n, v, sc in zip(names, spills, scratch) if v or sc]
    assert not bad, f"kernels with VGPR spills / scratch: {bad}"

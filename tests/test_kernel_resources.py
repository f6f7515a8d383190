"""Compile-time checks of the HIP kernels (CPU only: hipcc cross-compiles
gfx950): no kernel may use private (scratch) memory -- a register array
that lands in scratch turns every load of it into a round trip to memory --
and the expert GEMMs must fit two workgroups per CU."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_symmetric_memory_amd", "csrc")


def _usage(src):
    from combine_symmetric_memory_amd.build import HIPCC_FLAGS, hipcc
    out = os.path.join("/tmp", "cco_res_%d.o" % os.getpid())
    r = subprocess.run([hipcc(), *HIPCC_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src),
                        "-o", out, "-Rpass-analysis=kernel-resource-usage"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    cur = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: \s*([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["plan.hip", "dispatch.hip", "combine.hip", "expert.hip"])
def test_no_scratch(src):
    ks = _usage(src)
    assert ks, "no kernels reported for " + src
    for name, u in ks.items():
        assert u.get("ScratchSize", 0) == 0, "%s uses scratch: %s" % (name, u)
        if "grouped_gemm" in name:
            assert u.get("Occupancy", 0) >= 2, "%s occupancy %s" % (name, u)

"""Compile-time checks of the HIP kernels (CPU only: hipcc cross-compiles
gfx950).  A register array that lands in private (scratch) memory turns
every access into a round trip to memory: plan, dispatch and combine may use
no scratch at all, and the expert GEMMs none inside their MFMA loops (their
per-tile setup may spill a few loop-invariant values)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_symmetric_memory_amd", "csrc")


def _usage(src, defines=()):
    from combine_symmetric_memory_amd.build import HIPCC_FLAGS, hipcc
    out = os.path.join("/tmp", "cco_res_%d.o" % os.getpid())
    r = subprocess.run([hipcc(), *HIPCC_FLAGS, *["-D" + d for d in defines], "-x", "hip", "-c",
                        os.path.join(CSRC, src), "-o", out, "-Rpass-analysis=kernel-resource-usage"],
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
        if "grouped_gemm" in name:
            continue
        assert u.get("ScratchSize", 0) == 0, "%s uses scratch: %s" % (name, u)


def _asm(src):
    from combine_symmetric_memory_amd.build import HIPCC_FLAGS, hipcc
    out = os.path.join("/tmp", "cco_asm_%d.s" % os.getpid())
    r = subprocess.run([hipcc(), *HIPCC_FLAGS, "-x", "hip", "--cuda-device-only", "-S",
                        os.path.join(CSRC, src), "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_gemm_mfma_loops_touch_no_scratch():
    text = _asm("expert.hip")
    blocks = re.split(r"\n(?=\.LBB\d+_\d+:)", text)
    hot = [b for b in blocks if b.count("v_mfma") >= 8]
    assert hot, "no MFMA loop found"
    for b in hot:
        assert "scratch_" not in b, "scratch access inside an MFMA loop:\n" + b[:400]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_switched_off_single_launch_kernel_still_builds():
    # The single-launch kernel is left out of the library (its entry point
    # reports CCO_ERR_DISABLED) but shares its device code with the other
    # kernels; it must keep compiling against them, without scratch.
    ks = _usage("fused.hip", defines=("CCO_BUILD_FUSED",))
    fused = {n: u for n, u in ks.items() if "fused_kernel" in n}
    assert len(fused) == 3, sorted(ks)
    for name, u in fused.items():
        assert u.get("ScratchSize", 0) == 0, "%s uses scratch: %s" % (name, u)

"""Resource use of the persistent kernels, from the compiler (no GPU needed): every decode
and prompt kernel, of every body, and every tile count of the persistent prompt prefill,
runs with no scratch memory (no register spilled to memory: a reload would wait for
every load the wave has in flight, weight streams included) and within the 256
registers a wave may hold at two waves per SIMD."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "persistent_megakernel_loop_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _usage(tmp_path_factory, source):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc is not installed")
    out = tmp_path_factory.mktemp("res") / "k.o"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--offload-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, source), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    funcs, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = funcs.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return funcs


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    return _usage(tmp_path_factory, "mk_kernel.hip")


@pytest.fixture(scope="module")
def prefill_usage(tmp_path_factory):
    return _usage(tmp_path_factory, "mk_pprefill.hip")


def test_persistent_prefill_kernels_have_no_scratch(prefill_usage):
    """The persistent prompt prefill, at each of its tile counts (16 to 64 positions)."""
    kernels = {n: u for n, u in prefill_usage.items() if "pp_kernel" in n}
    assert len(kernels) == 4, sorted(kernels)
    for name, u in kernels.items():
        assert u.get("ScratchSize") == 0, (name, u)
        assert u.get("VGPRs Spill") == 0, (name, u)
        assert u.get("VGPRs", 999) <= 256, (name, u)


def test_persistent_kernels_have_no_scratch(usage):
    kernels = {n: u for n, u in usage.items() if "decode_kernel" in n or "prefill_kernel" in n}
    # three bodies; the hidden-1024 bf16 body also has its whole-attention form
    assert len(kernels) == 8, sorted(kernels)
    for name, u in kernels.items():
        assert u.get("ScratchSize") == 0, (name, u)
        assert u.get("VGPRs Spill") == 0, (name, u)
        assert u.get("VGPRs", 999) <= 256, (name, u)

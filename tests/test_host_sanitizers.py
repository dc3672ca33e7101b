"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
same sources built with the sanitizers on the host side only, then the C-ABI tests
(argument validation, error codes, exported symbols) run against that build in a child
process with the sanitizer runtime preloaded.  Any report aborts the child."""
import os
import subprocess
import sys

from persistent_megakernel_loop_amd import build as B


def test_abi_suite_clean_under_host_asan_ubsan(tmp_path):
    lib = B.build_host_sanitized(str(tmp_path / "libmk_hostsan.so"))
    env = B.sanitizer_env(lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(B.ROOT, "tests", "test_abi.py")],
                       cwd=B.ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail

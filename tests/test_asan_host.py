"""The C ABI's host code under AddressSanitizer (CPU only).

The library is rebuilt with the sanitizer on its host pass only (every
-fsanitize flag directly after -Xarch_host; device code is built as usual and
never runs here), and tests/test_abi.py -- argument validation, error
messages, the launch plan, exported symbols -- runs against it in a child
process with the sanitizer runtime preloaded.  Any report fails the test.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from means_nearest_centroid_amd import build as kbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def asan_library(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    if _asan_runtime() is None:
        pytest.skip("AddressSanitizer runtime not found")
    out = str(tmp_path_factory.mktemp("asan") / "libkmeans_mi355x.so")
    host_asan = ["-Xarch_host -fsanitize=address", "-Xarch_host -fno-omit-frame-pointer"]
    cmd = [kbuild.hipcc(), f"--offload-arch={kbuild.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
           "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *" ".join(host_asan).split(), "-I", kbuild.INCLUDE, "-I", kbuild.CSRC,
           *kbuild.SOURCES, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out


def test_abi_suite_under_address_sanitizer(asan_library):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86"
    env["KMEANS_MI355X_LIBRARY"] = asan_library
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                          "-q", "-s", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out and res.returncode != 86, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out

"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer of the C
oracles and of the host side of the C ABI (validation, workspace sizing, segment
planners), each driven through its entry points on small inputs by a driver in
tests/sanitize/.  A report of an out-of-bounds access, a use of freed memory, a
leak (oracle) or undefined arithmetic fails the test.  CPU only: the host driver
never reaches a kernel launch (its launchers are stubs that abort)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "hybrid_sparse_linear_la_amd", "csrc")


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, f"{exe} failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "clean" in res.stdout


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    subprocess.check_call([gcc, "-std=c11", "-g", "-O1", "-fopenmp", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                           os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "la_oracle.c"),
                           os.path.join(ROOT, "oracle", "sparse_oracle.c"), "-o", exe, "-lm"])
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})


def test_host_abi_under_sanitizers(tmp_path):
    from hybrid_sparse_linear_la_amd import _build
    exe = str(tmp_path / "host_san")
    # sanitizers on the host code only; the device code is built as usual
    subprocess.check_call([_build.hipcc(), f"--offload-arch={_build.ARCH}", "-std=c++17", "-g", "-O1",
                           "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                           "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           os.path.join(SAN, "host_driver.cpp"), os.path.join(CSRC, "la_api.hip"), "-o", exe])
    # the HIP runtime's own start-up allocations are not the library's: no leak check
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The fp64 oracle, built with gcc and the sanitizers into a C driver that runs
  every oracle entry point on small seeded problems (tests/sanitize/
  oracle_driver.c).
- The host side of the C ABI, built with the sanitizers on the host pass only
  (the device code is compiled as usual and never launched), linked into a
  C++ driver that sweeps workspace sizing and launch plans over ordinary,
  ragged, limit and invalid shapes and calls every entry point's argument
  checks (tests/sanitize/abi_driver.cpp).
Either driver aborts on the first memory or undefined-behaviour error.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ROOT / "tests" / "sanitize"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(exe, **env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=e, timeout=600)
    assert r.returncode == 0, f"{exe.name} failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", *SAN_FLAGS, "-o", str(exe), str(SAN / "oracle_driver.c"),
                    str(ROOT / "oracle" / "pararnn_oracle.c"), "-lm", "-lpthread"], check=True)
    out = _run(exe, ASAN_OPTIONS="detect_leaks=1")
    assert "all checks passed" in out


def test_abi_host_code_under_asan_ubsan(tmp_path):
    from nonlinear_rnn_solve_newton_amd import build

    clang = Path(os.environ.get("ROCM_PATH", "/opt/rocm")) / "lib" / "llvm" / "bin" / "clang++"
    if not clang.exists() or not Path(build.hipcc()).exists():
        pytest.skip("ROCm compilers not available")
    lib = tmp_path / "libpararnn_san.so"
    host = []
    for f in SAN_FLAGS:  # each sanitizer flag goes to the host pass only
        host += ["-Xarch_host", f]
    build.build_one(build.CSRC / "pararnn.hip", lib, host_flags=host)
    exe = tmp_path / "abi_driver"
    subprocess.run([str(clang), "-std=c++17", *SAN_FLAGS, str(SAN / "abi_driver.cpp"), f"-L{tmp_path}",
                    "-lpararnn_san", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)], check=True)
    # the HIP runtime the library links keeps allocations until exit: no leak report
    out = _run(exe, ASAN_OPTIONS="detect_leaks=0")
    assert "all checks passed" in out

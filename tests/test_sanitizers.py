"""Host address and undefined-behaviour sanitizer builds (CPU only, no GPU call).

* The C ABI's host code (api.cpp: validation, schedule choice, argument blocks) built by hipcc with the
  host-side sanitizers (device code untouched), kernel launchers replaced by host stubs
  (sanitize/stub_launch.cpp), driven through every entry point by sanitize/abi_driver.cpp.
* The fp64 oracle (oracle/oracle.c) built by gcc with the same sanitizers, driven by
  sanitize/oracle_driver.c on tiny inputs in every mode.
Any sanitizer report aborts the driver (non-zero exit)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "paged_skip_softmax_amd", "csrc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    base = ["hipcc", "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", "-x", "hip", *inc, *HOST_SAN]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(SAN, "stub_launch.cpp"), os.path.join(SAN, "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([*base, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_asan")
    _run(["hipcc", "--offload-arch=gfx950", *HOST_SAN, *objs, "-o", exe])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "0 unexpected statuses" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env={**os.environ, "OMP_NUM_THREADS": "2"})
    assert "0 failures" in r.stdout

"""The C-ABI layer (argument checking, error reporting, dispatch) built with
AddressSanitizer and UndefinedBehaviorSanitizer on the host, with the kernel
launchers replaced by recording stubs (tests/sanitize/stub_launchers.cpp), and
driven through every entry point by tests/sanitize/abi_driver.cpp: valid calls
must reach a launcher, invalid ones must return their status with a message,
and neither may trip a sanitizer.  Runs on the CPU; the sanitizers apply to
host code only."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["-O1", "-g", "-std=c++17", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not present")
@pytest.mark.timeout(600)
def test_abi_layer_under_asan_ubsan(tmp_path):
    abi = os.path.join(ROOT, "sparse_attention_hca_amd", "csrc", "hca_abi.cpp")
    # the ABI source holds a __device__ array, so it is compiled with its device part; the rest is host-only
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", *SAN, "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-c", abi, "-o", str(tmp_path / "abi.o")])
    for name in ("stub_launchers", "abi_driver"):
        _run([HIPCC, "-x", "hip", "--cuda-host-only", *SAN, "-c", os.path.join(ROOT, "tests", "sanitize", name + ".cpp"),
              "-o", str(tmp_path / (name + ".o"))])
    exe = str(tmp_path / "abi_san")
    _run([CLANG, "-fsanitize=address", "-fsanitize=undefined", str(tmp_path / "abi.o"),
          str(tmp_path / "stub_launchers.o"), str(tmp_path / "abi_driver.o"), "-L/opt/rocm/lib",
          "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ALL OK" in r.stdout, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]

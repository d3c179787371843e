"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/oracle.c) built with gcc's sanitizers and driven by
  tests/sanitize/oracle_drive.c: every entry point on exact-size buffers, the
  written-out and FFT routes checked against each other, leaks reported.
* The C ABI's host code (api.cpp: argument checks, planning, channel chunks,
  workspace layout, error mapping) built with the sanitizers on its host pass
  and linked with host stand-ins for the kernel launchers
  (tests/sanitize/stub_launch.cpp), driven by tests/sanitize/abi_drive.c.  The
  stand-ins touch the ends of every region a launch would use, so a chunk or
  offset that leaves the caller's buffer is a sanitizer report; a failing
  launch status checks the mapping to HYENAND_ERR_HIP.

Each build goes to a temporary directory; nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-D_GNU_SOURCE", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(SAN, "oracle_drive.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert r.stdout.strip().endswith("0 failed expectation(s)"), r.stdout


def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
@pytest.mark.skipif(_gpu_visible(), reason="the launcher stand-ins treat device pointers as host memory: "
                                           "the sanitizer build runs only where no GPU is visible")
def test_abi_host_code_under_sanitizers(tmp_path):
    inc = os.path.join(ROOT, "include")
    flags = ["-std=c++20", "-O1", "-g", "--offload-arch=gfx950", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc] + HOST_SAN
    api_o, stub_o, drv_o = (str(tmp_path / n) for n in ("api.o", "stub.o", "drive.o"))
    _run([HIPCC] + flags + ["-x", "hip", "-c", os.path.join(ROOT, "dimensional_fft_long_amd", "csrc", "api.cpp"),
                            "-o", api_o])
    _run([HIPCC] + flags + ["-x", "hip", "-c", os.path.join(SAN, "stub_launch.cpp"), "-o", stub_o])
    _run([CLANG, "-std=c99", "-O1", "-g", "-I", inc, "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(SAN, "abi_drive.c"), "-o", drv_o])
    exe = str(tmp_path / "abi_san")
    _run([CLANGXX, "-fsanitize=address,undefined", drv_o, api_o, stub_o, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # The HIP runtime's own allocations are not this library's: leaks are not checked here.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([exe], env=env, timeout=300)
    assert "ok: 0 failed expectation(s)" in r.stdout, r.stdout

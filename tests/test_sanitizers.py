"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (oracle/scan_oracle.c) is built with gcc and both sanitizers and
  driven by tests/sanitize/oracle_driver.c over exactly sized heap buffers.
- The scan library's host code (the C ABI and the single-pass host logic) is
  built with both sanitizers on the host side only; its device code is the
  library's own, unchanged. tests/sanitize/abi_driver.c, a plain C caller,
  drives every entry point's validation, the status strings and the
  tile-geometry queries, all of which return before any HIP call.

Any sanitizer report or failed check fails the test. Leak checking is on for
the oracle; for the library it is off, since the HIP runtime it links keeps
allocations of its own until exit."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
ENV_UBSAN = "print_stacktrace=1:halt_on_error=1"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _gcc():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    return gcc


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run([_gcc(), "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "scan_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS=ENV_UBSAN)
    r = _run([exe], env=env, timeout=120)
    assert "oracle driver: ok" in r.stdout


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    from device_wide_prefix_amd import build as hip_build
    host_sources = ("dws_abi.cpp", "dws_single_pass_host.cpp")
    device_objs = [os.path.join(hip_build.BUILD_DIR, os.path.splitext(s)[0] + ".o")
                   for s in hip_build.SOURCES if s not in host_sources]
    if not all(os.path.exists(o) for o in device_objs):
        hip_build.build(verbose=False)
    flags = [f"--offload-arch={hip_build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{hip_build.INCLUDE}", f"-I{hip_build.CSRC}",
             # host side only: the device code is built exactly as in the library
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    for src in host_sources:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, *flags, "-x", "hip", "-c", os.path.join(hip_build.CSRC, src), "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    _run([_gcc(), "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
          f"-I{hip_build.INCLUDE}", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c", os.path.join(SAN, "abi_driver.c"),
          "-o", drv])
    exe = str(tmp_path / "abi_driver")
    # link line: host sanitizer runtimes, no GPU sanitizer
    _run([HIPCC, f"--offload-arch={hip_build.ARCH}", "-fno-gpu-sanitize", "-fsanitize=address,undefined",
          drv, *objs, *device_objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS=ENV_UBSAN)
    r = _run([exe], env=env, timeout=120)
    assert "abi driver: ok" in r.stdout

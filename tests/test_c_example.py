"""The C ABI used from a C program (device_wide_prefix_amd/examples/
scan_from_c.c): it compiles against include/dws_scan.h and the built library
here; on a GPU it runs a scan, a compaction and a two-shard scan (dws_reduce,
dws_scan_seeded) and checks them itself."""
import os
import subprocess

import pytest

import device_wide_prefix_amd as dws

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "device_wide_prefix_amd", "examples", "scan_from_c.c")


def _build(tmp_path):
    if not os.path.exists(dws.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    exe = os.path.join(str(tmp_path), "scan_from_c")
    libdir = os.path.dirname(dws.LIB_PATH)
    cmd = ["/opt/rocm/bin/hipcc", "-O2", "-x", "c", SRC, "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-L", libdir, "-ldws_scan", "-L/opt/rocm/lib",
           "-lamdhip64", f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_example_compiles(tmp_path):
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
def test_c_example_runs(gpu, tmp_path):
    exe = _build(tmp_path)
    for n in ("1", "4097", "10000019"):
        r = subprocess.run([exe, n], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "correct" in r.stdout

"""Host-side logic of bench.py that runs without a GPU: the source fingerprint
that decides whether the stored HBM counters still apply, the stored counter
summary itself, and the refusal of a multi-GPU run."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_strip_comments_keeps_code_and_literals():
    src = 'int a = 1; // one\n/* two\n three */ char c = \'/\';\nconst char* s = "x // y \\" /* z */";  int  b;'
    assert bench.strip_comments(src) == 'int a = 1; char c = \'/\'; const char* s = "x // y \\" /* z */"; int b;'


def test_fingerprint_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "device_wide_prefix_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("__global__ void k(int* p) { p[0] = 1; }\n")
    base = bench.kernel_source_sha(("k.hip",))
    (csrc / "k.hip").write_text("// a note\n__global__ void k(int* p)\n{\n    p[0] = 1;  /* stored */\n}\n")
    assert bench.kernel_source_sha(("k.hip",)) == base
    (csrc / "k.hip").write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.kernel_source_sha(("k.hip",)) != base


def test_stored_traffic_is_consistent_and_current():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert sorted(t["kernel_sources"]) == sorted(bench.SINGLE_PASS_SOURCES)
    scaled = (t["fetch_size_kib_per_dispatch"] * t["fetch_scale"] + t["write_size_kib_per_dispatch"] *
              t["write_scale"]) * 1024
    assert abs(scaled - t["bytes_per_launch"]) <= 1024
    # 2 x 2^28 x 4 B moved, plus the descriptors and their polls: within 1%
    assert 1.0 <= t["bytes_per_launch"] / 2**31 < 1.01
    # the committed counters were taken on the committed kernel sources
    assert bench.traffic_for_current_kernel() == t["bytes_per_launch"]


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""

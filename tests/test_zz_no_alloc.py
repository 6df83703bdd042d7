"""dws_scan_noalloc, the scan entry point that allocates nothing, against the
entry points it is a variant of (scan_inclusive / scan_exclusive), called
through the C ABI on raw device pointers.

Bar: 32-bit integers bit-exact against the existing entry point's output (and
the oracle); fp32 both results within 1e-4 * sum_{j<=i}|x_j| + 1e-6 of the
fp64 oracle (the order of fp32 additions depends on scheduling, so the two
results need not share bits). Two calls in a row, the second smaller, so the
second runs on the array the first left behind.
"""
import numpy as np
import pytest

import device_wide_prefix_amd as dws
import scan_workloads as wl
from gpu_util import CODE, check, from_device, note, to_device

pytestmark = pytest.mark.gpu


def _noalloc(xd, out, n, dtype, exclusive):
    import torch
    st = dws.scan_noalloc_ptr(xd.data_ptr(), out.data_ptr(), n, CODE[dtype], exclusive,
                              torch.cuda.current_stream().cuda_stream)
    assert st == dws.OK, dws.status_string(st)


def _existing(xd, out, n, dtype, exclusive):
    import torch
    f = dws.scan_exclusive_ptr if exclusive else dws.scan_inclusive_ptr
    st = f(xd.data_ptr(), out.data_ptr(), n, CODE[dtype], torch.cuda.current_stream().cuda_stream)
    assert st == dws.OK, dws.status_string(st)


def _both(x, dtype, exclusive, in_place=False, offset=0):
    """(no-alloc result, existing entry point's result) on the same input."""
    import torch
    _, xd = to_device(x, extra_front=offset)
    if in_place:
        out_a = xd
    else:
        out_a = torch.empty(x.size + offset, dtype=xd.dtype, device="cuda")[offset:]
    _noalloc(xd, out_a, x.size, dtype, exclusive)
    a = from_device(out_a, dtype)
    _, xd2 = to_device(x, extra_front=offset)
    out_b = xd2 if in_place else torch.empty_like(xd2)
    _existing(xd2, out_b, x.size, dtype, exclusive)
    b = from_device(out_b, dtype)
    return a, b


def _compare(x, a, b, dtype, exclusive, label):
    check(x, a, dtype, exclusive, label=f"no-alloc {label}")
    check(x, b, dtype, exclusive, label=f"existing {label}")
    if dtype != "float32":
        assert np.array_equal(a, b), label


# sizes: the automatic shapes with and without non-temporal loads, ragged
# multi-tile sizes and one tile
SIZES_FIRST_SECOND = [((1 << 25) + 777, (1 << 22) + 3), ((1 << 23) + 5, 70_001), (300_001, 4097)]


@pytest.mark.parametrize("dtype", ["int32", "uint32", "float32"])
@pytest.mark.parametrize("exclusive", [False, True])
@pytest.mark.parametrize("sizes", SIZES_FIRST_SECOND, ids=lambda s: f"{s[0]}then{s[1]}")
def test_noalloc_matches_existing_entry_two_calls(gpu, dtype, exclusive, sizes):
    for k, n in enumerate(sizes):
        note(f"noalloc {dtype} excl={exclusive} call {k + 1}: n={n}")
        x = wl.random_input(dtype, n, seed=1000 + 7 * k + n % 97)
        a, b = _both(x, dtype, exclusive)
        _compare(x, a, b, dtype, exclusive, f"{dtype} n={n} call {k + 1}")


@pytest.mark.parametrize("dtype", ["int32", "float32"])
def test_noalloc_in_place_and_unaligned(gpu, dtype):
    for n, offset in (((1 << 24) + 11, 0), (1_000_003, 1), (65_537, 3)):
        for in_place in (True, False):
            note(f"noalloc {dtype} n={n} offset={offset} in_place={in_place}")
            x = wl.random_input(dtype, n, seed=n + offset)
            a, b = _both(x, dtype, True, in_place=in_place, offset=offset)
            _compare(x, a, b, dtype, True, f"{dtype} n={n} offset={offset} in_place={in_place}")


def test_noalloc_at_the_headline_size(gpu):
    """N = 2^28 fp32 exclusive in place, the benchmark's workload, then a
    smaller int32 call on the same array."""
    w = wl.WORKLOADS["f32_2p28_excl_inplace"]
    x = wl.generate_workload(w)
    note("noalloc 2^28 fp32 exclusive in place")
    a, b = _both(x, "float32", True, in_place=True)
    _compare(x, a, b, "float32", True, "2^28 fp32")
    del a, b
    x2 = wl.random_input("int32", (1 << 26) + 9, seed=77)
    note("noalloc then 2^26 + 9 int32 inclusive")
    a, b = _both(x2, "int32", False)
    _compare(x2, a, b, "int32", False, "2^26+9 int32")


def test_noalloc_interleaved_with_workspace_calls_and_graph(gpu):
    """No-alloc calls between workspace calls on the same stream, then one
    captured into a graph and replayed with eager work between the replays;
    every replay is checked."""
    import torch
    n = (1 << 22) + 123
    x = wl.random_input("int32", n, seed=5)
    want_incl = None
    for k in range(3):
        note(f"interleaved round {k}")
        a, b = _both(x, "int32", k % 2 == 1)
        _compare(x, a, b, "int32", k % 2 == 1, f"interleaved {k}")
        if k % 2 == 0:
            want_incl = a
    _, xd = to_device(x)
    out = torch.empty_like(xd)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("capture a no-alloc call")
    with torch.cuda.graph(g, stream=s):
        st = dws.scan_noalloc_ptr(xd.data_ptr(), out.data_ptr(), n, dws.INT32, False, s.cuda_stream)
    assert st == dws.OK, dws.status_string(st)
    for r in range(4):
        note(f"replay {r}")
        out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_device(out, "int32"), want_incl), f"replay {r}"
        # eager no-alloc work between the replays, on another size
        a, b = _both(x[: n // 3], "int32", True)
        _compare(x[: n // 3], a, b, "int32", True, f"between replays {r}")
    del g


def test_noalloc_watchdog_never_tripped(gpu):
    assert dws.watchdog_trips() == 0

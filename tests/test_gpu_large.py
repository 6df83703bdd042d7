"""GPU scans past 2^32 elements and at the largest supported count (2^35,
DWS_MAX_ELEMENTS in include/dws_scan.h), in place.

An all-ones input has a closed form: the exclusive scan is y[i] = i and the
inclusive one y[i] = i + 1, modulo 2^32 for 32-bit integers, so the result is
checked on the GPU slice by slice at any size. These sizes exercise 64-bit
element offsets, more than 2^16 tiles and the wrap of 32-bit sums, which the
seeded workloads (at most 2^30 elements) do not reach."""
import pytest

import device_wide_prefix_amd as dws
from gpu_util import note

pytestmark = pytest.mark.gpu

MAX_ELEMENTS = 1 << 35
SLICE = 1 << 28


def _need(nbytes: int):
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes + (2 << 30):
        pytest.skip(f"needs {nbytes >> 30} GiB of free device memory, {free >> 30} GiB free")


def _check_ramp(y, n: int, first: int, label: str):
    """y[i] == (first + i) mod 2^32 for every i, compared slice by slice."""
    import torch
    for s in range(0, n, SLICE):
        e = min(n, s + SLICE)
        want = torch.arange(s + first, e + first, dtype=torch.int64, device=y.device) & 0xFFFFFFFF
        got = y[s:e].to(torch.int64) & 0xFFFFFFFF
        if not torch.equal(got, want):
            i = int(torch.nonzero(got != want)[0])
            raise AssertionError(f"{label}: y[{s + i}] = {int(got[i])}, want {int(want[i])}")


@pytest.mark.parametrize("exclusive", [True, False], ids=["exclusive", "inclusive"])
@pytest.mark.parametrize("n", [(1 << 32) + 12345, MAX_ELEMENTS], ids=["2^32+12345", "2^35"])
def test_all_ones_past_32_bits(gpu, n, exclusive):
    import torch
    _need(4 * n)
    note(f"all-ones int32 scan n={n} exclusive={exclusive}, in place")
    x = torch.ones(n, dtype=torch.int32, device="cuda")
    try:
        (dws.scan_exclusive if exclusive else dws.scan_inclusive)(x, out=x)
        torch.cuda.synchronize()
        _check_ramp(x, n, 0 if exclusive else 1, f"n={n} exclusive={exclusive}")
    finally:
        del x
        torch.cuda.empty_cache()
    assert dws.watchdog_trips() == 0

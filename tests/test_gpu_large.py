"""GPU scans (and totals) past 2^32 elements and at the largest supported
count (2^35, DWS_MAX_ELEMENTS in include/dws_scan.h), in place.

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


@pytest.mark.parametrize("n", [(1 << 32) + 12345, MAX_ELEMENTS], ids=["2^32+12345", "2^35"])
def test_reduce_and_seeded_scan_past_32_bits(gpu, n):
    # the + of n ones is n (mod 2^32 for int32; fp32 within the bar of the
    # scans), and the exclusive scan of ones seeded with s is s + i
    import torch
    _need(4 * n)
    x = torch.ones(n, dtype=torch.int32, device="cuda")
    try:
        note(f"reduce of n={n} int32 ones")
        assert int(dws.reduce(x).item()) & 0xFFFFFFFF == n & 0xFFFFFFFF
        note(f"reduce of n={n} fp32 ones")
        xf = x.view(torch.float32)
        xf.fill_(1.0)
        total = float(dws.reduce(xf).item())
        assert abs(total - n) <= 1e-4 * n + 1e-6, total
        note(f"seeded exclusive scan of n={n} int32 ones, seed 7, in place")
        x.fill_(1)
        seed = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        dws.scan_seeded(x, seed, exclusive=True, out=x)
        torch.cuda.synchronize()
        _check_ramp(x, n, 7, f"seeded n={n}")
    finally:
        del x
        torch.cuda.empty_cache()
    assert dws.watchdog_trips() == 0


# The compaction family takes n below 2^32 (counts travel in 32-bit descriptor
# values): 2^32 - 1 is its largest input.
COMPACTION_MAX = (1 << 32) - 1


def _fill(t, n: int, fn):
    """t[i] = fn(i) (an int64 tensor expression of the indices), slice by slice."""
    import torch
    for s in range(0, n, SLICE):
        e = min(n, s + SLICE)
        t[s:e] = fn(torch.arange(s, e, dtype=torch.int64, device=t.device)).to(t.dtype)


def test_select_at_the_count_limit(gpu):
    # x[i] = i mod 2^32, selected where i mod 3 != 0; the j-th selected index
    # is 3 (j // 2) + j % 2 + 1
    import torch
    n = COMPACTION_MAX
    _need(12 * n)
    note(f"select n={n} (i mod 3 != 0)")
    x = torch.empty(n, dtype=torch.int32, device="cuda")
    flags = torch.empty(n, dtype=torch.int32, device="cuda")
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    try:
        _fill(x, n, lambda i: (i & 0xFFFFFFFF) - ((i & 0x80000000) << 1))
        _fill(flags, n, lambda i: (i % 3 != 0).to(torch.int64))
        _, cnt = dws.select_flagged(x, flags, out=out)
        torch.cuda.synchronize()
        count = int(cnt.item())
        assert count == n - (n + 2) // 3
        for s in range(0, count, SLICE):
            e = min(count, s + SLICE)
            j = torch.arange(s, e, dtype=torch.int64, device="cuda")
            want = (3 * (j // 2) + j % 2 + 1) & 0xFFFFFFFF
            got = out[s:e].to(torch.int64) & 0xFFFFFFFF
            assert torch.equal(got, want), f"select mismatch in [{s}, {e})"
    finally:
        del x, flags, out
        torch.cuda.empty_cache()


def test_runs_at_the_count_limit(gpu):
    # keys[i] = i // 7: runs of 7 and a last one of 3; reduce-by-key of
    # all-ones values gives the same lengths as run-length encoding
    import torch
    n = COMPACTION_MAX
    _need(16 * n)
    runs = (n + 6) // 7
    keys = torch.empty(n, dtype=torch.int32, device="cuda")
    try:
        _fill(keys, n, lambda i: i // 7)
        ones = torch.ones(n, dtype=torch.int32, device="cuda")
        for kind in ("rle", "sums"):
            note(f"{kind} n={n} (runs of 7)")
            if kind == "rle":
                uk, ag, cnt = dws.run_length_encode(keys)
            else:
                uk, ag, cnt = dws.reduce_by_key(keys, ones)
            torch.cuda.synchronize()
            assert int(cnt.item()) == runs
            for s in range(0, runs, SLICE):
                e = min(runs, s + SLICE)
                r = torch.arange(s, e, dtype=torch.int64, device="cuda")
                assert torch.equal(uk[s:e].to(torch.int64), r), f"{kind}: keys in [{s}, {e})"
                want = torch.where(r == runs - 1, n - 7 * (runs - 1), 7)
                assert torch.equal(ag[s:e].to(torch.int64), want), f"{kind}: lengths in [{s}, {e})"
            del uk, ag, cnt
        del ones
    finally:
        del keys
        torch.cuda.empty_cache()
    assert dws.watchdog_trips() == 0


def test_operators_past_32_bits(gpu):
    # dws_scan_op past 2^32 elements, in place, against closed forms:
    # max of x[i] = i mod 2^32 (uint32) climbs to 2^32 - 1 and stays there after
    # the wrap; the componentwise sum of all-ones uint32 pairs is (i + 1, i + 1)
    # mod 2^32, inclusive
    import torch
    n = (1 << 32) + 12345
    stream = torch.cuda.current_stream().cuda_stream
    _need(8 * n)
    x = torch.empty(n, dtype=torch.int32, device="cuda")
    try:
        _fill(x, n, lambda i: (i & 0xFFFFFFFF) - ((i & 0x80000000) << 1))
        for exclusive in (False, True):
            note(f"uint32 max scan n={n} exclusive={exclusive}, in place")
            if exclusive:
                _fill(x, n, lambda i: (i & 0xFFFFFFFF) - ((i & 0x80000000) << 1))
            st = dws.scan_op_ptr(x.data_ptr(), x.data_ptr(), n, dws.UINT32, dws.OP_MAX, exclusive, stream)
            assert st == dws.OK, dws.status_string(st)
            torch.cuda.synchronize()
            for s in range(0, n, SLICE):
                e = min(n, s + SLICE)
                i = torch.arange(s, e, dtype=torch.int64, device="cuda")
                last = i - 1 if exclusive else i                 # the last index the max covers
                want = torch.clamp(last, 0, 0xFFFFFFFF)          # exclusive y[0] is the identity 0
                got = x[s:e].to(torch.int64) & 0xFFFFFFFF
                assert torch.equal(got, want), f"max exclusive={exclusive}: mismatch in [{s}, {e})"
    finally:
        del x
        torch.cuda.empty_cache()
    _need(8 * n)
    pairs = torch.ones((n, 2), dtype=torch.int32, device="cuda")
    try:
        note(f"uint32 pair sum n={n} pairs, in place")
        st = dws.scan_op_ptr(pairs.data_ptr(), pairs.data_ptr(), n, dws.PAIR_U32, dws.OP_SUM, False, stream)
        assert st == dws.OK, dws.status_string(st)
        torch.cuda.synchronize()
        for s in range(0, n, SLICE):
            e = min(n, s + SLICE)
            want = torch.arange(s + 1, e + 1, dtype=torch.int64, device="cuda") & 0xFFFFFFFF
            for w in range(2):
                got = pairs[s:e, w].to(torch.int64) & 0xFFFFFFFF
                assert torch.equal(got, want), f"pair sum word {w}: mismatch in [{s}, {e})"
    finally:
        del pairs
        torch.cuda.empty_cache()
    assert dws.watchdog_trips() == 0

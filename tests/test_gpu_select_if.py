"""GPU parity of select-if and partition-if (dws_select_if, dws_partition_if):
the selection x[i] `pred` t computed in the kernel from the values, against
the oracle's select / partition by flags, with the flags written out by numpy's
comparison of the same values (the plain definition of the predicate: for
fp32 a NaN satisfies only "not equal", as in IEEE and numpy).

Bar: bit-exact (elements are moved, not computed), and the count exact.
"""
import numpy as np
import pytest

import device_wide_prefix_amd as dws
import oracle
import scan_workloads as wl
from gpu_util import CODE, from_device, note, to_device

pytestmark = pytest.mark.gpu

SENTINEL = -7
PREDS = {dws.PRED_EQ: np.equal, dws.PRED_NE: np.not_equal, dws.PRED_LT: np.less, dws.PRED_LE: np.less_equal,
         dws.PRED_GT: np.greater, dws.PRED_GE: np.greater_equal}
NAMES = {dws.PRED_EQ: "eq", dws.PRED_NE: "ne", dws.PRED_LT: "lt", dws.PRED_LE: "le", dws.PRED_GT: "gt",
         dws.PRED_GE: "ge"}
# around every select tile (4,096 below 2^22, 32,768 from there, non-temporal
# loads from 2^23, the in-place drawn index from 2^25) with ragged ends
SIZES = [1, 5, 4095, 4097, 3 * 4096 + 7, 1_000_003, (1 << 22) + 5, (1 << 23) + 33, (1 << 25) + 3]


def _input(dtype, n, seed):
    """Values with repeats, so that == and != select non-trivial sets."""
    rng = np.random.default_rng(seed)
    if dtype == "float32":
        x = (rng.integers(-50, 50, n) * 0.5).astype(np.float32)
        if n > 10:
            x[rng.integers(0, n, max(1, n // 1000))] = np.nan
            x[rng.integers(0, n, max(1, n // 1000))] = -0.0
        return x
    if dtype == "int32":
        return rng.integers(-100, 100, n).astype(np.int32)
    return rng.integers(0, 200, n).astype(np.uint32)


def _threshold(dtype):
    return {"float32": 0.0, "int32": -3, "uint32": 100}[dtype]


def _run(x, dtype, pred, t, partition=False, in_place=False, offset=0):
    import torch
    n = x.size
    _, xd = to_device(x, extra_front=offset)
    if in_place:
        out = xd
    else:
        ostore = torch.full((n + offset,), SENTINEL, dtype=torch.int32, device="cuda")
        out = ostore[offset:]
    count = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    st = dws.select_if_ptr(xd.data_ptr(), out.data_ptr(), n, CODE[dtype], pred, t, count.data_ptr(),
                           torch.cuda.current_stream().cuda_stream, partition=partition)
    assert st == dws.OK, dws.status_string(st)
    return from_device(out, dtype), int(count.item())


def _flags(x, dtype, pred, t):
    with np.errstate(invalid="ignore"):
        return PREDS[pred](x, x.dtype.type(t)).astype(np.int32)


def _check(x, dtype, pred, t, got, cnt, partition, in_place, label):
    flags = _flags(x, dtype, pred, t)
    xb, gb = x.view(np.uint32), got.view(np.uint32)
    if partition:
        want, wcnt = oracle.partition_flagged(x, flags)
        assert cnt == wcnt, f"{label}: count {cnt} != {wcnt}"
        wb = want.view(np.uint32)
        if not np.array_equal(gb, wb):
            i = int(np.flatnonzero(gb != wb)[0])
            raise AssertionError(f"{label}: mismatch at {i}: gpu {gb[i]:#x} oracle {wb[i]:#x}")
        return
    want = oracle.select_flagged(x, flags).view(np.uint32)
    assert cnt == want.size, f"{label}: count {cnt} != {want.size}"
    if not np.array_equal(gb[:cnt], want):
        i = int(np.flatnonzero(gb[:cnt] != want)[0])
        raise AssertionError(f"{label}: mismatch at {i}/{cnt}: gpu {gb[i]:#x} oracle {want[i]:#x}")
    rest = xb[cnt:] if in_place else np.full(x.size - cnt, SENTINEL, dtype=np.int32).view(np.uint32)
    assert np.array_equal(gb[cnt:], rest), f"{label}: output changed past the count"


@pytest.mark.parametrize("dtype", ["int32", "uint32", "float32"])
def test_select_if_every_predicate(gpu, dtype):
    t = _threshold(dtype)
    for i, n in enumerate(SIZES):
        x = _input(dtype, n, seed=n)
        for pred in PREDS:
            in_place = (i + pred) % 2 == 1
            note(f"select_if {dtype} {NAMES[pred]} n={n} in_place={in_place}")
            got, cnt = _run(x, dtype, pred, t, in_place=in_place)
            _check(x, dtype, pred, t, got, cnt, False, in_place, f"{dtype} {NAMES[pred]} n={n}")


@pytest.mark.parametrize("dtype", ["int32", "float32"])
def test_partition_if_and_unaligned(gpu, dtype):
    t = _threshold(dtype)
    for n in (7, 4097, 1_000_003, (1 << 23) + 33):
        x = _input(dtype, n, seed=3 * n)
        for pred in (dws.PRED_LT, dws.PRED_NE, dws.PRED_EQ):
            note(f"partition_if {dtype} {NAMES[pred]} n={n}")
            got, cnt = _run(x, dtype, pred, t, partition=True)
            _check(x, dtype, pred, t, got, cnt, True, False, f"partition {dtype} {NAMES[pred]} n={n}")
            note(f"select_if unaligned {dtype} {NAMES[pred]} n={n}")
            got, cnt = _run(x, dtype, pred, t, offset=1)
            _check(x, dtype, pred, t, got, cnt, False, False, f"unaligned {dtype} {NAMES[pred]} n={n}")


def test_select_if_full_size_flags(gpu):
    """The 2^30 - 12,345 int32 flag workload selected by x != 0 through the
    predicate, in place: the same result as dws_select_flagged with the input
    as its own flags."""
    import torch
    w = wl.WORKLOADS["flags_2p30m12345_excl"]
    note(f"select_if x != 0 on {w.description}, in place")
    x = wl.generate_workload(w)
    store, xd = to_device(x)
    count = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    st = dws.select_if_ptr(xd.data_ptr(), xd.data_ptr(), w.n, dws.INT32, dws.PRED_NE, 0, count.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == dws.OK, dws.status_string(st)
    cnt = int(count.item())
    assert cnt == int(np.count_nonzero(x))
    # every selected element of 0/1 flags is a 1; the rest of the array is untouched
    head = xd[:cnt]
    assert int((head != 1).sum().item()) == 0
    tail = from_device(xd[cnt:], "int32")
    assert np.array_equal(tail, x[cnt:])
    del store, xd
    assert dws.watchdog_trips() == 0

"""Shared helpers of the GPU tests: upload, call the C ABI by raw pointer,
download, and compare with the oracle to the parity bar
(bit-exact for 32-bit integers; |y - y_ref| <= 1e-4 * sum_{j<=i}|x_j| + 1e-6
for fp32, with y_ref and the running |x| sum from the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np

import device_wide_prefix_amd as dws
import oracle

RTOL = 1e-4
ATOL = 1e-6

CODE = {"int32": dws.INT32, "uint32": dws.UINT32, "float32": dws.FLOAT32}


def note(msg: str):
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, extra_front: int = 0):
    """Copy x to the GPU as int32/float32 storage (uint32 travels as int32
    bits). extra_front elements are prepended so that a view can start at a
    4-byte but not 16-byte aligned address. Returns (storage, view)."""
    import torch
    if x.dtype == np.float32:
        host = torch.from_numpy(np.ascontiguousarray(x))
        tdtype = torch.float32
    else:
        host = torch.from_numpy(np.ascontiguousarray(x).view(np.int32))
        tdtype = torch.int32
    store = torch.empty(x.size + extra_front, dtype=tdtype, device="cuda")
    view = store[extra_front:]
    view.copy_(host)
    return store, view


def from_device(t, dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype == "uint32":
        return a.view(np.uint32)
    return a


def run(x_dev, out_dev, n: int, dtype: str, exclusive: bool, variant=0, order=0, shape=0, nt=0, tile_index=0):
    """Call dws_scan_ex on raw device pointers on torch's current stream."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    if variant == 0 and order == 0 and shape == 0 and nt == 0 and tile_index == 0:
        f = dws.scan_exclusive_ptr if exclusive else dws.scan_inclusive_ptr
        st = f(x_dev.data_ptr(), out_dev.data_ptr(), n, CODE[dtype], stream)
    else:
        opt = dws.DwsOptions(variant, order, shape, nt, tile_index)
        st = dws.scan_opts_ptr(x_dev.data_ptr(), out_dev.data_ptr(), n, CODE[dtype], exclusive, opt, stream)
    assert st == dws.OK, f"scan returned {st}: {dws.status_string(st)}"


def check(x: np.ndarray, y: np.ndarray, dtype: str, exclusive: bool, label: str = ""):
    """Compare a GPU result with the oracle; returns the max fp32 tolerance
    ratio (0 for integers)."""
    assert y.shape == x.shape
    if dtype == "float32":
        ref, sabs = oracle.scan_f32(x, exclusive=exclusive)
        err = np.abs(y.astype(np.float64) - ref)
        bound = RTOL * sabs + ATOL
        ok = err <= bound
        if not ok.all():
            i = int(np.flatnonzero(~ok)[0])
            raise AssertionError(f"{label} fp32 mismatch at {i}/{x.size}: gpu {y[i]!r} ref {ref[i]!r} "
                                 f"bound {bound[i]:.3g}; {int((~ok).sum())} elements out of tolerance")
        return float((err / bound).max()) if x.size else 0.0
    ref = oracle.scan_u32(x, exclusive=exclusive)
    yb, rb = y.view(np.uint32), ref.view(np.uint32)
    if not np.array_equal(yb, rb):
        bad = np.flatnonzero(yb != rb)
        i = int(bad[0])
        raise AssertionError(f"{label} int mismatch at {i}/{x.size} ({bad.size} elements): "
                             f"gpu {int(yb[i])} ref {int(rb[i])}")
    return 0.0


def check_chunked(x: np.ndarray, y: np.ndarray, dtype: str, exclusive: bool, label: str = "",
                  chunk: int = 1 << 26):
    """Same bar as check() for very large arrays: the oracle runs once over the
    whole input, the comparison runs in chunks to bound host memory."""
    if dtype == "float32":
        ref, sabs = oracle.scan_f32(x, exclusive=exclusive)
        worst = 0.0
        for s in range(0, x.size, chunk):
            e = slice(s, min(s + chunk, x.size))
            err = np.abs(y[e].astype(np.float64) - ref[e])
            bound = RTOL * sabs[e] + ATOL
            ok = err <= bound
            if not ok.all():
                i = s + int(np.flatnonzero(~ok)[0])
                raise AssertionError(f"{label} fp32 mismatch at {i}/{x.size}: gpu {y[i]!r} ref {ref[i]!r}")
            worst = max(worst, float((err / bound).max()))
        return worst
    ref = oracle.scan_u32(x, exclusive=exclusive)
    yb, rb = y.view(np.uint32), ref.view(np.uint32)
    for s in range(0, x.size, chunk):
        e = slice(s, min(s + chunk, x.size))
        if not np.array_equal(yb[e], rb[e]):
            i = s + int(np.flatnonzero(yb[e] != rb[e])[0])
            raise AssertionError(f"{label} int mismatch at {i}/{x.size}: gpu {int(yb[i])} ref {int(rb[i])}")
    return 0.0


def decode_desc(words: np.ndarray):
    """Split descriptor words into (epoch, status, value bits)."""
    w = words.astype(np.uint64)
    hi = (w >> np.uint64(32)).astype(np.uint64)
    return (hi >> np.uint64(2)).astype(np.int64), (hi & np.uint64(3)).astype(np.int64), \
        (w & np.uint64(0xFFFFFFFF)).astype(np.uint32)

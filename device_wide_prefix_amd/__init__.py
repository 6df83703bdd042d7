"""Python binding of libdws_scan.so, the gfx950 device-wide + prefix scan.

Argument marshalling only: every step of the scan runs in the library's HIP
kernels. torch supplies device buffers and the current stream. There is no CPU
fallback; if the library is not built, importing the binding's functions raises.

    scan_inclusive(x, out=None)            -> out
    scan_exclusive(x, out=None)            -> out      (out may be x: in place)
    scan_ex(x, out=None, exclusive=False, variant=SINGLE_PASS) -> out
    scan_opts(x, out=None, exclusive=False, variant=..., memory_order=...,
              tile_shape=0, nontemporal=None, tile_index=...) -> out
    scan_seeded(x, seed, exclusive=False, out=None) -> out  (seed: 1-element GPU tensor)
    reduce(x, out=None)                    -> 1-element GPU tensor holding the + of x
    scan_debug(x, out, tile_elems, ...)    -> descriptor words (numpy uint64)
    watchdog_trips()                       -> int
    selftest_wave(x)                       -> (incl, shift)
The C entry points take raw device pointers; the *_ptr functions expose them.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libdws_scan.so")

# dws_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_OVERLAP, ERR_HIP, ERR_OOM, ERR_MISALIGNED = range(7)
# dws_dtype
INT32, UINT32, FLOAT32, PAIR_I32_F32, PAIR_U32 = 0, 1, 2, 3, 4
# dws_op
OP_SUM, OP_MAX, OP_MIN, OP_AFFINE, OP_SEGMENTED_SUM = 0, 1, 2, 3, 4
# dws_variant
SINGLE_PASS, REDUCE_THEN_SCAN, CHAINED, SCAN_THEN_PROPAGATE = 0, 1, 2, 3
# dws_memory_order
ORDER_RELAXED, ORDER_ACQ_REL = 0, 1
# dws_tile_index
TILE_AUTO, TILE_DRAWN, TILE_DISPATCH = 0, 1, 2
# dws_pred
PRED_EQ, PRED_NE, PRED_LT, PRED_LE, PRED_GT, PRED_GE = range(6)
# dws_options.nontemporal
NT_AUTO, NT_ON, NT_OFF = 0, 1, 2

EXPORTED_SYMBOLS = (
    "scan_inclusive", "scan_exclusive", "dws_scan_ex", "dws_scan_opts", "dws_status_string", "dws_version",
    "dws_num_tile_shapes", "dws_tile_elems", "dws_tile_threads", "dws_reserve",
    "dws_release_workspaces", "dws_watchdog_trips", "dws_scan_debug", "dws_selftest_wave",
    "dws_scan_profiled", "dws_select_flagged", "dws_scan_op", "dws_partition_flagged", "dws_reduce_by_key",
    "dws_run_length_encode", "dws_device_memory_info", "dws_scan_noalloc", "dws_scan_plan", "dws_scan_seeded",
    "dws_reduce", "dws_scan_op_seeded", "dws_reduce_op", "dws_select_if", "dws_partition_if",
)


class ScanError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class DwsOptions(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("memory_order", ctypes.c_int),
                ("tile_shape", ctypes.c_int), ("nontemporal", ctypes.c_int),
                ("tile_index", ctypes.c_int)]


class LaunchPlan(ctypes.Structure):
    """dws_launch_plan: what a single-pass or chained call would launch."""
    _fields_ = [("threads", ctypes.c_uint), ("tile_elems", ctypes.c_uint), ("num_tiles", ctypes.c_uint),
                ("tile_index", ctypes.c_int), ("nontemporal", ctypes.c_int), ("pause_units", ctypes.c_int)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libdws_scan.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m device_wide_prefix_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, ci, cu = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint
    for name in ("scan_inclusive", "scan_exclusive"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, sz, ci, vp]
        f.restype = ci
    lib.dws_scan_ex.argtypes = [vp, vp, sz, ci, ci, ci, vp]
    lib.dws_scan_ex.restype = ci
    lib.dws_scan_opts.argtypes = [vp, vp, sz, ci, ci, ctypes.POINTER(DwsOptions), vp]
    lib.dws_scan_opts.restype = ci
    lib.dws_scan_noalloc.argtypes = [vp, vp, sz, ci, ci, vp]
    lib.dws_scan_noalloc.restype = ci
    lib.dws_scan_plan.argtypes = [vp, vp, sz, ci, ci, ctypes.POINTER(DwsOptions), ctypes.POINTER(LaunchPlan)]
    lib.dws_scan_plan.restype = ci
    lib.dws_scan_seeded.argtypes = [vp, vp, sz, ci, ci, vp, vp]
    lib.dws_scan_seeded.restype = ci
    lib.dws_reduce.argtypes = [vp, sz, ci, vp, vp]
    lib.dws_reduce.restype = ci
    lib.dws_scan_op_seeded.argtypes = [vp, vp, sz, ci, ci, ci, vp, vp]
    lib.dws_scan_op_seeded.restype = ci
    lib.dws_reduce_op.argtypes = [vp, sz, ci, ci, vp, vp]
    lib.dws_reduce_op.restype = ci
    for name in ("dws_select_if", "dws_partition_if"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, sz, ci, ci, vp, vp, vp]
        f.restype = ci
    lib.dws_status_string.argtypes = [ci]
    lib.dws_status_string.restype = ctypes.c_char_p
    lib.dws_version.restype = ci
    lib.dws_num_tile_shapes.restype = ci
    lib.dws_tile_elems.argtypes = [ci, sz, ci]
    lib.dws_tile_elems.restype = cu
    lib.dws_tile_threads.argtypes = [ci, sz, ci]
    lib.dws_tile_threads.restype = cu
    lib.dws_reserve.argtypes = [sz, vp]
    lib.dws_reserve.restype = ci
    lib.dws_release_workspaces.restype = ci
    lib.dws_watchdog_trips.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
    lib.dws_watchdog_trips.restype = ci
    lib.dws_device_memory_info.argtypes = [ctypes.POINTER(ctypes.c_int)] * 3
    lib.dws_device_memory_info.restype = ci
    lib.dws_scan_debug.argtypes = [vp, vp, sz, ci, ci, ci, cu, cu, cu, cu,
                                   ctypes.POINTER(ctypes.c_ulonglong), vp]
    lib.dws_scan_debug.restype = ci
    lib.dws_scan_profiled.argtypes = [vp, vp, sz, ci, ci, vp, sz, ctypes.POINTER(cu), vp]
    lib.dws_scan_profiled.restype = ci
    lib.dws_scan_op.argtypes = [vp, vp, sz, ci, ci, ci, vp]
    lib.dws_scan_op.restype = ci
    lib.dws_partition_flagged.argtypes = [vp, vp, vp, sz, ci, vp, vp]
    lib.dws_partition_flagged.restype = ci
    lib.dws_reduce_by_key.argtypes = [vp, vp, vp, vp, sz, ci, vp, vp]
    lib.dws_reduce_by_key.restype = ci
    lib.dws_run_length_encode.argtypes = [vp, vp, vp, sz, vp, vp]
    lib.dws_run_length_encode.restype = ci
    lib.dws_select_flagged.argtypes = [vp, vp, vp, sz, ci, vp, vp]
    lib.dws_select_flagged.restype = ci
    lib.dws_selftest_wave.argtypes = [vp, vp, vp, sz, ci, vp]
    lib.dws_selftest_wave.restype = ci
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().dws_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != OK:
        raise ScanError(status, what)


# ---- raw-pointer entry points (same names as the C ABI, plus _ptr) --------

def scan_inclusive_ptr(d_in: int, d_out: int, n: int, dtype: int, stream: int = 0) -> int:
    return load_library().scan_inclusive(d_in, d_out, n, dtype, stream)


def scan_exclusive_ptr(d_in: int, d_out: int, n: int, dtype: int, stream: int = 0) -> int:
    return load_library().scan_exclusive(d_in, d_out, n, dtype, stream)


def scan_ex_ptr(d_in: int, d_out: int, n: int, dtype: int, exclusive: bool, variant: int,
                stream: int = 0) -> int:
    return load_library().dws_scan_ex(d_in, d_out, n, dtype, int(bool(exclusive)), int(variant), stream)


def scan_noalloc_ptr(d_in: int, d_out: int, n: int, dtype: int, exclusive: bool, stream: int = 0) -> int:
    return load_library().dws_scan_noalloc(d_in, d_out, n, dtype, int(bool(exclusive)), stream)


def scan_seeded_ptr(d_in: int, d_out: int, n: int, dtype: int, exclusive: bool, d_seed: int,
                    stream: int = 0) -> int:
    return load_library().dws_scan_seeded(d_in, d_out, n, dtype, int(bool(exclusive)), d_seed, stream)


def reduce_ptr(d_in: int, n: int, dtype: int, d_total: int, stream: int = 0) -> int:
    return load_library().dws_reduce(d_in, n, dtype, d_total, stream)


def scan_opts_ptr(d_in: int, d_out: int, n: int, dtype: int, exclusive: bool,
                  options: DwsOptions | None, stream: int = 0) -> int:
    opt = ctypes.byref(options) if options is not None else None
    return load_library().dws_scan_opts(d_in, d_out, n, dtype, int(bool(exclusive)), opt, stream)


def scan_plan_ptr(d_in: int, d_out: int, n: int, dtype: int, exclusive: bool,
                  options: DwsOptions | None = None) -> tuple[int, LaunchPlan]:
    """dws_scan_plan: (status, plan) for what dws_scan_opts would launch with
    these arguments; the pointers are only compared and checked for alignment."""
    plan = LaunchPlan()
    opt = ctypes.byref(options) if options is not None else None
    st = load_library().dws_scan_plan(d_in, d_out, n, dtype, int(bool(exclusive)), opt, ctypes.byref(plan))
    return st, plan


# ---- torch-tensor entry points --------------------------------------------

def _dtype_code(t) -> int:
    import torch
    codes = {torch.int32: INT32, torch.float32: FLOAT32}
    u32 = getattr(torch, "uint32", None)
    if u32 is not None:
        codes[u32] = UINT32
    if t.dtype not in codes:
        raise TypeError(f"scan supports int32, uint32 and float32 tensors, got {t.dtype}")
    return codes[t.dtype]


def _prepare(x, out):
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("scan expects a GPU tensor (there is no CPU path)")
    if not x.is_contiguous():
        raise ValueError("input tensor must be contiguous")
    code = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.numel() != x.numel() or not out.is_contiguous() or \
            out.device != x.device:
        raise ValueError("out must be a contiguous tensor with the dtype, size and device of x")
    return code, out


def _stream(x, stream):
    import torch
    if stream is not None:
        return int(stream)
    return int(torch.cuda.current_stream(x.device).cuda_stream)


def scan_inclusive(x, out=None, stream=None):
    """Inclusive + scan of a contiguous GPU tensor; returns ``out``."""
    code, out = _prepare(x, out)
    with _device_of(x):
        _check(scan_inclusive_ptr(x.data_ptr(), out.data_ptr(), x.numel(), code, _stream(x, stream)),
               "scan_inclusive")
    return out


def scan_exclusive(x, out=None, stream=None):
    """Exclusive + scan of a contiguous GPU tensor; returns ``out`` (may be x)."""
    code, out = _prepare(x, out)
    with _device_of(x):
        _check(scan_exclusive_ptr(x.data_ptr(), out.data_ptr(), x.numel(), code, _stream(x, stream)),
               "scan_exclusive")
    return out


def scan_ex(x, out=None, exclusive=False, variant=SINGLE_PASS, stream=None):
    """Scan by the global strategy ``variant`` (dws_variant); returns ``out``."""
    code, out = _prepare(x, out)
    with _device_of(x):
        _check(scan_ex_ptr(x.data_ptr(), out.data_ptr(), x.numel(), code, exclusive, variant,
                           _stream(x, stream)), "dws_scan_ex")
    return out


def scan_opts(x, out=None, exclusive=False, variant=SINGLE_PASS, memory_order=ORDER_RELAXED,
              tile_shape=0, nontemporal=None, tile_index=TILE_AUTO, stream=None):
    """Scan with explicit options (variant, descriptor memory order, tile shape,
    non-temporal loads: None for the library's choice, True or False to force
    them on or off; tile index source); returns ``out``."""
    code, out = _prepare(x, out)
    nt = NT_AUTO if nontemporal is None else (NT_ON if nontemporal else NT_OFF)
    opt = DwsOptions(int(variant), int(memory_order), int(tile_shape), nt, int(tile_index))
    with _device_of(x):
        _check(scan_opts_ptr(x.data_ptr(), out.data_ptr(), x.numel(), code, exclusive, opt,
                             _stream(x, stream)), "dws_scan_opts")
    return out


def scan_seeded(x, seed, exclusive=False, out=None, stream=None):
    """Scan of x with the 1-element GPU tensor ``seed`` (dtype of x) as the
    prefix of the whole array (dws_scan_seeded); returns ``out`` (may be x)."""
    import torch
    code, out = _prepare(x, out)
    if not isinstance(seed, torch.Tensor) or seed.device != x.device or seed.dtype != x.dtype or \
            seed.numel() != 1:
        raise ValueError("seed must be a 1-element tensor with the dtype and device of x")
    with _device_of(x):
        _check(scan_seeded_ptr(x.data_ptr(), out.data_ptr(), x.numel(), code, exclusive, seed.data_ptr(),
                               _stream(x, stream)), "dws_scan_seeded")
    return out


def reduce(x, out=None, stream=None):
    """+ of every element of x (dws_reduce) into the 1-element GPU tensor
    ``out`` (a new one by default); returns ``out``."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("reduce expects a GPU tensor (there is no CPU path)")
    if not x.is_contiguous():
        raise ValueError("input tensor must be contiguous")
    code = _dtype_code(x)
    if out is None:
        out = torch.empty(1, dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype or out.numel() != 1 or out.device != x.device:
        raise ValueError("out must be a 1-element tensor with the dtype and device of x")
    with _device_of(x):
        _check(reduce_ptr(x.data_ptr(), x.numel(), code, out.data_ptr(), _stream(x, stream)), "dws_reduce")
    return out


def scan_debug(x, out, tile_elems, exclusive=False, variant=SINGLE_PASS, delay_every=0,
               delay_phase=0, delay_ticks=0, want_descriptors=True, stream=None):
    """Run the protocol-inspection kernel (one wavefront per tile of
    ``tile_elems`` <= 64 elements). Returns the final descriptor words as a numpy
    uint64 array (synchronises) or None."""
    import numpy as np
    code, out = _prepare(x, out)
    n = x.numel()
    num_tiles = max(1, -(-n // int(tile_elems))) if n else 0
    desc = None
    ptr = None
    if want_descriptors and n:
        desc = np.zeros(num_tiles, dtype=np.uint64)
        ptr = desc.ctypes.data_as(ctypes.POINTER(ctypes.c_ulonglong))
    with _device_of(x):
        _check(load_library().dws_scan_debug(x.data_ptr(), out.data_ptr(), n, code, int(bool(exclusive)),
                                             int(variant), int(tile_elems), int(delay_every),
                                             int(delay_phase), int(delay_ticks), ptr, _stream(x, stream)),
               "dws_scan_debug")
    return desc


STAMPS_PER_TILE = 5
STAMP_NAMES = ("start", "tile_index_known", "aggregate_published", "prefix_known", "stores_issued")


def profiled_num_tiles(n: int) -> int:
    t = ctypes.c_uint(0)
    _check(load_library().dws_scan_profiled(None, None, int(n), INT32, 0, None, 0, ctypes.byref(t), None),
           "dws_scan_profiled")
    return int(t.value)


def scan_profiled(x, out=None, exclusive=False, stream=None):
    """Instrumented single-pass scan. Returns (out, stamps) where stamps is a
    (num_tiles, 5) int64 GPU tensor of 100 MHz real-time counter values:
    start, tile index known, aggregate published, prefix known, stores issued."""
    import torch
    code, out = _prepare(x, out)
    tiles = profiled_num_tiles(x.numel())
    stamps = torch.zeros((max(tiles, 1), STAMPS_PER_TILE), dtype=torch.int64, device=x.device)
    t = ctypes.c_uint(0)
    with _device_of(x):
        _check(load_library().dws_scan_profiled(x.data_ptr(), out.data_ptr(), x.numel(), code, int(bool(exclusive)),
                                                stamps.data_ptr(), stamps.numel(), ctypes.byref(t),
                                                _stream(x, stream)), "dws_scan_profiled")
    return out, stamps[:tiles]


def scan_op_ptr(d_in: int, d_out: int, n: int, dtype: int, op: int, exclusive: bool, stream: int = 0) -> int:
    return load_library().dws_scan_op(d_in, d_out, n, dtype, op, int(bool(exclusive)), stream)


def scan_op_seeded_ptr(d_in: int, d_out: int, n: int, dtype: int, op: int, exclusive: bool, d_seed: int,
                       stream: int = 0) -> int:
    return load_library().dws_scan_op_seeded(d_in, d_out, n, dtype, op, int(bool(exclusive)), d_seed, stream)


def select_if_ptr(d_in: int, d_out: int, n: int, dtype: int, pred: int, threshold, d_count: int,
                  stream: int = 0, partition: bool = False) -> int:
    """dws_select_if (dws_partition_if with partition=True); ``threshold`` is a
    Python number converted to dtype on the host."""
    import numpy as np
    np_t = {INT32: np.int32, UINT32: np.uint32, FLOAT32: np.float32}.get(int(dtype), np.uint32)
    buf = np.array([threshold], dtype=np_t)
    f = load_library().dws_partition_if if partition else load_library().dws_select_if
    return f(d_in, d_out, n, dtype, int(pred), buf.ctypes.data, d_count, stream)


def reduce_op_ptr(d_in: int, n: int, dtype: int, op: int, d_total: int, stream: int = 0) -> int:
    return load_library().dws_reduce_op(d_in, n, dtype, op, d_total, stream)


def reduce_op(x, op, dtype=None, out=None, stream=None):
    """Combination under ``op`` of every element of x in order (dws_reduce_op)
    into ``out``: a GPU tensor of one element's bytes (a new int32 tensor of 1
    or 2 words by default, bits as for scan_op). Returns ``out``."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("reduce_op expects a GPU tensor (there is no CPU path)")
    if not x.is_contiguous():
        raise ValueError("input tensor must be contiguous")
    if dtype is None:
        dtype = _dtype_code(x)
    esize = 8 if dtype in (PAIR_I32_F32, PAIR_U32) else 4
    nbytes = x.numel() * x.element_size()
    if nbytes % esize:
        raise ValueError(f"tensor of {nbytes} bytes does not hold whole {esize}-byte elements")
    if out is None:
        out = torch.empty(esize // 4, dtype=torch.int32, device=x.device)
    if out.numel() * out.element_size() != esize or not out.is_contiguous() or out.device != x.device:
        raise ValueError(f"out must be a contiguous tensor of {esize} bytes on the device of x")
    with _device_of(x):
        _check(reduce_op_ptr(x.data_ptr(), nbytes // esize, int(dtype), int(op), out.data_ptr(),
                             _stream(x, stream)), "dws_reduce_op")
    return out


def scan_op(x, op, dtype=None, exclusive=False, out=None, stream=None, seed=None):
    """Scan of a contiguous GPU tensor under a generic operator (OP_*).

    For the 32-bit types dtype defaults from the tensor. Pair types
    (PAIR_I32_F32, PAIR_U32) take any contiguous tensor whose bytes hold the
    pairs, e.g. an (n, 2) int32 tensor of bits; n is its byte size / 8.
    ``seed``: a GPU tensor on x's device whose bytes hold one element, the
    initial value before the whole array (dws_scan_op_seeded).
    Returns ``out`` (same shape and dtype as x; may be x)."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("scan_op expects a GPU tensor (there is no CPU path)")
    if not x.is_contiguous():
        raise ValueError("input tensor must be contiguous")
    if dtype is None:
        dtype = _dtype_code(x)
    esize = 8 if dtype in (PAIR_I32_F32, PAIR_U32) else 4
    nbytes = x.numel() * x.element_size()
    if nbytes % esize:
        raise ValueError(f"tensor of {nbytes} bytes does not hold whole {esize}-byte elements")
    if out is None:
        out = torch.empty_like(x)
    if out.numel() * out.element_size() != nbytes or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor of the same byte size on the device of x")
    if seed is not None:
        if not isinstance(seed, torch.Tensor) or seed.device != x.device or not seed.is_contiguous() or \
                seed.numel() * seed.element_size() != esize:
            raise ValueError(f"seed must be a contiguous tensor of {esize} bytes on the device of x")
        with _device_of(x):
            _check(scan_op_seeded_ptr(x.data_ptr(), out.data_ptr(), nbytes // esize, int(dtype), int(op),
                                      exclusive, seed.data_ptr(), _stream(x, stream)), "dws_scan_op_seeded")
        return out
    with _device_of(x):
        _check(scan_op_ptr(x.data_ptr(), out.data_ptr(), nbytes // esize, int(dtype), int(op), exclusive,
                           _stream(x, stream)), "dws_scan_op")
    return out


def select_flagged_ptr(d_in: int, d_flags: int, d_out: int, n: int, dtype: int, d_count: int,
                      stream: int = 0) -> int:
    return load_library().dws_select_flagged(d_in, d_flags, d_out, n, dtype, d_count, stream)


def select_flagged(x, flags, out=None, count=None, stream=None):
    """Stream compaction: the elements of x whose int32 flag is non-zero, in
    order, written to out[:count]. Returns (out, count) with count a one-element
    int64 GPU tensor (no synchronisation). out may be x (in place)."""
    import torch
    code, out = _prepare(x, out)
    if not isinstance(flags, torch.Tensor) or flags.dtype != torch.int32 or \
            flags.numel() != x.numel() or not flags.is_contiguous() or flags.device != x.device:
        raise ValueError("flags must be a contiguous int32 tensor with the size and device of x")
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=x.device)
    if count.dtype != torch.int64 or count.numel() < 1 or count.device != x.device:
        raise ValueError("count must be an int64 tensor on the device of x")
    with _device_of(x):
        _check(select_flagged_ptr(x.data_ptr(), flags.data_ptr(), out.data_ptr(), x.numel(), code,
                                  count.data_ptr(), _stream(x, stream)), "dws_select_flagged")
    return out, count


def _count_tensor(x, count):
    import torch
    if count is None:
        count = torch.empty(1, dtype=torch.int64, device=x.device)
    if count.dtype != torch.int64 or count.numel() < 1 or count.device != x.device:
        raise ValueError("count must be an int64 tensor on the device of x")
    return count


def _check_like(t, x, what):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.device != x.device or \
            t.numel() != x.numel() or t.element_size() != 4:
        raise ValueError(f"{what} must be a contiguous 4-byte GPU tensor with the size and device of the keys")


def partition_flagged(x, flags, out=None, count=None, stream=None):
    """Partition by flags: out[:count] the selected elements in order,
    out[count:] the rejected ones in reverse order. Returns (out, count) with
    count a one-element int64 GPU tensor. out must not overlap x."""
    import torch
    code, _ = _prepare(x, x)
    if out is None:
        out = torch.empty_like(x)
    _check_like(out, x, "out")
    _check_like(flags, x, "flags")
    count = _count_tensor(x, count)
    with _device_of(x):
        _check(load_library().dws_partition_flagged(x.data_ptr(), flags.data_ptr(), out.data_ptr(), x.numel(), code,
                                                    count.data_ptr(), _stream(x, stream)), "dws_partition_flagged")
    return out, count


def reduce_by_key(keys, values, unique_keys=None, aggregates=None, count=None, stream=None):
    """Runs of equal keys (32-bit patterns): unique_keys[:r], aggregates[:r]
    (+ of the values per run), r in the int64 GPU tensor ``count``."""
    import torch
    _check_like(keys, keys, "keys")
    code = _dtype_code(values)
    _check_like(values, keys, "values")
    unique_keys = torch.empty_like(keys) if unique_keys is None else unique_keys
    aggregates = torch.empty_like(values) if aggregates is None else aggregates
    _check_like(unique_keys, keys, "unique_keys")
    _check_like(aggregates, keys, "aggregates")
    count = _count_tensor(keys, count)
    with _device_of(keys):
        _check(load_library().dws_reduce_by_key(keys.data_ptr(), values.data_ptr(), unique_keys.data_ptr(),
                                                aggregates.data_ptr(), keys.numel(), code, count.data_ptr(),
                                                _stream(keys, stream)), "dws_reduce_by_key")
    return unique_keys, aggregates, count


def run_length_encode(keys, unique_keys=None, lengths=None, count=None, stream=None):
    """Runs of equal keys: unique_keys[:r], int32 tensor of uint32 lengths[:r],
    r in the int64 GPU tensor ``count``."""
    import torch
    _check_like(keys, keys, "keys")
    unique_keys = torch.empty_like(keys) if unique_keys is None else unique_keys
    lengths = torch.empty(keys.numel(), dtype=torch.int32, device=keys.device) if lengths is None else lengths
    _check_like(unique_keys, keys, "unique_keys")
    _check_like(lengths, keys, "lengths")
    count = _count_tensor(keys, count)
    with _device_of(keys):
        _check(load_library().dws_run_length_encode(keys.data_ptr(), unique_keys.data_ptr(), lengths.data_ptr(),
                                                    keys.numel(), count.data_ptr(), _stream(keys, stream)),
               "dws_run_length_encode")
    return unique_keys, lengths, count


def device_memory_info() -> dict:
    """Memory clock (kHz), memory bus width (bits) and compute units of the
    current device, as the HIP runtime reports them."""
    clk, width, cus = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(load_library().dws_device_memory_info(ctypes.byref(clk), ctypes.byref(width), ctypes.byref(cus)),
           "dws_device_memory_info")
    return {"memory_clock_khz": clk.value, "memory_bus_width_bits": width.value, "compute_units": cus.value}


def watchdog_trips() -> int:
    v = ctypes.c_ulonglong(0)
    _check(load_library().dws_watchdog_trips(ctypes.byref(v)), "dws_watchdog_trips")
    return int(v.value)


def selftest_wave(x, stream=None):
    """Apply the kernels' wave64 primitives to each group of 64 elements of x:
    returns (in-wave inclusive scan, previous-lane value)."""
    import torch
    code, _ = _prepare(x, None)
    if x.numel() % 64:
        raise ValueError("selftest_wave needs a multiple of 64 elements")
    incl = torch.empty_like(x)
    shift = torch.empty_like(x)
    with _device_of(x):
        _check(load_library().dws_selftest_wave(x.data_ptr(), incl.data_ptr(), shift.data_ptr(),
                                                x.numel() // 64, code, _stream(x, stream)),
               "dws_selftest_wave")
    return incl, shift


def reserve(n: int, stream=None, device=None):
    import torch
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
    with torch.cuda.device(dev):
        s = int(torch.cuda.current_stream(dev).cuda_stream) if stream is None else int(stream)
        _check(load_library().dws_reserve(int(n), s), "dws_reserve")


def release_workspaces():
    _check(load_library().dws_release_workspaces(), "dws_release_workspaces")


def tile_elems(tile_shape: int = 0, n: int = 1 << 28, aligned: bool = True) -> int:
    """Elements per tile the single-pass kernel uses (tile_shape 0 = automatic
    choice for n)."""
    return int(load_library().dws_tile_elems(int(tile_shape), int(n), int(bool(aligned))))


def tile_threads(tile_shape: int = 0, n: int = 1 << 28, aligned: bool = True) -> int:
    return int(load_library().dws_tile_threads(int(tile_shape), int(n), int(bool(aligned))))


def num_tile_shapes() -> int:
    return int(load_library().dws_num_tile_shapes())


class _device_of:
    """Make x's device current for the C call (the library works on the
    current HIP device)."""

    def __init__(self, x):
        self.x = x
        self.ctx = None

    def __enter__(self):
        import torch
        self.ctx = torch.cuda.device(self.x.device)
        self.ctx.__enter__()

    def __exit__(self, *exc):
        self.ctx.__exit__(*exc)
        return False

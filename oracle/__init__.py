"""Sequential CPU oracle for the + prefix scan (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of bench.py may
import this package. The product library (device_wide_prefix_amd) never imports
it, and it imports nothing from the product library.

The arithmetic lives in ``scan_oracle.c`` (one sequential loop per dtype; the
header of that file gives the definitions and the pages they follow). This
module only compiles it with gcc and marshals numpy arrays through ctypes.

Functions:
    scan_u32(x, exclusive)  -> same dtype as x (uint32 or int32, scanned as bits)
    scan_i32                -> alias of scan_u32
    scan_f32(x, exclusive)  -> (y fp64, sabs fp64)
    scan(x, exclusive)      -> dispatch on x.dtype
    select_flagged(x, flags) -> the x[i] with flags[i] != 0, in order
    partition_flagged(x, flags) -> (selected in order then rejected reversed, count)
    reduce_by_key(keys, vals)   -> (unique keys, sums per run[, |value| sums per run])
    run_length_encode(keys)     -> (unique keys, run lengths)
    scan_minmax(x, is_max, exclusive)        -> running max/min (int32 signed, uint32 unsigned)
    scan_pair_sum_u32 / scan_affine_u32 / scan_segsum_u32(x, exclusive)
                            -> (n, 2) uint32 pairs in, (n, 2) uint32 out
    scan_pair_sum_i32_f32 / scan_segsum_i32_f32(x, exclusive)
                            -> (int32 part, fp64 part, |fp| sum), pairs in as (n, 2) words
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "scan_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_scan.so")
_ABI_VERSION = 1

# gcc flags: no fast-math and no contraction, so every fp64 addition rounds once,
# in the order the loop states.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """Compile one C source of the oracle into a shared library at ``out``."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile scan_oracle.c into liboracle_scan.so."""
    if not force and os.path.exists(LIBRARY):
        return LIBRARY
    return compile_source(SOURCE, LIBRARY)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class OracleLib:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_abi_version.restype = ctypes.c_int
        if lib.oracle_abi_version() != _ABI_VERSION:
            raise RuntimeError(f"{path} is stale; rebuild it")
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.oracle_scan_u32.argtypes = [vp, sz, vp, ctypes.c_int]
        lib.oracle_scan_u32.restype = ctypes.c_int
        lib.oracle_scan_f32.argtypes = [vp, sz, vp, vp, ctypes.c_int]
        lib.oracle_scan_f32.restype = ctypes.c_int
        lib.oracle_select_flagged.argtypes = [vp, vp, sz, vp]
        lib.oracle_select_flagged.restype = sz
        lib.oracle_partition_flagged.argtypes = [vp, vp, sz, vp]
        lib.oracle_partition_flagged.restype = sz
        lib.oracle_reduce_by_key_u32.argtypes = [vp, vp, sz, vp, vp]
        lib.oracle_reduce_by_key_u32.restype = sz
        lib.oracle_reduce_by_key_f32.argtypes = [vp, vp, sz, vp, vp, vp]
        lib.oracle_reduce_by_key_f32.restype = sz
        lib.oracle_run_length_encode.argtypes = [vp, sz, vp, vp]
        lib.oracle_run_length_encode.restype = sz
        ci = ctypes.c_int
        lib.oracle_scan_minmax.argtypes = [vp, sz, vp, ci, ci, ci]
        for name in ("oracle_scan_pair_sum_u32", "oracle_scan_affine_u32", "oracle_scan_segsum_u32"):
            getattr(lib, name).argtypes = [vp, sz, vp, ci]
        for name in ("oracle_scan_pair_sum_i32_f32", "oracle_scan_segsum_i32_f32"):
            getattr(lib, name).argtypes = [vp, sz, vp, vp, vp, ci]
        for name in ("oracle_scan_minmax", "oracle_scan_pair_sum_u32", "oracle_scan_affine_u32",
                     "oracle_scan_segsum_u32", "oracle_scan_pair_sum_i32_f32", "oracle_scan_segsum_i32_f32"):
            getattr(lib, name).restype = ci
        self._lib = lib
        self.path = path

    def scan_u32(self, x: np.ndarray, exclusive: bool = False,
                 out: np.ndarray | None = None) -> np.ndarray:
        """Prefix sum of 32-bit integers modulo 2^32 (uint32 or int32 in,
        same dtype out). ``out`` may be ``x`` itself."""
        x = np.ascontiguousarray(x)
        if x.dtype not in (np.uint32, np.int32):
            raise TypeError(f"scan_u32 wants uint32/int32, got {x.dtype}")
        y = np.empty_like(x) if out is None else out
        if y.shape != x.shape or y.dtype != x.dtype or not y.flags.c_contiguous:
            raise ValueError("out must be a contiguous array like x")
        rc = self._lib.oracle_scan_u32(_ptr(x), x.size, _ptr(y), int(bool(exclusive)))
        if rc != 0:
            raise RuntimeError(f"oracle_scan_u32 failed ({rc})")
        return y

    def scan_f32(self, x: np.ndarray, exclusive: bool = False, want_sabs: bool = True):
        """Prefix sum of fp32 values accumulated in fp64. Returns (y, sabs),
        both fp64; sabs[i] = sum of |x[j]| for j <= i (None if not asked)."""
        x = np.ascontiguousarray(x)
        if x.dtype != np.float32:
            raise TypeError(f"scan_f32 wants float32, got {x.dtype}")
        y = np.empty(x.shape, dtype=np.float64)
        s = np.empty(x.shape, dtype=np.float64) if want_sabs else None
        rc = self._lib.oracle_scan_f32(_ptr(x), x.size, _ptr(y),
                                       _ptr(s) if s is not None else None,
                                       int(bool(exclusive)))
        if rc != 0:
            raise RuntimeError(f"oracle_scan_f32 failed ({rc})")
        return y, s


    def select_flagged(self, x: np.ndarray, flags: np.ndarray) -> np.ndarray:
        """Elements of x (any 4-byte dtype, moved as bits) whose int32 flag is
        non-zero, in order."""
        x = np.ascontiguousarray(x)
        flags = np.ascontiguousarray(flags, dtype=np.int32)
        if x.itemsize != 4 or x.shape != flags.shape:
            raise ValueError("x must hold 4-byte elements, one flag each")
        out = np.empty_like(x)
        cnt = self._lib.oracle_select_flagged(_ptr(x), _ptr(flags), x.size, _ptr(out))
        return out[:cnt]


    # -- compaction family --------------------------------------------------

    def partition_flagged(self, x: np.ndarray, flags: np.ndarray):
        """(out, count): selected x in order, then the rejected ones reversed."""
        x = np.ascontiguousarray(x)
        flags = np.ascontiguousarray(flags, dtype=np.int32)
        if x.itemsize != 4 or x.shape != flags.shape:
            raise ValueError("x must hold 4-byte elements, one flag each")
        out = np.empty_like(x)
        cnt = self._lib.oracle_partition_flagged(_ptr(x), _ptr(flags), x.size, _ptr(out))
        return out, int(cnt)

    def reduce_by_key(self, keys: np.ndarray, vals: np.ndarray):
        """Runs of equal 32-bit keys: (unique keys, aggregates[, |value| sums]).
        float32 values give fp64 aggregates and the |value| sums; 32-bit
        integer values give wrapped sums of the same dtype and no |value| sums."""
        keys = np.ascontiguousarray(keys)
        vals = np.ascontiguousarray(vals)
        if keys.itemsize != 4 or vals.itemsize != 4 or keys.shape != vals.shape:
            raise ValueError("keys and values are equal-length 4-byte arrays")
        n = keys.size
        uk = np.empty(n, dtype=np.uint32)
        if vals.dtype == np.float32:
            ag = np.empty(n, dtype=np.float64)
            ab = np.empty(n, dtype=np.float64)
            r = self._lib.oracle_reduce_by_key_f32(_ptr(keys), _ptr(vals), n, _ptr(uk), _ptr(ag), _ptr(ab))
            return uk[:r].view(keys.dtype), ag[:r], ab[:r]
        ag = np.empty(n, dtype=vals.dtype)
        r = self._lib.oracle_reduce_by_key_u32(_ptr(keys), _ptr(vals), n, _ptr(uk), _ptr(ag))
        return uk[:r].view(keys.dtype), ag[:r], None

    def run_length_encode(self, keys: np.ndarray):
        """Runs of equal 32-bit keys: (unique keys, uint32 lengths)."""
        keys = np.ascontiguousarray(keys)
        if keys.itemsize != 4:
            raise ValueError("keys are 4-byte elements")
        n = keys.size
        uk = np.empty(n, dtype=np.uint32)
        ln = np.empty(n, dtype=np.uint32)
        r = self._lib.oracle_run_length_encode(_ptr(keys), n, _ptr(uk), _ptr(ln))
        return uk[:r].view(keys.dtype), ln[:r]

    # -- generic operators ---------------------------------------------------
    # Pairs travel as (n, 2) uint32 arrays of bits: column 0 the first
    # component, column 1 the second.

    def scan_minmax(self, x: np.ndarray, is_max: bool, exclusive: bool = False) -> np.ndarray:
        """Running max/min of int32 (signed) or uint32 (unsigned) values."""
        x = np.ascontiguousarray(x)
        if x.dtype not in (np.int32, np.uint32):
            raise TypeError("scan_minmax wants int32 or uint32")
        y = np.empty_like(x)
        rc = self._lib.oracle_scan_minmax(_ptr(x), x.size, _ptr(y), int(x.dtype == np.int32), int(bool(is_max)),
                                          int(bool(exclusive)))
        if rc != 0:
            raise RuntimeError("oracle_scan_minmax failed")
        return y

    def _pair_u32(self, name: str, x: np.ndarray, exclusive: bool) -> np.ndarray:
        x = _as_pairs(x)
        y = np.empty_like(x)
        if getattr(self._lib, name)(_ptr(x), x.shape[0], _ptr(y), int(bool(exclusive))) != 0:
            raise RuntimeError(f"{name} failed")
        return y

    def scan_pair_sum_u32(self, x, exclusive=False):
        """Componentwise + of uint32 pairs, modulo 2^32; (n, 2) uint32."""
        return self._pair_u32("oracle_scan_pair_sum_u32", x, exclusive)

    def scan_affine_u32(self, x, exclusive=False):
        """Composition of the affine maps v -> a v + b (mod 2^32), element
        (a, b); returns the running (A, B) as (n, 2) uint32."""
        return self._pair_u32("oracle_scan_affine_u32", x, exclusive)

    def scan_segsum_u32(self, x, exclusive=False):
        """Segmented + on (flag, value) uint32 pairs; (n, 2) uint32 of
        (OR of flags so far, segment sum)."""
        return self._pair_u32("oracle_scan_segsum_u32", x, exclusive)

    def _pair_if(self, name: str, x: np.ndarray, exclusive: bool):
        x = _as_pairs(x)
        n = x.shape[0]
        yi = np.empty(n, dtype=np.int32)
        yf = np.empty(n, dtype=np.float64)
        sa = np.empty(n, dtype=np.float64)
        if getattr(self._lib, name)(_ptr(x), n, _ptr(yi), _ptr(yf), _ptr(sa), int(bool(exclusive))) != 0:
            raise RuntimeError(f"{name} failed")
        return yi, yf, sa

    def scan_pair_sum_i32_f32(self, x, exclusive=False):
        """Componentwise + of {int32, fp32} pairs: (int32 part, fp64 part,
        running |fp part| over j <= i)."""
        return self._pair_if("oracle_scan_pair_sum_i32_f32", x, exclusive)

    def scan_segsum_i32_f32(self, x, exclusive=False):
        """Segmented + on {int32 flag, fp32 value} pairs: (OR of flags so far,
        fp64 segment sum, sum of |value| over the elements in that sum)."""
        return self._pair_if("oracle_scan_segsum_i32_f32", x, exclusive)


def _as_pairs(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.ndim != 2 or x.shape[1] != 2 or x.dtype.itemsize != 4:
        raise ValueError("pairs are (n, 2) arrays of 4-byte words")
    return x.view(np.uint32)


def make_pairs(first: np.ndarray, second: np.ndarray) -> np.ndarray:
    """(n, 2) uint32 bit array from two 4-byte columns (any 4-byte dtypes)."""
    out = np.empty((first.size, 2), dtype=np.uint32)
    out[:, 0] = np.ascontiguousarray(first).view(np.uint32)
    out[:, 1] = np.ascontiguousarray(second).view(np.uint32)
    return out


_default: OracleLib | None = None


def _oracle() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build(force=True)
        _default = OracleLib(LIBRARY)
    return _default


def scan_u32(x, exclusive=False, out=None):
    return _oracle().scan_u32(x, exclusive, out)


scan_i32 = scan_u32


def scan_f32(x, exclusive=False, want_sabs=True):
    return _oracle().scan_f32(x, exclusive, want_sabs)


def select_flagged(x, flags):
    return _oracle().select_flagged(x, flags)


def partition_flagged(x, flags):
    return _oracle().partition_flagged(x, flags)


def reduce_by_key(keys, vals):
    return _oracle().reduce_by_key(keys, vals)


def run_length_encode(keys):
    return _oracle().run_length_encode(keys)


def scan_minmax(x, is_max, exclusive=False):
    return _oracle().scan_minmax(x, is_max, exclusive)


def scan_pair_sum_u32(x, exclusive=False):
    return _oracle().scan_pair_sum_u32(x, exclusive)


def scan_affine_u32(x, exclusive=False):
    return _oracle().scan_affine_u32(x, exclusive)


def scan_segsum_u32(x, exclusive=False):
    return _oracle().scan_segsum_u32(x, exclusive)


def scan_pair_sum_i32_f32(x, exclusive=False):
    return _oracle().scan_pair_sum_i32_f32(x, exclusive)


def scan_segsum_i32_f32(x, exclusive=False):
    return _oracle().scan_segsum_i32_f32(x, exclusive)


def scan(x: np.ndarray, exclusive: bool = False):
    """Integers give the wrapped integer scan; float32 gives the fp64 sums."""
    if x.dtype in (np.uint32, np.int32):
        return scan_u32(x, exclusive)
    if x.dtype == np.float32:
        return scan_f32(x, exclusive, want_sabs=False)[0]
    raise TypeError(f"unsupported dtype {x.dtype}")

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


def scan(x: np.ndarray, exclusive: bool = False):
    """Integers give the wrapped integer scan; float32 gives the fp64 sums."""
    if x.dtype in (np.uint32, np.int32):
        return scan_u32(x, exclusive)
    if x.dtype == np.float32:
        return scan_f32(x, exclusive, want_sabs=False)[0]
    raise TypeError(f"unsupported dtype {x.dtype}")

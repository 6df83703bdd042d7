"""Seeded synthetic inputs for the device-wide prefix scan.

This module only draws random numbers and names the workloads. It holds none of
the scan's arithmetic, and it is the one piece of code that both the oracle side
(tests, CPU baseline) and the HIP side (tests, bench, smoke) use, so that both
see the same input array.

Generator: numpy PCG64 through ``numpy.random.default_rng(seed)``. The pages give
no generator; only seeds, sizes and value distributions are fixed by the
workloads below, and parity does not depend on the choice because both sides
consume the same array.

Workloads (sizes, dtypes, distributions and scan kinds of the measured
configurations):
  i32_4096_incl                 N = 4096          int32   uniform integers 0..9        inclusive, seed 0
  f32_2p20_incl                 N = 2^20          float32 uniform [-1, 1)              inclusive, seed 1
  u32_2p26_incl                 N = 2^26          uint32  uniform over [0, 2^32)       inclusive, seed 2
  f32_2p28_excl_inplace         N = 2^28          float32 uniform [0, 1), in place     exclusive, seed 3
  flags_2p30m12345_excl N = 2^30 - 12345  int32   Bernoulli(0.5) 0/1 flags     exclusive, seed 4

Stream compaction (select by flags) reuses the 0/1 flags workload's flags as the selection and
draws the values to move as uniform int32 with seed 5 (SELECT_VALUE_SEED).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    dtype: str          # "int32" | "uint32" | "float32"
    dist: str           # key of DISTRIBUTIONS
    seed: int
    exclusive: bool
    in_place: bool
    description: str

    @property
    def itemsize(self) -> int:
        return 4

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes a scan must move at minimum: read n elements, write n."""
        return 2 * self.n * self.itemsize


WORKLOADS = {
    "i32_4096_incl": Workload(
        "i32_4096_incl", 4096, "int32", "int_0_9", 0, False, False,
        "inclusive + scan, N=4096 int32 uniform integers 0..9, seed 0"),
    "f32_2p20_incl": Workload(
        "f32_2p20_incl", 1 << 20, "float32", "f32_pm1", 1, False, False,
        "inclusive + scan, N=2^20 fp32 uniform [-1,1), seed 1"),
    "u32_2p26_incl": Workload(
        "u32_2p26_incl", 1 << 26, "uint32", "u32_full", 2, False, False,
        "inclusive + scan mod 2^32, N=2^26 uint32 uniform over [0,2^32), seed 2"),
    "f32_2p28_excl_inplace": Workload(
        "f32_2p28_excl_inplace", 1 << 28, "float32", "f32_01", 3, True, True,
        "exclusive + scan in place, N=2^28 fp32 uniform [0,1), seed 3"),
    "flags_2p30m12345_excl": Workload(
        "flags_2p30m12345_excl", (1 << 30) - 12345, "int32", "flags_half", 4, True, False,
        "exclusive + scan, N=2^30-12345 int32 0/1 flags Bernoulli(0.5), seed 4"),
}


SELECT_VALUE_SEED = 5


def _int_0_9(rng, n):
    return rng.integers(0, 10, size=n, dtype=np.int32)


def _f32_pm1(rng, n):
    # uniform on [-1, 1): draw fp32 in [0, 1) and map affinely (exact in fp32
    # up to one rounding of 2u - 1)
    u = rng.random(n, dtype=np.float32)
    return (u * np.float32(2.0) - np.float32(1.0)).astype(np.float32, copy=False)


def _u32_full(rng, n):
    return rng.integers(0, 1 << 32, size=n, dtype=np.uint32)


def _f32_01(rng, n):
    return rng.random(n, dtype=np.float32)


def _flags_half(rng, n):
    return rng.integers(0, 2, size=n, dtype=np.int32)


def _i32_full(rng, n):
    return rng.integers(-(1 << 31), 1 << 31, size=n, dtype=np.int32)


def _f32_normal(rng, n):
    return rng.standard_normal(n, dtype=np.float32)


DISTRIBUTIONS = {
    "int_0_9": _int_0_9,
    "f32_pm1": _f32_pm1,
    "u32_full": _u32_full,
    "f32_01": _f32_01,
    "flags_half": _flags_half,
    "i32_full": _i32_full,
    "f32_normal": _f32_normal,
}

# default distribution per dtype for ad-hoc parity cases
DEFAULT_DIST = {"int32": "i32_full", "uint32": "u32_full", "float32": "f32_pm1"}


def selection_flags(n: int, density: float, seed: int, any_nonzero: bool = False) -> np.ndarray:
    """int32 selection flags, each non-zero with probability ``density``
    (Bernoulli from PCG64(seed)). Non-zero flags are 1, or with
    ``any_nonzero`` a uniform non-zero int32 (negative values included)."""
    rng = np.random.default_rng(seed)
    on = rng.random(int(n)) < density
    if not any_nonzero:
        return on.astype(np.int32)
    v = rng.integers(-(1 << 31), 1 << 31, size=int(n), dtype=np.int64)
    v[v == 0] = 1
    return np.where(on, v, 0).astype(np.int32)


OP_INPUTS = ("i32_full", "u32_full", "pair_i32_f32", "pair_u32", "affine_u32", "segsum_u32", "segsum_i32_f32")


def op_input(kind: str, n: int, seed: int, head_density: float = 0.01) -> np.ndarray:
    """Seeded inputs for the generic-operator scans. 32-bit kinds give (n,)
    arrays; pair kinds give (n, 2) uint32 arrays of bits (column 0 the first
    component):
      pair_i32_f32    uniform int32, uniform [-1, 1) fp32
      pair_u32        two uniform uint32
      affine_u32      (a, b): a odd with probability 0.9 (else uniform), b
                      uniform, so that most running products stay non-zero
      segsum_u32      (flag, value): flag non-zero (uniform non-zero int32
                      bits) with probability head_density, value uniform
      segsum_i32_f32  the same flags, value uniform [-1, 1) fp32"""
    rng = np.random.default_rng(seed)
    n = int(n)
    if kind == "i32_full":
        return _i32_full(rng, n)
    if kind == "u32_full":
        return _u32_full(rng, n)
    out = np.empty((n, 2), dtype=np.uint32)
    if kind == "pair_i32_f32":
        out[:, 0] = _i32_full(rng, n).view(np.uint32)
        out[:, 1] = _f32_pm1(rng, n).view(np.uint32)
    elif kind == "pair_u32":
        out[:, 0] = _u32_full(rng, n)
        out[:, 1] = _u32_full(rng, n)
    elif kind == "affine_u32":
        a = _u32_full(rng, n)
        odd = rng.random(n) < 0.9
        out[:, 0] = np.where(odd, a | np.uint32(1), a)
        out[:, 1] = _u32_full(rng, n)
    elif kind in ("segsum_u32", "segsum_i32_f32"):
        heads = rng.random(n) < head_density
        f = _u32_full(rng, n)
        f[f == 0] = 1
        out[:, 0] = np.where(heads, f, np.uint32(0))
        out[:, 1] = _u32_full(rng, n) if kind == "segsum_u32" else _f32_pm1(rng, n).view(np.uint32)
    else:
        raise KeyError(kind)
    return out


def run_keys(n: int, mean_run: float, seed: int) -> np.ndarray:
    """uint32 keys in runs: each element starts a new run with probability
    1 / mean_run (element 0 always does); run r gets the key r * 2654435761
    mod 2^32, so adjacent runs differ. mean_run = 1 gives all-distinct keys,
    mean_run >= n typically one run."""
    rng = np.random.default_rng(seed)
    n = int(n)
    starts = rng.random(n) < (1.0 / mean_run)
    if n:
        starts[0] = True
    run = np.cumsum(starts, dtype=np.uint64) - np.uint64(1)
    return ((run * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def generate(dist: str, n: int, seed: int) -> np.ndarray:
    """Draw ``n`` values of distribution ``dist`` from PCG64(seed)."""
    rng = np.random.default_rng(seed)
    return DISTRIBUTIONS[dist](rng, int(n))


def generate_workload(w: Workload) -> np.ndarray:
    return generate(w.dist, w.n, w.seed)


def random_input(dtype: str, n: int, seed: int) -> np.ndarray:
    return generate(DEFAULT_DIST[dtype], n, seed)

"""Pins for the CPU oracle: each check ties it to something other than itself.

- values the pages print: the 16-element worked examples of the PMPP 11.3
  (hierarchical scan) and 11.2 (three-phase coarsened scan) notes, and the
  premise of Fig 6 of the decoupled look-back paper (tests/golden/);
- the exclusive definition (identity first, then the inclusive shifted by one),
  as the smarter.xin RTX 4090 scan notes state it in their section on
  inclusive/exclusive conversion;
- closed forms (constant and arithmetic inputs, with the modulo-2^32 wrap);
- a witness that fp32 inputs are accumulated in fp64;
- O(n^2) brute force on small n with exact Python integers / math.fsum;
- numpy's cumsum, an independent library routine, on the seeded workloads;
- for the generic operators: numpy's maximum/minimum.accumulate and per-column
  cumsum, the affine recurrence run directly from several start values, and
  brute-force segmented sums.

The last test plants plausible mistakes in copies of the oracle's C source,
compiles each copy with gcc on the CPU and checks that every mutant fails at
least one of the pins above.
"""
import math
import os

import numpy as np
import pytest

import oracle
import scan_workloads as wl
from golden_io import read_golden

M32 = 0xFFFFFFFF


def _golden_checks(lib, fname, fail):
    g = read_golden(fname)
    x = np.array(g["input"], dtype=np.int32)
    b = g["block_size"]
    incl = lib.scan_u32(x, exclusive=False)
    excl = lib.scan_u32(x, exclusive=True)
    if incl.tolist() != g["inclusive"]:
        fail(f"{fname}: inclusive")
    # the scanned block sums are the final values at the block ends
    if incl[b - 1::b].tolist() != g["scanned_block_sums"]:
        fail(f"{fname}: block-end values")
    # step 1 of the example: each block scanned on its own
    for k in range(len(g["block_sums"])):
        local = lib.scan_u32(x[k * b:(k + 1) * b], exclusive=False)
        if local.tolist() != g["block_local_inclusive"][k * b:(k + 1) * b]:
            fail(f"{fname}: block {k} local scan")
        if int(local[-1]) != g["block_sums"][k]:
            fail(f"{fname}: block {k} sum")
    # step 2: scanning the block sums gives the scanned block sums
    s = lib.scan_u32(np.array(g["block_sums"], dtype=np.int32))
    if s.tolist() != g["scanned_block_sums"]:
        fail(f"{fname}: scan of block sums")
    # exclusive: identity first, then the inclusive result shifted by one
    if excl.tolist() != [0] + g["inclusive"][:-1]:
        fail(f"{fname}: exclusive")
    # the fp32 oracle gives the same integers (small exact values)
    yf, sf = lib.scan_f32(x.astype(np.float32))
    if yf.tolist() != [float(v) for v in g["inclusive"]]:
        fail(f"{fname}: fp32 inclusive")
    if sf.tolist() != [float(v) for v in g["inclusive"]]:   # inputs are >= 0
        fail(f"{fname}: fp32 running |x|")
    yfe, _ = lib.scan_f32(x.astype(np.float32), exclusive=True)
    if yfe.tolist() != [0.0] + [float(v) for v in g["inclusive"][:-1]]:
        fail(f"{fname}: fp32 exclusive")


def _fig6_checks(lib, fail):
    g = read_golden("decoupled_lookback_fig6.txt")
    p, s = g["partitions"], g["partition_sum"]
    rng = np.random.default_rng(6)
    # partitions of 5 elements whose values are non-negative and sum to s
    parts = []
    for _ in range(p):
        cut = np.sort(rng.integers(0, s + 1, size=4))
        parts.append(np.diff(np.concatenate([[0], cut, [s]])))
    x = np.concatenate(parts).astype(np.int32)
    incl = lib.scan_u32(x)
    if incl[4::5].tolist() != [s * (t + 1) for t in range(p)]:
        fail("fig6: inclusive prefix at partition ends")


def _closed_form_checks(lib, fail):
    n = 1000
    ones = np.ones(n, dtype=np.int32)
    if lib.scan_u32(ones).tolist() != list(range(1, n + 1)):
        fail("ones inclusive")
    if lib.scan_u32(ones, exclusive=True).tolist() != list(range(n)):
        fail("ones exclusive")
    c = np.full(n, 7, dtype=np.uint32)
    if lib.scan_u32(c).tolist() != [7 * (i + 1) for i in range(n)]:
        fail("constant inclusive")
    # arithmetic input x[i] = i; the sums pass 2^32 and wrap
    n = 100_000
    ar = np.arange(n, dtype=np.uint32)
    want = [(i * (i + 1) // 2) & M32 for i in range(n)]
    if lib.scan_u32(ar).tolist() != want:
        fail("arithmetic inclusive mod 2^32")
    want_ex = [(i * (i - 1) // 2) & M32 for i in range(n)]
    if lib.scan_u32(ar, exclusive=True).tolist() != want_ex:
        fail("arithmetic exclusive mod 2^32")
    # int32 is the same bits
    got = lib.scan_u32(ar.view(np.int32)).view(np.uint32).tolist()
    if got != want:
        fail("arithmetic int32 bits")
    # wrap at the boundary
    if lib.scan_u32(np.array([M32, 1, 5], dtype=np.uint32)).tolist() != [M32, 0, 5]:
        fail("uint32 wrap")
    imax = np.array([2**31 - 1, 1, 1], dtype=np.int32)
    if lib.scan_u32(imax).tolist() != [2**31 - 1, -2**31, -2**31 + 1]:
        fail("int32 wrap")
    # fp32 closed form, exact in fp64
    h = np.full(n, 0.5, dtype=np.float32)
    y, s = lib.scan_f32(h)
    if not np.array_equal(y, 0.5 * np.arange(1, n + 1)):
        fail("fp32 constant inclusive")
    ye, se = lib.scan_f32(h, exclusive=True)
    if not np.array_equal(ye, 0.5 * np.arange(n)):
        fail("fp32 constant exclusive")
    # the running |x| covers element i itself, for both scan kinds
    neg = np.full(10, -1.0, dtype=np.float32)
    y, s = lib.scan_f32(neg)
    if y.tolist() != [-float(i) for i in range(1, 11)] or s.tolist() != [float(i) for i in range(1, 11)]:
        fail("fp32 negative constant / running |x|")
    _, se = lib.scan_f32(neg, exclusive=True)
    if se.tolist() != [float(i) for i in range(1, 11)]:
        fail("fp32 exclusive running |x|")
    mixed = np.array([3.0, -2.0, 0.5], dtype=np.float32)
    y, s = lib.scan_f32(mixed)
    if y.tolist() != [3.0, 1.0, 1.5] or s.tolist() != [3.0, 5.0, 5.5]:
        fail("fp32 mixed signs")


def _fp64_witness_checks(lib, fail):
    # 2^24 + 1 is not an fp32 number; an fp32 accumulator would stall at 2^24
    x = np.array([2.0**24, 1.0, 1.0, 1.0], dtype=np.float32)
    y, _ = lib.scan_f32(x)
    if y.tolist() != [2.0**24, 2.0**24 + 1, 2.0**24 + 2, 2.0**24 + 3]:
        fail("fp64 accumulation (inclusive)")
    ye, _ = lib.scan_f32(x, exclusive=True)
    if ye.tolist() != [0.0, 2.0**24, 2.0**24 + 1, 2.0**24 + 2]:
        fail("fp64 accumulation (exclusive)")


def _brute_force_checks(lib, fail):
    rng = np.random.default_rng(123)
    for n in (1, 2, 3, 17, 64, 65, 300):
        x = rng.integers(-(2**31), 2**31, size=n, dtype=np.int64).astype(np.int32)
        xs = [int(v) for v in x]
        want = [sum(xs[:i + 1]) & M32 for i in range(n)]
        want_ex = [sum(xs[:i]) & M32 for i in range(n)]
        if lib.scan_u32(x).view(np.uint32).tolist() != want:
            fail(f"brute force int32 inclusive n={n}")
        if lib.scan_u32(x, exclusive=True).view(np.uint32).tolist() != want_ex:
            fail(f"brute force int32 exclusive n={n}")
        # dyadic fp32 inputs: every partial sum is exact in fp64, so the fp64
        # running sum must equal the correctly rounded (= exact) fsum
        f = (rng.integers(-1024, 1025, size=n) / 1024.0).astype(np.float32)
        fl = [float(v) for v in f]
        y, s = lib.scan_f32(f)
        if y.tolist() != [math.fsum(fl[:i + 1]) for i in range(n)]:
            fail(f"brute force fp32 inclusive n={n}")
        if s.tolist() != [math.fsum(abs(v) for v in fl[:i + 1]) for i in range(n)]:
            fail(f"brute force fp32 running |x| n={n}")
        ye, _ = lib.scan_f32(f, exclusive=True)
        if ye.tolist() != [math.fsum(fl[:i]) for i in range(n)]:
            fail(f"brute force fp32 exclusive n={n}")


def _select_checks(lib, fail):
    rng = np.random.default_rng(77)
    # closed forms
    x = np.arange(1000, dtype=np.uint32)
    if lib.select_flagged(x, np.ones(1000, np.int32)).tolist() != x.tolist():
        fail("select all")
    if lib.select_flagged(x, np.zeros(1000, np.int32)).size != 0:
        fail("select none")
    alt = (np.arange(1000) % 2 == 0).astype(np.int32)
    if lib.select_flagged(x, alt).tolist() != list(range(0, 1000, 2)):
        fail("select even positions")
    # any non-zero flag selects, negative ones included
    f = np.array([0, -1, 5, 0, 2**31 - 1, -(2**31)], dtype=np.int32)
    if lib.select_flagged(np.arange(6, dtype=np.uint32), f).tolist() != [1, 2, 4, 5]:
        fail("select non-zero flags")
    # brute force against a Python list comprehension, and the scatter form:
    # selected element i lands at the exclusive prefix sum of the 0/1 flags
    for n in (1, 2, 7, 64, 65, 300):
        xs = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        fl = rng.integers(-2, 3, size=n).astype(np.int32)
        got = lib.select_flagged(xs, fl)
        if got.tolist() != [int(v) for v, g in zip(xs, fl) if g != 0]:
            fail(f"select brute force n={n}")
        excl = lib.scan_u32((fl != 0).astype(np.int32), exclusive=True)
        scat = np.zeros(int(np.count_nonzero(fl)), dtype=np.uint32)
        dest = excl[fl != 0].astype(np.int64)
        if dest.size and (dest.min() < 0 or dest.max() >= scat.size):
            fail(f"select scatter offsets out of range n={n}")
            continue
        scat[dest] = xs[fl != 0]
        if not np.array_equal(got, scat):
            fail(f"select vs scatter to exclusive offsets n={n}")
    # float bits are moved unchanged
    fx = np.array([1.5, -0.0, np.inf, 3.25], dtype=np.float32)
    got = lib.select_flagged(fx, np.array([1, 1, 1, 0], np.int32))
    if got.view(np.uint32).tolist() != fx[:3].view(np.uint32).tolist():
        fail("select float bits")


def _minmax_checks(lib, fail):
    rng = np.random.default_rng(31)
    for dt, lo, hi in ((np.int32, -(2**31), 2**31), (np.uint32, 0, 2**32)):
        info = np.iinfo(dt)
        for n in (1, 2, 5, 64, 65, 1000):
            x = rng.integers(lo, hi, size=n, dtype=np.int64).astype(dt)
            xs = [int(v) for v in x]
            for is_max, acc, ident in ((True, np.maximum, info.min), (False, np.minimum, info.max)):
                y = lib.scan_minmax(x, is_max)
                ye = lib.scan_minmax(x, is_max, exclusive=True)
                # numpy's accumulate, an independent routine
                if not np.array_equal(y, acc.accumulate(x)):
                    fail(f"{dt.__name__} {'max' if is_max else 'min'} vs numpy n={n}")
                # brute force over every prefix
                f = max if is_max else min
                if n <= 65 and y.tolist() != [f(xs[:i + 1]) for i in range(n)]:
                    fail(f"{dt.__name__} {'max' if is_max else 'min'} brute force n={n}")
                # exclusive: the type's extreme first, then the shifted inclusive
                if ye.tolist() != [int(ident)] + y[:-1].tolist():
                    fail(f"{dt.__name__} {'max' if is_max else 'min'} exclusive n={n}")
    # signed and unsigned order differ on the top bit
    x = np.array([1, 0x80000000, 5], dtype=np.uint32)
    if lib.scan_minmax(x, True).tolist() != [1, 0x80000000, 0x80000000]:
        fail("unsigned max order")
    if lib.scan_minmax(x.view(np.int32), True).tolist() != [1, 1, 5]:
        fail("signed max order")


def _pair_sum_checks(lib, fail):
    rng = np.random.default_rng(32)
    for n in (1, 3, 64, 1000):
        a = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        b = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        y = lib.scan_pair_sum_u32(oracle.make_pairs(a, b))
        for col, v in ((0, a), (1, b)):
            want = (np.cumsum(v.astype(np.uint64)) & M32).astype(np.uint32)
            if not np.array_equal(y[:, col], want):
                fail(f"pair sum u32 column {col} n={n}")
        ye = lib.scan_pair_sum_u32(oracle.make_pairs(a, b), exclusive=True)
        if ye[0].tolist() != [0, 0] or not np.array_equal(ye[1:], y[:-1]):
            fail(f"pair sum u32 exclusive n={n}")
        # {int32, fp32}: the int part against numpy's integer cumsum, the fp
        # part against numpy's fp64 cumsum (both sequential)
        ia = rng.integers(-(2**31), 2**31, size=n, dtype=np.int64).astype(np.int32)
        fb = (rng.standard_normal(n)).astype(np.float32)
        yi, yf, sa = lib.scan_pair_sum_i32_f32(oracle.make_pairs(ia, fb))
        want_i = (np.cumsum(ia.astype(np.int64)) & M32).astype(np.uint32).view(np.int32)
        if not np.array_equal(yi, want_i):
            fail(f"pair sum i32 part n={n}")
        if not np.array_equal(yf, np.cumsum(fb.astype(np.float64))):
            fail(f"pair sum f32 part n={n}")
        if not np.array_equal(sa, np.cumsum(np.abs(fb.astype(np.float64)))):
            fail(f"pair sum running |f| n={n}")
        yie, yfe, sae = lib.scan_pair_sum_i32_f32(oracle.make_pairs(ia, fb), exclusive=True)
        if yie[0] != 0 or yfe[0] != 0.0 or not np.array_equal(yie[1:], yi[:-1]) or \
                not np.array_equal(yfe[1:], yf[:-1]) or not np.array_equal(sae, sa):
            fail(f"pair sum i32/f32 exclusive n={n}")


def _affine_checks(lib, fail):
    rng = np.random.default_rng(33)
    for n in (1, 2, 7, 64, 500):
        a = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        b = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        y = lib.scan_affine_u32(oracle.make_pairs(a, b))
        ye = lib.scan_affine_u32(oracle.make_pairs(a, b), exclusive=True)
        # the defining property: running the recurrence v = a v + b from any
        # start s gives A_i s + B_i at every i (checked for three starts)
        for s in (0, 1, int(rng.integers(0, 2**32))):
            v = s
            for i in range(n):
                v = (int(a[i]) * v + int(b[i])) & M32
                if v != (int(y[i, 0]) * s + int(y[i, 1])) & M32:
                    fail(f"affine recurrence n={n} s={s} i={i}")
                    break
        if ye[0].tolist() != [1, 0] or not np.array_equal(ye[1:], y[:-1]):
            fail(f"affine exclusive n={n}")
        # a = 1: B is the prefix sum of b; b = 0: A is the prefix product of a
        ones = np.ones(n, dtype=np.uint32)
        y1 = lib.scan_affine_u32(oracle.make_pairs(ones, b))
        if not np.array_equal(y1[:, 1], (np.cumsum(b.astype(np.uint64)) & M32).astype(np.uint32)) or \
                not np.all(y1[:, 0] == 1):
            fail(f"affine a=1 n={n}")
        y0 = lib.scan_affine_u32(oracle.make_pairs(a, np.zeros(n, np.uint32)))
        prod, want = 1, []
        for v in a:
            prod = (prod * int(v)) & M32
            want.append(prod)
        if y0[:, 0].tolist() != want or np.any(y0[:, 1] != 0):
            fail(f"affine b=0 n={n}")
    # order matters: the same two maps in the two orders
    p = lib.scan_affine_u32(np.array([[2, 1], [3, 4]], dtype=np.uint32))[-1].tolist()
    q = lib.scan_affine_u32(np.array([[3, 4], [2, 1]], dtype=np.uint32))[-1].tolist()
    if p != [6, 7] or q != [6, 9]:
        fail("affine composition order")


def _segsum_checks(lib, fail):
    rng = np.random.default_rng(34)
    for n in (1, 2, 9, 64, 300):
        flags = np.where(rng.random(n) < 0.2, rng.integers(1, 2**31, size=n), 0).astype(np.uint32)
        vals = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        y = lib.scan_segsum_u32(oracle.make_pairs(flags, vals))
        ye = lib.scan_segsum_u32(oracle.make_pairs(flags, vals), exclusive=True)
        # brute force: the sum since the last head at or before i, and the OR
        # of all flags up to i
        for i in range(n):
            h = max([j for j in range(i + 1) if flags[j] != 0], default=0)
            v = sum(int(vals[j]) for j in range(h, i + 1)) & M32
            f = 0
            for j in range(i + 1):
                f |= int(flags[j])
            if [int(y[i, 0]), int(y[i, 1])] != [f, v]:
                fail(f"segsum u32 brute force n={n} i={i}")
                break
        if ye[0].tolist() != [0, 0] or not np.array_equal(ye[1:], y[:-1]):
            fail(f"segsum u32 exclusive n={n}")
        # fp32 values (dyadic: every fp64 partial sum is exact), brute force
        # with fsum, and the |value| sum over the same elements
        fv = (rng.integers(-1024, 1025, size=n) / 64.0).astype(np.float32)
        yfl, yf, sa = lib.scan_segsum_i32_f32(oracle.make_pairs(flags, fv))
        yfle, yfe, sae = lib.scan_segsum_i32_f32(oracle.make_pairs(flags, fv), exclusive=True)
        for i in range(n):
            h = max([j for j in range(i + 1) if flags[j] != 0], default=0)
            seg = [float(fv[j]) for j in range(h, i + 1)]
            if yf[i] != math.fsum(seg) or sa[i] != math.fsum(abs(v) for v in seg):
                fail(f"segsum f32 brute force n={n} i={i}")
                break
        if yfle[0] != 0 or yfe[0] != 0.0 or sae[0] != 0.0 or not np.array_equal(yfe[1:], yf[:-1]) or \
                not np.array_equal(sae[1:], sa[:-1]) or not np.array_equal(yfle[1:], yfl[:-1]):
            fail(f"segsum f32 exclusive n={n}")
    # closed forms: every element a head gives the values back; no heads gives
    # the plain prefix sum (numpy)
    v = np.arange(1, 101, dtype=np.uint32)
    if not np.array_equal(lib.scan_segsum_u32(oracle.make_pairs(np.ones(100, np.uint32), v))[:, 1], v):
        fail("segsum all heads")
    if not np.array_equal(lib.scan_segsum_u32(oracle.make_pairs(np.zeros(100, np.uint32), v))[:, 1],
                          np.cumsum(v).astype(np.uint32)):
        fail("segsum no heads")


def _compaction_family_checks(lib, fail):
    import itertools
    rng = np.random.default_rng(35)
    for n in (1, 2, 7, 64, 1000):
        x = rng.integers(-(2**31), 2**31, size=n, dtype=np.int64).astype(np.int32)
        f = (rng.random(n) < 0.4).astype(np.int32) * rng.integers(-5, 6, size=n).astype(np.int32)
        out, cnt = lib.partition_flagged(x, f)
        # numpy's boolean indexing: selected in order, then rejected reversed
        if cnt != int(np.count_nonzero(f)) or not np.array_equal(out[:cnt], x[f != 0]) or \
                not np.array_equal(out[cnt:], x[f == 0][::-1]):
            fail(f"partition n={n}")
        # runs of keys drawn from a small alphabet, so that runs have length > 1
        keys = rng.integers(0, 3, size=n).astype(np.int32)
        vals = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
        groups = [(k, [int(vals[i]) for i, _ in g]) for k, g in itertools.groupby(enumerate(keys), key=lambda t: t[1])]
        uk, ag, _ = lib.reduce_by_key(keys, vals)
        if uk.tolist() != [int(k) for k, _ in groups] or ag.tolist() != [sum(v) & M32 for _, v in groups]:
            fail(f"reduce by key (groupby) n={n}")
        starts = np.concatenate([[0], np.flatnonzero(np.diff(keys) != 0) + 1])
        if not np.array_equal(ag, (np.add.reduceat(vals.astype(np.uint64), starts) & M32).astype(np.uint32)):
            fail(f"reduce by key (numpy reduceat) n={n}")
        fv = (rng.integers(-512, 513, size=n) / 32.0).astype(np.float32)
        ukf, agf, abf = lib.reduce_by_key(keys, fv)
        want = [math.fsum(float(fv[i]) for i, _ in g) for _, g in itertools.groupby(enumerate(keys), key=lambda t: t[1])]
        want_abs = [math.fsum(abs(float(fv[i])) for i, _ in g)
                    for _, g in itertools.groupby(enumerate(keys), key=lambda t: t[1])]
        if not np.array_equal(ukf, uk) or agf.tolist() != want or abf.tolist() != want_abs:
            fail(f"reduce by key fp32 n={n}")
        ur, ln = lib.run_length_encode(keys.view(np.uint32))
        if ur.tolist() != [int(k) for k, _ in groups] or ln.tolist() != [len(v) for _, v in groups]:
            fail(f"run-length encode n={n}")
        if not np.array_equal(ln, np.diff(np.concatenate([starts, [n]]))):
            fail(f"run-length encode (numpy diff) n={n}")
    # closed forms: one run, all distinct, and keys compared as bit patterns
    k1 = np.full(50, 7, dtype=np.uint32)
    v = np.arange(50, dtype=np.uint32)
    if lib.reduce_by_key(k1, v)[1].tolist() != [sum(range(50))] or lib.run_length_encode(k1)[1].tolist() != [50]:
        fail("one run")
    kd = np.arange(50, dtype=np.uint32)
    if not np.array_equal(lib.reduce_by_key(kd, v)[1], v) or not np.all(lib.run_length_encode(kd)[1] == 1):
        fail("all distinct")
    zf = np.array([0.0, -0.0, -0.0, 0.0], dtype=np.float32).view(np.uint32)
    if lib.run_length_encode(zf)[1].tolist() != [1, 2, 1]:
        fail("keys are bit patterns")
    sel_all, c_all = lib.partition_flagged(v, np.ones(50, np.int32))
    sel_none, c_none = lib.partition_flagged(v, np.zeros(50, np.int32))
    if c_all != 50 or not np.array_equal(sel_all, v) or c_none != 0 or not np.array_equal(sel_none, v[::-1]):
        fail("partition all / none")


def _generic_checks(lib, fail):
    for f in (_minmax_checks, _pair_sum_checks, _affine_checks, _segsum_checks, _compaction_family_checks):
        try:
            f(lib, fail)
        except (IndexError, ValueError, RuntimeError) as e:   # a broken oracle may produce nonsense shapes
            fail(f"{f.__name__}: {e}")


def pin_failures(lib) -> list:
    """Run every pin against an oracle library; return the names that fail."""
    failures = []
    fail = failures.append
    for fname in ("pmpp_11_3_hierarchical_example.txt", "pmpp_11_2_coarsened_example.txt"):
        _golden_checks(lib, fname, fail)
    _fig6_checks(lib, fail)
    _closed_form_checks(lib, fail)
    _fp64_witness_checks(lib, fail)
    _brute_force_checks(lib, fail)
    _select_checks(lib, fail)
    _generic_checks(lib, fail)
    return failures


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle.OracleLib(oracle.LIBRARY)


def test_golden_examples(lib):
    failures = []
    for fname in ("pmpp_11_3_hierarchical_example.txt", "pmpp_11_2_coarsened_example.txt"):
        _golden_checks(lib, fname, failures.append)
    _fig6_checks(lib, failures.append)
    assert failures == []


def test_closed_forms(lib):
    failures = []
    _closed_form_checks(lib, failures.append)
    assert failures == []


def test_fp64_accumulation(lib):
    failures = []
    _fp64_witness_checks(lib, failures.append)
    assert failures == []


def test_brute_force(lib):
    failures = []
    _brute_force_checks(lib, failures.append)
    assert failures == []


def test_select_flagged(lib):
    failures = []
    _select_checks(lib, failures.append)
    assert failures == []
    # numpy's boolean indexing as an independent routine, on an input like the 2^30 - 12345 flags workload
    x = np.arange(1 << 20, dtype=np.uint32)
    flags = wl.generate("flags_half", 1 << 20, 4)
    assert np.array_equal(lib.select_flagged(x, flags), x[flags != 0])
    # in place
    y = x.copy()
    out = lib._lib.oracle_select_flagged(y.ctypes.data, flags.ctypes.data, y.size, y.ctypes.data)
    assert np.array_equal(y[:out], x[flags != 0])


@pytest.mark.parametrize("checks", [_minmax_checks, _pair_sum_checks, _affine_checks, _segsum_checks,
                                    _compaction_family_checks],
                         ids=["minmax", "pair_sum", "affine", "segsum", "compaction_family"])
def test_generic_operators(lib, checks):
    failures = []
    checks(lib, failures.append)
    assert failures == []


def test_empty_and_in_place(lib):
    e = np.zeros(0, dtype=np.int32)
    assert lib.scan_u32(e).size == 0
    assert lib.scan_f32(np.zeros(0, dtype=np.float32))[0].size == 0
    x = wl.random_input("uint32", 5000, 9)
    want = lib.scan_u32(x.copy(), exclusive=True)
    lib.scan_u32(x, exclusive=True, out=x)
    assert np.array_equal(x, want)


@pytest.mark.parametrize("name", ["i32_4096_incl", "f32_2p20_incl", "u32_2p26_incl"])
def test_numpy_cumsum_on_workloads(lib, name):
    w = wl.WORKLOADS[name]
    x = wl.generate_workload(w)
    if w.dtype == "float32":
        y, s = lib.scan_f32(x, exclusive=w.exclusive)
        c = np.cumsum(x.astype(np.float64))
        want = np.concatenate([[0.0], c[:-1]]) if w.exclusive else c
        assert np.array_equal(y, want)          # both are sequential fp64 sums
        assert np.array_equal(s, np.cumsum(np.abs(x.astype(np.float64))))
    else:
        y = lib.scan_u32(x, exclusive=w.exclusive)
        c = np.cumsum(x.astype(np.int64)) & M32
        want = np.concatenate([[0], c[:-1]]) if w.exclusive else c
        assert np.array_equal(y.view(np.uint32).astype(np.int64), want)


@pytest.mark.parametrize("dtype", ["int32", "uint32", "float32"])
def test_exclusive_is_shifted_inclusive(lib, dtype):
    x = wl.random_input(dtype, 100_003, 5)
    if dtype == "float32":
        inc, _ = lib.scan_f32(x)
        exc, _ = lib.scan_f32(x, exclusive=True)
        assert exc[0] == 0.0
        assert np.array_equal(exc[1:], inc[:-1])
    else:
        inc = lib.scan_u32(x)
        exc = lib.scan_u32(x, exclusive=True)
        assert exc[0] == 0
        assert np.array_equal(exc[1:], inc[:-1])
        # the last inclusive value is the total modulo 2^32
        assert int(inc[-1]) & M32 == int(np.sum(x.astype(np.int64))) & M32


# Plausible mistakes planted in copies of the oracle's C source: (label, text
# to find, replacement). Each mutant must fail at least one pin.
MUTANTS = [
    ("inclusive stores before adding",
     "running += xi;\n            y[i] = running;", "y[i] = running;\n            running += xi;"),
    ("exclusive stores after adding",
     "y[i] = running;\n            running += xi;", "running += xi;\n            y[i] = running;"),
    ("fp32 accumulator", "double running = 0.0;", "float running = 0.0f;"),
    ("running |x| without abs", "running_abs += fabs(xi);", "running_abs += xi;"),
    ("running |x| excludes element i",
     "running_abs += fabs(xi);\n            sabs[i] = running_abs;",
     "sabs[i] = running_abs;\n            running_abs += fabs(xi);"),
    ("loop skips element 0", "for (size_t i = 0; i < n; ++i) {", "for (size_t i = 1; i < n; ++i) {"),
    ("wrong sign", "running += xi;", "running -= xi;"),
    ("reversed index", "uint32_t xi = x[i];", "uint32_t xi = x[n - 1 - i];"),
    ("stale element", "double xi = (double)x[i];", "double xi = (double)x[i > 0 ? i - 1 : 0];"),
    ("select tests sign", "if (flags[i] != 0) {", "if (flags[i] > 0) {"),
    ("select drops the last element", "for (size_t i = 0; i < n; ++i) {\n        if (flags[i]", "for (size_t i = 0; i + 1 < n; ++i) {\n        if (flags[i]"),
    ("select writes past the slot", "out[count] = x[i];\n            ++count;", "++count;\n            out[count - 1 + (count > 1)] = x[i];"),
    ("max compares unsigned as signed", "else take = is_max ? (xi > running) : (xi < running);",
     "else take = is_max ? ((int32_t)xi > (int32_t)running) : (xi < running);"),
    ("min identity", "else running = is_signed ? 0x7fffffffu : 0xffffffffu;",
     "else running = is_signed ? 0x7fffffffu : 0x7fffffffu;"),
    ("pair sum drops the fp part", "        rf += xf;\n", "        rf = xf;\n"),
    ("affine composed in the wrong order", "B = a * B + b;", "B = B + b * A;"),
    ("affine uses the updated A", "        A = a * A;\n        B = a * B + b;", "        A = a * A;\n        B = A * B + b;"),
    ("segsum does not restart", "if (f != 0u) V = v;", "if (f != 0u) V += v;"),
    ("segsum flag not accumulated", "F |= f;", "F = f;"),
    ("segsum fp restarts before the head", "            V = v;\n            S = fabs(v);",
     "            V = 0.0;\n            S = 0.0;"),
    ("partition moves the wrong rejected element", "out[n - 1 - rej] = x[i];", "out[n - 1 - rej] = x[n - 1 - i];"),
    ("runs start only on increasing keys", "if (i == 0 || keys[i] != keys[i - 1]) {",
     "if (i == 0 || keys[i] > keys[i - 1]) {"),
    ("run aggregate keeps only the last value", "aggs[runs - 1] += vals[i];", "aggs[runs - 1] = vals[i];"),
    ("run |value| sum without abs", "abs_sums[runs - 1] += fabs((double)vals[i]);",
     "abs_sums[runs - 1] += (double)vals[i];"),
    ("run length counts one", "lengths[runs - 1] += 1u;", "lengths[runs - 1] = 1u;"),
]


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistakes(tmp_path, label, old, new):
    with open(oracle.SOURCE, encoding="utf-8") as f:
        src = f.read()
    assert old in src, f"mutant '{label}' no longer matches the oracle source"
    mutated = src.replace(old, new, 1)
    csrc = os.path.join(tmp_path, "mutant.c")
    with open(csrc, "w", encoding="utf-8") as f:
        f.write(mutated)
    so = oracle.compile_source(csrc, os.path.join(tmp_path, "libmutant.so"))
    mutant = oracle.OracleLib(so)
    assert pin_failures(mutant), f"no pin catches the planted mistake: {label}"


def test_real_oracle_passes_every_pin(lib):
    assert pin_failures(lib) == []

"""GPU parity of the generic-operator scans (dws_scan_op) against the CPU
oracle, element by element on the same seeded inputs.

Bar: integer results (max/min, uint32 pairs, the int32 and flag parts of the
{int32, fp32} pairs, affine maps, uint32 segmented sums) bit-exact; fp32 parts
within 1e-4 * (sum of |value| over the elements the oracle combined) + 1e-6.
"""
import numpy as np
import pytest

import device_wide_prefix_amd as dws
import oracle
import scan_workloads as wl
from gpu_util import ATOL, RTOL, note

pytestmark = pytest.mark.gpu

# name: (op, dtype, input kind, element words)
COMBOS = {
    "max_i32": (dws.OP_MAX, dws.INT32, "i32_full", 1),
    "max_u32": (dws.OP_MAX, dws.UINT32, "u32_full", 1),
    "min_i32": (dws.OP_MIN, dws.INT32, "i32_full", 1),
    "min_u32": (dws.OP_MIN, dws.UINT32, "u32_full", 1),
    "sum_pair_i32_f32": (dws.OP_SUM, dws.PAIR_I32_F32, "pair_i32_f32", 2),
    "sum_pair_u32": (dws.OP_SUM, dws.PAIR_U32, "pair_u32", 2),
    "affine_u32": (dws.OP_AFFINE, dws.PAIR_U32, "affine_u32", 2),
    "segsum_u32": (dws.OP_SEGMENTED_SUM, dws.PAIR_U32, "segsum_u32", 2),
    "segsum_i32_f32": (dws.OP_SEGMENTED_SUM, dws.PAIR_I32_F32, "segsum_i32_f32", 2),
}

# around the tile sizes of every shape (small 4096 / 2048, medium 16384 / 8192
# from 2^20, large 65536 / 32768 from 2^24, elements of one / two words) and
# the switch to non-temporal loads at 2^25
SIZES = [1, 2, 63, 64, 65, 2047, 2048, 2049, 4095, 4096, 4097, 3 * 4096 + 5, 100_003,
         (1 << 20) - 1, (1 << 20) + 7, 3 * (1 << 20) + 5, (1 << 24) - 3, (1 << 24) + 5, (1 << 25) + 9,
         (1 << 26) + 3]


def expected(name, x, exclusive):
    """The oracle's result: (exact part as uint32 bits, fp64 part or None,
    |value| sums or None)."""
    if name.startswith("max") or name.startswith("min"):
        return oracle.scan_minmax(x, name.startswith("max"), exclusive).view(np.uint32), None, None
    if name == "sum_pair_u32":
        return oracle.scan_pair_sum_u32(x, exclusive), None, None
    if name == "affine_u32":
        return oracle.scan_affine_u32(x, exclusive), None, None
    if name == "segsum_u32":
        return oracle.scan_segsum_u32(x, exclusive), None, None
    if name == "sum_pair_i32_f32":
        yi, yf, sa = oracle.scan_pair_sum_i32_f32(x, exclusive)
        return yi.view(np.uint32), yf, sa
    if name == "segsum_i32_f32":
        yi, yf, sa = oracle.scan_segsum_i32_f32(x, exclusive)
        return yi.view(np.uint32), yf, sa
    raise KeyError(name)


def run_op(name, x, exclusive, in_place=False, offset_elems=0, seed=None):
    """Upload x, run dws_scan_op (dws_scan_op_seeded with ``seed``, one
    element of x's kind) through the C ABI, return the result as uint32 bits
    with x's shape."""
    import torch
    op, dtype, _, words = COMBOS[name]
    n = x.shape[0]
    flat = np.ascontiguousarray(x).view(np.uint32).reshape(-1).view(np.int32)
    pad = offset_elems * words
    store = torch.empty(flat.size + pad, dtype=torch.int32, device="cuda")
    xd = store[pad:]
    xd.copy_(torch.from_numpy(flat))
    if in_place:
        out = xd
    else:
        ostore = torch.empty(flat.size + pad, dtype=torch.int32, device="cuda")
        out = ostore[pad:]
    stream = torch.cuda.current_stream().cuda_stream
    if seed is None:
        st = dws.scan_op_ptr(xd.data_ptr(), out.data_ptr(), n, dtype, op, exclusive, stream)
    else:
        sd = torch.from_numpy(np.ascontiguousarray(seed).view(np.uint32).reshape(-1).view(np.int32)).to("cuda")
        st = dws.scan_op_seeded_ptr(xd.data_ptr(), out.data_ptr(), n, dtype, op, exclusive, sd.data_ptr(), stream)
    assert st == dws.OK, dws.status_string(st)
    return out.cpu().numpy().view(np.uint32).reshape(x.shape)


def check_op(name, x, y, exclusive, label, ref=None):
    """y against the oracle's scan of x, or against ``ref`` (the same triple
    expected() returns) when given."""
    exact, yf, sabs = expected(name, x, exclusive) if ref is None else ref
    if yf is None:
        if not np.array_equal(y, exact):
            bad = np.flatnonzero(np.any((y != exact).reshape(y.shape[0], -1), axis=1))
            i = int(bad[0])
            raise AssertionError(f"{label}: mismatch at element {i}/{y.shape[0]} ({bad.size} elements): "
                                 f"gpu {y[i]} oracle {exact[i]}")
        return
    # {int32 or flag, fp32}: first word exact, second within the bar
    if not np.array_equal(y[:, 0], exact):
        i = int(np.flatnonzero(y[:, 0] != exact)[0])
        raise AssertionError(f"{label}: integer part mismatch at {i}: gpu {y[i, 0]} oracle {exact[i]}")
    g = y[:, 1].copy().view(np.float32).astype(np.float64)
    err = np.abs(g - yf)
    bound = RTOL * sabs + ATOL
    if not np.all(err <= bound):
        i = int(np.flatnonzero(err > bound)[0])
        raise AssertionError(f"{label}: fp32 part at {i}: gpu {g[i]!r} oracle {yf[i]!r} bound {bound[i]:.3g}")


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("name", list(COMBOS))
def test_op_sizes(gpu, name, exclusive):
    kind = COMBOS[name][2]
    for n in SIZES:
        note(f"op={name} excl={exclusive} n={n}")
        x = wl.op_input(kind, n, seed=n + 17)
        y = run_op(name, x, exclusive)
        check_op(name, x, y, exclusive, f"{name} n={n}")


@pytest.mark.parametrize("name", list(COMBOS))
def test_op_in_place_and_unaligned(gpu, name):
    kind = COMBOS[name][2]
    for n in (5, 3 * 4096 + 1, (1 << 20) + 3, (1 << 24) + 1):
        for exclusive in (False, True):
            x = wl.op_input(kind, n, seed=2 * n + exclusive)
            note(f"op={name} in place excl={exclusive} n={n}")
            check_op(name, x, run_op(name, x, exclusive, in_place=True), exclusive, f"{name} in place n={n}")
            # one element off 16-byte alignment: the one-element-per-access kernel
            note(f"op={name} unaligned excl={exclusive} n={n}")
            check_op(name, x, run_op(name, x, exclusive, offset_elems=1), exclusive, f"{name} unaligned n={n}")
            check_op(name, x, run_op(name, x, exclusive, in_place=True, offset_elems=1), exclusive,
                     f"{name} unaligned in place n={n}")


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("name", list(COMBOS))
def test_op_seeded(gpu, name, exclusive):
    """dws_scan_op_seeded against the oracle's scan of the sequence seed,
    x[0], ..., x[n-1] without its first (inclusive) or last (exclusive)
    element: the seed is the earlier operand of every combine it enters."""
    kind = COMBOS[name][2]
    for i, n in enumerate((1, 5, 3 * 4096 + 5, (1 << 20) + 7, (1 << 25) + 9)):
        x = wl.op_input(kind, n, seed=3 * n + 1)
        seed = wl.op_input(kind, 1, seed=1000 + i)
        if name.startswith("segsum") and i % 2 == 1:
            seed[0, 0] = 0       # a seed without a head: x[0] continues its segment
        in_place = i % 2 == 0
        note(f"op={name} seeded excl={exclusive} n={n} in_place={in_place}")
        y = run_op(name, x, exclusive, in_place=in_place, seed=seed)
        z = np.concatenate([seed, x])
        exact, yf, sabs = expected(name, z, False)
        part = slice(0, -1) if exclusive else slice(1, None)
        ref = (exact[part], None if yf is None else yf[part], None if sabs is None else sabs[part])
        check_op(name, x, y, exclusive, f"{name} seeded n={n}", ref=ref)


def _upload(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.uint32).reshape(-1).view(np.int32)).to("cuda")


def check_total(name, x, got, label):
    """got (one element as uint32 words) against the last element of the
    oracle's inclusive scan of x, or the identity when x is empty."""
    exact, yf, sabs = expected(name, x, False)
    words = COMBOS[name][3]
    got = got.reshape(-1)
    if x.shape[0] == 0:
        return
    if yf is None:
        want = np.asarray(exact[-1]).reshape(-1).astype(np.uint32)
        assert np.array_equal(got[:words], want), f"{label}: gpu {got} oracle {want}"
        return
    assert got[0] == exact[-1], f"{label}: integer part gpu {got[0]} oracle {exact[-1]}"
    g = float(got[1:2].view(np.float32)[0])
    assert abs(g - yf[-1]) <= RTOL * sabs[-1] + ATOL, f"{label}: fp32 part gpu {g!r} oracle {yf[-1]!r}"


IDENTITY = {"max_i32": [0x80000000], "max_u32": [0], "min_i32": [0x7FFFFFFF], "min_u32": [0xFFFFFFFF],
            "sum_pair_i32_f32": [0, 0], "sum_pair_u32": [0, 0], "affine_u32": [1, 0], "segsum_u32": [0, 0],
            "segsum_i32_f32": [0, 0]}


@pytest.mark.parametrize("name", list(COMBOS))
def test_reduce_op(gpu, name):
    """dws_reduce_op at sizes around every tile and group boundary, aligned
    and not, against the oracle; the empty input gives the identity, and fp32
    parts repeat bit for bit."""
    import torch
    op, dtype, kind, words = COMBOS[name]
    for off in (0, 1):
        for n in (0, 1, 5, 4097, 8192, 8193, 16385, 1_000_003, 1024 * 8192 + 3, (1 << 25) + 9):
            if n == 0 and off:
                continue
            note(f"reduce_op={name} n={n} offset={off}")
            x = wl.op_input(kind, n, seed=5 * n + off) if n else wl.op_input(kind, 1, seed=1)[:0]
            flat = np.ascontiguousarray(x).view(np.uint32).reshape(-1).view(np.int32)
            store = torch.empty(flat.size + off * words + 1, dtype=torch.int32, device="cuda")
            xd = store[off * words:off * words + flat.size]
            if n:
                xd.copy_(torch.from_numpy(flat))
            total = torch.full((words,), 12345, dtype=torch.int32, device="cuda")
            stream = torch.cuda.current_stream().cuda_stream
            st = dws.reduce_op_ptr(xd.data_ptr(), n, dtype, op, total.data_ptr(), stream)
            assert st == dws.OK, dws.status_string(st)
            first = total.cpu().numpy().view(np.uint32).copy()
            if n == 0:
                assert first.tolist() == IDENTITY[name], first
                continue
            check_total(name, x, first, f"{name} n={n} offset={off}")
            st = dws.reduce_op_ptr(xd.data_ptr(), n, dtype, op, total.data_ptr(), stream)
            assert st == dws.OK
            assert np.array_equal(total.cpu().numpy().view(np.uint32), first), "not repeatable"


@pytest.mark.parametrize("name", list(COMBOS))
def test_sharded_op_scan(gpu, name):
    """A generic-operator scan split into uneven shards (one empty, one
    shorter than a tile): each shard's total (dws_reduce_op), the exclusive
    scan of the totals (dws_scan_op), each shard scanned seeded with its
    offset (dws_scan_op_seeded), reassembled and compared with the oracle's
    scan of the whole array. The operators that are not commutative depend on
    every shard keeping its place."""
    import torch
    op, dtype, kind, words = COMBOS[name]
    n = (1 << 22) + 33
    cuts = [0, 3, 700_001, 700_001, (1 << 21) + 5, n]
    x = wl.op_input(kind, n, seed=77)
    xd = _upload(x)
    stream = torch.cuda.current_stream().cuda_stream
    g = len(cuts) - 1
    totals = torch.empty(g * words, dtype=torch.int32, device="cuda")
    for i in range(g):
        a, b = cuts[i], cuts[i + 1]
        st = dws.reduce_op_ptr(xd[a * words:].data_ptr(), b - a, dtype, op, totals[i * words:].data_ptr(), stream)
        assert st == dws.OK, dws.status_string(st)
    offsets = torch.empty_like(totals)
    assert dws.scan_op_ptr(totals.data_ptr(), offsets.data_ptr(), g, dtype, op, True, stream) == dws.OK
    for exclusive in (False, True):
        note(f"sharded op={name} excl={exclusive} shards={g}")
        out = torch.empty_like(xd)
        for i in range(g):
            a, b = cuts[i], cuts[i + 1]
            if b > a:
                st = dws.scan_op_seeded_ptr(xd[a * words:].data_ptr(), out[a * words:].data_ptr(), b - a, dtype, op,
                                            exclusive, offsets[i * words:].data_ptr(), stream)
                assert st == dws.OK, dws.status_string(st)
        y = out.cpu().numpy().view(np.uint32).reshape(x.shape)
        check_op(name, x, y, exclusive, f"{name} sharded")


def test_sharded_op_scan_graph_replays(gpu):
    """The operator steps of a split scan (affine maps: not commutative)
    captured in one graph and replayed with new inputs and eager launches on
    the same workspace between replays; every replay is checked."""
    import torch
    op, dtype, kind, words = COMBOS["affine_u32"]
    n = (1 << 21) + 7
    cuts = [0, 500_001, (1 << 20) + 3, n]
    g = len(cuts) - 1
    s = torch.cuda.Stream()
    xd = torch.empty(n * words, dtype=torch.int32, device="cuda")
    out = torch.empty_like(xd)
    totals = torch.empty(g * words, dtype=torch.int32, device="cuda")
    offsets = torch.empty_like(totals)
    dws.reserve(n, stream=s.cuda_stream)

    def steps():
        st = s.cuda_stream
        for i in range(g):
            a, b = cuts[i], cuts[i + 1]
            assert dws.reduce_op_ptr(xd[a * words:].data_ptr(), b - a, dtype, op, totals[i * words:].data_ptr(),
                                     st) == dws.OK
        assert dws.scan_op_ptr(totals.data_ptr(), offsets.data_ptr(), g, dtype, op, True, st) == dws.OK
        for i in range(g):
            a, b = cuts[i], cuts[i + 1]
            assert dws.scan_op_seeded_ptr(xd[a * words:].data_ptr(), out[a * words:].data_ptr(), b - a, dtype, op,
                                          False, offsets[i * words:].data_ptr(), st) == dws.OK

    with torch.cuda.stream(s):          # warm-up outside the capture
        steps()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        steps()
    for rep in range(3):
        note(f"sharded affine graph replay rep={rep}")
        x = wl.op_input(kind, n, seed=500 + rep)
        xd.copy_(_upload(x))
        with torch.cuda.stream(s):        # eager launches on the workspace between replays
            dws.reduce_op(xd, op, dtype)
            dws.scan_op(xd, op, dtype)
        s.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check_op("affine_u32", x, out.cpu().numpy().view(np.uint32).reshape(x.shape), False, f"replay {rep}")


def test_segsum_head_densities(gpu):
    # no heads (one long segment), every element a head, and sparse heads
    # whose segments span many tiles
    for density in (0.0, 1.0, 1e-6):
        for name in ("segsum_u32", "segsum_i32_f32"):
            n = (1 << 22) + 3
            note(f"segsum density={density} {name}")
            x = wl.op_input(COMBOS[name][2], n, seed=5, head_density=density)
            for exclusive in (False, True):
                check_op(name, x, run_op(name, x, exclusive), exclusive, f"{name} density {density}")


def test_affine_reduces_to_sum_and_recurrence(gpu):
    # a = 1 everywhere: the b part is the + scan of b; and the result drives
    # the recurrence v_i = a_i v_{i-1} + b_i from a start value
    n = (1 << 21) + 11
    x = wl.op_input("affine_u32", n, seed=8)
    ones = x.copy()
    ones[:, 0] = 1
    note("affine a=1")
    y = run_op("affine_u32", ones, False)
    assert np.all(y[:, 0] == 1)
    assert np.array_equal(y[:, 1], (np.cumsum(ones[:, 1].astype(np.uint64)) & 0xFFFFFFFF).astype(np.uint32))
    note("affine recurrence")
    y = run_op("affine_u32", x, False)
    s = 12345
    v = s
    for i in range(0, 5000):
        v = (int(x[i, 0]) * v + int(x[i, 1])) & 0xFFFFFFFF
        assert v == (int(y[i, 0]) * s + int(y[i, 1])) & 0xFFFFFFFF, i


def test_op_binding_and_full_size(gpu):
    # through the Python binding, at 2^27 pairs (1 GiB each way) for the
    # {int32, fp32} pair sum, and 2^28 int32 for max
    import torch
    n = 1 << 27
    note(f"pair sum binding n={n}")
    x = wl.op_input("pair_i32_f32", n, seed=3)
    xd = torch.from_numpy(x.view(np.int32)).cuda()
    y = dws.scan_op(xd, dws.OP_SUM, dws.PAIR_I32_F32).cpu().numpy().view(np.uint32)
    check_op("sum_pair_i32_f32", x, y, False, "pair sum 2^27")
    del xd
    n = 1 << 28
    note(f"max binding n={n}")
    x = wl.op_input("i32_full", n, seed=4)
    xd = torch.from_numpy(x).cuda()
    y = dws.scan_op(xd, dws.OP_MAX, exclusive=True).cpu().numpy().view(np.uint32)
    check_op("max_i32", x, y, True, "max 2^28")

"""GPU parity of the per-device pieces of a scan split into contiguous shards:
dws_reduce (a shard's total) and dws_scan_seeded (a shard's scan seeded with
the total of the shards before it), called through the C ABI and compared with
the CPU oracle on the same seeded inputs.

Expected values come from the oracle's plain scans only:
  - the + of x is the last element of the oracle's inclusive scan of x;
  - the scan of x seeded with s is the oracle's inclusive scan of the
    sequence s, x[0], ..., x[n-1] without its first element (inclusive) or its
    last (exclusive).
Bar: 32-bit integers bit-exact (modulo 2^32); fp32 within 1e-4 * (the running
sum of |values|) + 1e-6 of the fp64 oracle, as for the scans.
"""
import numpy as np
import pytest

import device_wide_prefix_amd as dws
import oracle
import scan_workloads as wl
from gpu_util import ATOL, CODE, RTOL, check_chunked, from_device, note, to_device

pytestmark = pytest.mark.gpu

DTYPES = ["int32", "uint32", "float32"]
RT = 16384          # elements per reduction tile
GROUPS = 1024       # most workgroups of one reduction


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _scalar_on_device(v, dtype):
    """One element of `dtype` in its own GPU allocation."""
    return to_device(np.array([v], dtype=np.dtype(dtype)))[1]


def _reduce(xd, n, dtype, total):
    st = dws.reduce_ptr(xd.data_ptr(), n, CODE[dtype], total.data_ptr(), _stream())
    assert st == dws.OK, dws.status_string(st)


def _seeded(xd, out, n, dtype, exclusive, seed_ptr):
    st = dws.scan_seeded_ptr(xd.data_ptr(), out.data_ptr(), n, CODE[dtype], exclusive, seed_ptr, _stream())
    assert st == dws.OK, dws.status_string(st)


def _check_total(x, got, dtype, label):
    """got (one element read back) against the oracle's + of x."""
    if x.size == 0:
        assert got.view(np.uint32)[0] == 0, f"{label}: empty input gave {got[0]!r}"
        return
    if dtype == "float32":
        ref, sabs = oracle.scan_f32(x, exclusive=False)
        err = abs(float(got[0]) - float(ref[-1]))
        bound = RTOL * float(sabs[-1]) + ATOL
        assert err <= bound, f"{label}: gpu {got[0]!r} oracle {ref[-1]!r} bound {bound:.3g}"
    else:
        ref = oracle.scan_u32(x, exclusive=False)
        assert int(got.view(np.uint32)[0]) == int(ref.view(np.uint32)[-1]), \
            f"{label}: gpu {int(got.view(np.uint32)[0])} oracle {int(ref.view(np.uint32)[-1])}"


def _check_seeded(x, seed, y, dtype, exclusive, label):
    """y against the oracle's inclusive scan of (seed, x[0], ..., x[n-1])."""
    z = np.concatenate([np.array([seed], dtype=x.dtype), x])
    if dtype == "float32":
        ref, sabs = oracle.scan_f32(z, exclusive=False)
        part = slice(0, -1) if exclusive else slice(1, None)
        ref, sabs = ref[part], sabs[part]
        err = np.abs(y.astype(np.float64) - ref)
        ok = err <= RTOL * sabs + ATOL
        if not ok.all():
            i = int(np.flatnonzero(~ok)[0])
            raise AssertionError(f"{label}: fp32 mismatch at {i}/{x.size}: gpu {y[i]!r} oracle {ref[i]!r}")
        return
    ref = oracle.scan_u32(z, exclusive=False)
    ref = ref[:-1] if exclusive else ref[1:]
    yb, rb = y.view(np.uint32), ref.view(np.uint32)
    if not np.array_equal(yb, rb):
        i = int(np.flatnonzero(yb != rb)[0])
        raise AssertionError(f"{label}: int mismatch at {i}/{x.size}: gpu {int(yb[i])} oracle {int(rb[i])}")


# sizes around the wave, the reduction tile, the switch from one tile per
# workgroup to two (GROUPS tiles) and non-temporal loads (2^23)
REDUCE_SIZES = [0, 1, 2, 63, 64, 65, 1023, RT - 1, RT, RT + 1, 3 * RT + 17, 1_000_003,
                GROUPS * RT - 1, GROUPS * RT, GROUPS * RT + 1, (1 << 25) + 7, 5 * GROUPS * RT + RT // 2 + 3]


@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_sizes(gpu, dtype):
    import torch
    for n in REDUCE_SIZES:
        note(f"reduce dtype={dtype} n={n}")
        x = wl.random_input(dtype, n, seed=31 + n)
        _, xd = to_device(x) if n else (None, torch.empty(0, dtype=torch.int32, device="cuda"))
        total = _scalar_on_device(12345, dtype)   # overwritten, also for n == 0
        _reduce(xd, n, dtype, total)
        _check_total(x, from_device(total, dtype), dtype, f"reduce n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_unaligned_and_repeated(gpu, dtype):
    """4-byte but not 16-byte aligned inputs take the dword-load kernel; calls
    in a row with different workgroup counts on one stream all agree with the
    oracle, so no call reads a partial left by the one before; fp32 results
    repeat bit for bit."""
    import torch
    sizes = [(1 << 22) + 5, 7, GROUPS * RT + 3, 100_001, (1 << 25) + 1]
    xs = {n: wl.random_input(dtype, n, seed=57 + n) for n in sizes}
    for off in (0, 1, 3):
        for n in sizes:
            note(f"reduce dtype={dtype} offset={off} n={n}")
            _, xd = to_device(xs[n], extra_front=off)
            total = _scalar_on_device(0, dtype)
            _reduce(xd, n, dtype, total)
            first = from_device(total, dtype).copy()
            _check_total(xs[n], first, dtype, f"reduce offset {off} n={n}")
            _reduce(xd, n, dtype, total)
            again = from_device(total, dtype)
            assert first.view(np.uint32)[0] == again.view(np.uint32)[0], f"offset {off} n={n}: not repeatable"
    torch.cuda.synchronize()


def test_reduce_binding_and_streams(gpu):
    """The tensor binding, and two streams (two workspaces) reducing at once."""
    import torch
    x1 = wl.random_input("float32", (1 << 23) + 9, seed=5)
    x2 = wl.random_input("int32", (1 << 22) + 1, seed=6)
    _, d1 = to_device(x1)
    _, d2 = to_device(x2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = dws.reduce(d1)
        with torch.cuda.stream(s2):
            b = dws.reduce(d2)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        _check_total(x1, from_device(a, "float32"), "float32", "stream 1")
        _check_total(x2, from_device(b, "int32"), "int32", "stream 2")
    with pytest.raises(ValueError):
        dws.reduce(d1, out=torch.empty(2, dtype=torch.float32, device="cuda"))


SEEDED_SIZES = [1, 5, 4095, 4097, 3 * 4096 + 5, (1 << 20) + 3, (1 << 23) + 1, (1 << 24) + 77]
SEEDS = {"int32": [0, -123456, 2**31 - 5], "uint32": [0, 4_000_000_000], "float32": [0.0, 1234.5, -7.25]}


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_scan_seeded(gpu, dtype, exclusive):
    import torch
    for i, n in enumerate(SEEDED_SIZES):
        seed = SEEDS[dtype][i % len(SEEDS[dtype])]
        in_place = i % 2 == 1
        note(f"seeded dtype={dtype} excl={exclusive} n={n} seed={seed} in_place={in_place}")
        x = wl.random_input(dtype, n, seed=71 + n)
        _, xd = to_device(x)
        out = xd if in_place else torch.empty_like(xd)
        sd = _scalar_on_device(seed, dtype)
        _seeded(xd, out, n, dtype, exclusive, sd.data_ptr())
        _check_seeded(x, x.dtype.type(seed), from_device(out, dtype), dtype, exclusive, f"n={n}")


@pytest.mark.parametrize("dtype", ["int32", "float32"])
def test_scan_seeded_edge_cases(gpu, dtype):
    """A seed read from the input array itself (out of place), unaligned
    pointers, the binding, and a seed of 0 matching the unseeded scan bit for
    bit (integers) or to the bar (fp32)."""
    import torch
    n = (1 << 21) + 33
    x = wl.random_input(dtype, n, seed=3)
    _, xd = to_device(x)
    out = torch.empty_like(xd)
    k = n // 2
    note(f"seeded dtype={dtype}: seed taken from the input, element {k}")
    _seeded(xd, out, n, dtype, True, xd[k:].data_ptr())
    _check_seeded(x, x[k], from_device(out, dtype), dtype, True, "seed inside the input")

    for off in (1, 2):
        note(f"seeded dtype={dtype}: offset {off}")
        _, xo = to_device(x, extra_front=off)
        ostore = torch.empty(n + off, dtype=xo.dtype, device="cuda")
        sd = _scalar_on_device(77, dtype)
        _seeded(xo, ostore[off:], n, dtype, False, sd.data_ptr())
        _check_seeded(x, x.dtype.type(77), from_device(ostore[off:], dtype), dtype, False, f"offset {off}")

    note(f"seeded dtype={dtype}: binding, seed 0")
    zero = torch.zeros(1, dtype=xd.dtype, device="cuda")
    y0 = dws.scan_seeded(xd, zero, exclusive=False)
    y1 = dws.scan_inclusive(xd)
    torch.cuda.synchronize()
    if dtype == "int32":
        assert torch.equal(y0, y1)
    _check_seeded(x, x.dtype.type(0), from_device(y0, dtype), dtype, False, "binding")
    with pytest.raises(ValueError):
        dws.scan_seeded(xd, torch.zeros(2, dtype=xd.dtype, device="cuda"))


def _sharded_scan(xd, out, n, dtype, exclusive, shards):
    """The per-device steps of a split scan, all on this GPU and stream: every
    shard's total (dws_reduce), the exclusive scan of the totals (the step the
    devices would share), then every shard's scan seeded with its offset."""
    import torch
    bounds = [0] + [int(b) for b in shards] + [n]
    g = len(bounds) - 1
    totals = torch.empty(g, dtype=xd.dtype, device="cuda")
    for i in range(g):
        a, b = bounds[i], bounds[i + 1]
        st = dws.reduce_ptr(xd[a:].data_ptr(), b - a, CODE[dtype], totals[i:].data_ptr(), _stream())
        assert st == dws.OK, dws.status_string(st)
    offsets = torch.empty_like(totals)
    st = dws.scan_exclusive_ptr(totals.data_ptr(), offsets.data_ptr(), g, CODE[dtype], _stream())
    assert st == dws.OK, dws.status_string(st)
    for i in range(g):
        a, b = bounds[i], bounds[i + 1]
        if b > a:
            _seeded(xd[a:], out[a:], b - a, dtype, exclusive, offsets[i:].data_ptr())


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_sharded_scan_matches_the_whole_scan(gpu, dtype, exclusive):
    """Uneven shards (one empty, one shorter than a tile, ragged ends) put
    back together give the oracle's scan of the whole array."""
    import torch
    n = (1 << 24) + 12345
    cuts = [[n // 2], [5, 70_000, 70_000, (1 << 23) + 3], sorted({(n * k) // 8 + (k * 977) % 4096 for k in range(1, 8)})]
    x = wl.random_input(dtype, n, seed=909)
    _, xd = to_device(x)
    for cut in cuts:
        note(f"sharded dtype={dtype} excl={exclusive} n={n} shards={len(cut) + 1}")
        out = torch.empty_like(xd)
        _sharded_scan(xd, out, n, dtype, exclusive, cut)
        torch.cuda.synchronize()
        check_chunked(x, from_device(out, dtype), dtype, exclusive, label=f"{len(cut) + 1} shards")


def test_sharded_headline_scan(gpu):
    """The 2^28-element fp32 exclusive in-place scan split into 8 shards of
    2^25 (each device's share at that size), put back together on one GPU."""
    import torch
    w = wl.WORKLOADS["f32_2p28_excl_inplace"]
    note(f"sharded {w.description}, 8 shards")
    x = wl.generate_workload(w)
    store, xd = to_device(x)
    _sharded_scan(xd, xd, w.n, "float32", True, [k * (w.n // 8) for k in range(1, 8)])
    torch.cuda.synchronize()
    y = from_device(xd, "float32")
    del store, xd
    worst = check_chunked(x, y, "float32", True, label="8 shards")
    note(f"sharded headline scan: parity ok, max fp32 tolerance ratio {worst:.3g}")


def test_sharded_scan_graph_replays(gpu):
    """The per-device steps captured in one graph: every replay reads the
    epoch word the previous launch on the workspace advanced, so it sees only
    its own partials and descriptors. Eager launches on the same workspace run
    between replays, and every replay is checked against the oracle."""
    import torch
    n = (1 << 22) + 7
    cut = [1_000_003, 1_000_003 + (1 << 21)]
    s = torch.cuda.Stream()
    x = torch.empty(n, dtype=torch.int32, device="cuda")
    out = torch.empty_like(x)
    dws.reserve(n, stream=s.cuda_stream)
    with torch.cuda.stream(s):          # warm-up outside the capture
        _sharded_scan(x, out, n, "int32", True, cut)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _sharded_scan(x, out, n, "int32", True, cut)
    for rep in range(4):
        note(f"sharded graph replay rep={rep}")
        data = wl.random_input("int32", n, seed=400 + rep)
        x.copy_(torch.from_numpy(data))
        with torch.cuda.stream(s):        # eager launches on the workspace between replays
            dws.reduce(x)
            dws.scan_inclusive(x, torch.empty_like(x))
        s.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_chunked(data, from_device(out, "int32"), "int32", True, label=f"replay {rep}")


def test_zz_shard_watchdog_never_tripped(gpu):
    assert dws.watchdog_trips() == 0

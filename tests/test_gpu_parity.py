"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle,
element by element on the same seeded inputs.

Bar: 32-bit integers bit-exact (modulo 2^32); fp32 within
1e-4 * sum_{j<=i}|x_j| + 1e-6 of the fp64 oracle. Where several fp32 results
are correct (the order of additions depends on scheduling), the tolerance is the
check; the descriptors' statuses and epochs, which are unique, are compared
exactly.
"""
import numpy as np
import pytest

import device_wide_prefix_amd as dws
import oracle
import scan_workloads as wl
from golden_io import read_golden
from gpu_util import (check, check_chunked, decode_desc, from_device, note, run, to_device)

pytestmark = pytest.mark.gpu

TILE = 4096
DTYPES = ["int32", "uint32", "float32"]


def _roundtrip(x, dtype, exclusive, in_place=False, offset=0, **opts):
    import torch
    store, xd = to_device(x, extra_front=offset)
    if in_place:
        out = xd
    else:
        ostore = torch.empty(x.size + offset, dtype=xd.dtype, device="cuda")
        out = ostore[offset:]
    run(xd, out, x.size, dtype, exclusive, **opts)
    return from_device(out, dtype)


# ---------------------------------------------------------------------------
# wavefront primitives
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["uint32", "float32"])
def test_wave_primitives_lane_layout(gpu, dtype):
    import torch
    note(f"selftest_wave {dtype}")
    waves = 257
    if dtype == "uint32":
        x = wl.generate("u32_full", waves * 64, 11)
    else:
        # small integers: every partial sum is exact in fp32
        x = wl.generate("int_0_9", waves * 64, 11).astype(np.float32) - 4.0
    _, xd = to_device(x)
    incl, shift = dws.selftest_wave(xd)
    incl = from_device(incl, dtype).reshape(waves, 64)
    shift = from_device(shift, dtype).reshape(waves, 64)
    xr = x.reshape(waves, 64)
    if dtype == "uint32":
        want = (np.cumsum(xr.astype(np.uint64), axis=1) & 0xFFFFFFFF).astype(np.uint32)
    else:
        want = np.cumsum(xr.astype(np.float64), axis=1).astype(np.float32)
    assert np.array_equal(incl, want)
    want_shift = np.concatenate([np.zeros((waves, 1), dtype=xr.dtype), xr[:, :-1]], axis=1)
    assert np.array_equal(shift, want_shift)


# ---------------------------------------------------------------------------
# sizes around tile and wave boundaries, all dtypes, both kinds
# ---------------------------------------------------------------------------
# sizes around wave and tile boundaries of every automatic tile size (4096
# below 2^20, 16384 from 2^20, 32768 from 2^23, 65536 from 2^24), around the
# switch to non-temporal loads at 2^23 and around 2^27
M, L, H = 16384, 32768, 65536
EDGE_SIZES = [1, 2, 3, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, TILE - 1, TILE, TILE + 1,
              2 * TILE - 1, 2 * TILE, 2 * TILE + 1, 17 * TILE + 333, 64 * TILE + 17, 255 * TILE + 3,
              (1 << 20) - 1, 1 << 20, (1 << 20) + 1, (1 << 20) + M - 1, 150 * M + 7, (1 << 22) + 1,
              (1 << 23) - 1, 1 << 23, (1 << 23) + 1, (1 << 23) + L + 1, 301 * L - 5,
              (1 << 24) - 1, 1 << 24, (1 << 24) + 1, (1 << 24) + H + 3, 301 * H - 7,
              (1 << 25) - 1, (1 << 25) + 1, (1 << 27) - 1, (1 << 27) + 1]


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_edge_sizes(gpu, dtype, exclusive):
    for n in EDGE_SIZES:
        note(f"edge dtype={dtype} excl={exclusive} n={n}")
        x = wl.random_input(dtype, n, seed=n)
        y = _roundtrip(x, dtype, exclusive)
        check(x, y, dtype, exclusive, label=f"n={n}")


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_in_place(gpu, dtype, exclusive):
    for n in (5, 3 * TILE + 5, 1_000_003):
        note(f"in-place dtype={dtype} excl={exclusive} n={n}")
        x = wl.random_input(dtype, n, seed=7 + n)
        y = _roundtrip(x, dtype, exclusive, in_place=True)
        check(x, y, dtype, exclusive, label=f"in-place n={n}")


@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_unaligned_pointers(gpu, dtype, exclusive):
    # 4-byte aligned but not 16-byte aligned: the scalar-load kernel
    for off in (1, 2, 3):
        for n in (TILE - 1, 5 * TILE + 7, 300_001, (1 << 20) + 9, (1 << 22) + 5, (1 << 24) + 3):
            note(f"unaligned off={off} dtype={dtype} excl={exclusive} n={n}")
            x = wl.random_input(dtype, n, seed=100 * off + n)
            y = _roundtrip(x, dtype, exclusive, offset=off)
            check(x, y, dtype, exclusive, label=f"offset {off} n={n}")
            y = _roundtrip(x, dtype, exclusive, in_place=True, offset=off)
            check(x, y, dtype, exclusive, label=f"in-place offset {off} n={n}")


def test_input_aligned_output_unaligned(gpu):
    import torch
    n = 10 * TILE + 9
    x = wl.random_input("int32", n, seed=3)
    _, xd = to_device(x)
    ostore = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    out = ostore[1:]
    run(xd, out, n, "int32", False)
    check(x, from_device(out, "int32"), "int32", False)


# ---------------------------------------------------------------------------
# comparison variants, tile shapes, descriptor memory order, non-temporal
# ---------------------------------------------------------------------------
VARIANT_SIZES = [1, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, TILE * TILE + 1, (1 << 20) + 3, (1 << 22) + 11,
                 (1 << 24) + 5]


@pytest.mark.parametrize("variant", [dws.REDUCE_THEN_SCAN, dws.CHAINED, dws.SCAN_THEN_PROPAGATE],
                         ids=["rts", "chained", "stp"])
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_comparison_variants(gpu, dtype, exclusive, variant):
    for n in VARIANT_SIZES:
        for in_place in (False, True):
            note(f"variant={variant} dtype={dtype} excl={exclusive} n={n} in_place={in_place}")
            x = wl.random_input(dtype, n, seed=n + variant)
            y = _roundtrip(x, dtype, exclusive, in_place=in_place, variant=variant)
            check(x, y, dtype, exclusive, label=f"variant {variant} n={n}")
    # unaligned
    n = 5 * TILE + 3
    x = wl.random_input(dtype, n, seed=99)
    y = _roundtrip(x, dtype, exclusive, offset=1, variant=variant)
    check(x, y, dtype, exclusive, label=f"variant {variant} unaligned")


def test_tile_shapes(gpu):
    for shape in range(1, dws.num_tile_shapes()):
        t = dws.tile_elems(shape, 1 << 28, True)
        for dtype in ("uint32", "float32"):
            for exclusive in (False, True):
                for n in (t - 1, 5 * t + 3, (1 << 21) + 1):
                    note(f"shape={shape} dtype={dtype} excl={exclusive} n={n}")
                    x = wl.random_input(dtype, n, seed=shape * 1000 + n)
                    y = _roundtrip(x, dtype, exclusive, shape=shape)
                    check(x, y, dtype, exclusive, label=f"shape {shape} n={n}")


@pytest.mark.parametrize("tile_index", [dws.TILE_DRAWN, dws.TILE_DISPATCH], ids=["drawn", "dispatch"])
def test_tile_index_sources(gpu, tile_index):
    # every shape with the tile index from the counter or the workgroup index,
    # and the automatic shape across the size regimes, aligned and not
    for shape in range(dws.num_tile_shapes()):
        t = dws.tile_elems(shape, 1 << 28, True)
        for dtype in ("int32", "float32"):
            for n in (t + 1, 7 * t - 5, 300 * t + 3):
                exclusive = n % 2 == 1
                note(f"tile_index={tile_index} shape={shape} dtype={dtype} n={n}")
                x = wl.random_input(dtype, n, seed=shape * 7 + n)
                y = _roundtrip(x, dtype, exclusive, in_place=exclusive, shape=shape, tile_index=tile_index)
                check(x, y, dtype, exclusive, label=f"tile_index {tile_index} shape {shape} n={n}")
    for n in (TILE + 7, (1 << 20) + 5, (1 << 22) + 3, (1 << 24) + 9):
        note(f"tile_index={tile_index} unaligned n={n}")
        x = wl.random_input("uint32", n, seed=n)
        y = _roundtrip(x, "uint32", False, offset=1, tile_index=tile_index)
        check(x, y, "uint32", False, label=f"tile_index {tile_index} unaligned n={n}")


def test_epochs_across_launch_kinds(gpu):
    # drawn, dispatch-order, chained, compaction and debug launches share one
    # workspace's descriptors; each must see only its own epoch
    import torch
    n = 40 * 65536 + 11
    x = wl.random_input("int32", n, seed=4)
    flags = wl.selection_flags(n, 0.5, seed=5)
    want_sel = oracle.select_flagged(x, flags)
    _, xd = to_device(x)
    _, fd = to_device(flags)
    for rep in range(4):
        for kind in ("drawn", "dispatch", "chained", "select", "debug"):
            note(f"epochs rep={rep} kind={kind}")
            out = torch.empty_like(xd)
            if kind == "select":
                cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
                dws.select_flagged(xd, fd, out=out, count=cnt)
                c = int(cnt.item())
                assert c == want_sel.size and np.array_equal(out[:c].cpu().numpy(), want_sel)
                continue
            if kind == "debug":
                m = 64 * 200 + 5
                dws.scan_debug(xd[:m], out[:m], 64, want_descriptors=False)
                check(x[:m], from_device(out[:m], "int32"), "int32", False, label="debug")
                continue
            opts = {"drawn": dict(tile_index=dws.TILE_DRAWN), "dispatch": dict(tile_index=dws.TILE_DISPATCH),
                    "chained": dict(variant=dws.CHAINED)}[kind]
            run(xd, out, n, "int32", rep % 2 == 1, **opts)
            check(x, from_device(out, "int32"), "int32", rep % 2 == 1, label=f"{kind} rep {rep}")


@pytest.mark.parametrize("opts", [dict(order=dws.ORDER_ACQ_REL), dict(nt=1), dict(nt=2),
                                  dict(variant=dws.CHAINED, order=dws.ORDER_ACQ_REL)],
                         ids=["acq_rel", "nontemporal", "nontemporal_off", "chained_acq_rel"])
def test_order_and_nontemporal(gpu, opts):
    for dtype in DTYPES:
        for exclusive in (False, True):
            for n in (TILE + 1, 40 * TILE, (1 << 20) + 5, (1 << 22) + 3, (1 << 24) + 9):
                note(f"opts={opts} dtype={dtype} excl={exclusive} n={n}")
                x = wl.random_input(dtype, n, seed=n + 5)
                y = _roundtrip(x, dtype, exclusive, in_place=exclusive, **opts)
                check(x, y, dtype, exclusive, label=f"{opts} n={n}")
    x = wl.random_input("float32", 3 * TILE + 1, seed=1)
    y = _roundtrip(x, "float32", True, offset=1, **opts)   # non-temporal is a hint; unaligned ignores it
    check(x, y, "float32", True)


def test_dispatch_nontemporal(gpu):
    # non-temporal loads with the workgroup index, built for the 32,768- and
    # 65,536-element tiles: the automatic choice from 2^23 elements, here also
    # asked for explicitly, in and out of place, with ragged last tiles
    for n in ((1 << 23) + 5, (1 << 24) - 3, (1 << 25) + 65536 + 7):
        for dtype in DTYPES:
            for exclusive in (False, True):
                note(f"dispatch non-temporal dtype={dtype} excl={exclusive} n={n}")
                x = wl.random_input(dtype, n, seed=n + 11)
                y = _roundtrip(x, dtype, exclusive, in_place=exclusive, nt=1, tile_index=dws.TILE_DISPATCH)
                check(x, y, dtype, exclusive, label=f"dispatch nt n={n}")


# ---------------------------------------------------------------------------
# the pages' worked examples and Fig 6, through the protocol-inspection kernel
# ---------------------------------------------------------------------------
def _debug(x, dtype, exclusive, tile_elems, variant=dws.SINGLE_PASS, **kw):
    import torch
    _, xd = to_device(x)
    out = torch.empty_like(xd)
    desc = dws.scan_debug(xd, out, tile_elems, exclusive=exclusive, variant=variant, **kw)
    return from_device(out, dtype), desc


@pytest.mark.parametrize("fname", ["pmpp_11_3_hierarchical_example.txt", "pmpp_11_2_coarsened_example.txt"])
@pytest.mark.parametrize("variant", [dws.SINGLE_PASS, dws.CHAINED], ids=["lookback", "chained"])
def test_page_worked_example(gpu, fname, variant):
    g = read_golden(fname)
    x = np.array(g["input"], dtype=np.int32)
    note(f"worked example {fname} variant={variant}")
    y, desc = _debug(x, "int32", False, g["block_size"], variant=variant)
    assert y.tolist() == g["inclusive"]
    epoch, status, value = decode_desc(desc)
    assert status.tolist() == [2] * len(g["block_sums"])          # every tile ends P
    assert len(set(epoch.tolist())) == 1 and epoch[0] > 0
    assert value.view(np.int32).tolist() == g["scanned_block_sums"]  # S' of the example
    ye, _ = _debug(x, "int32", True, g["block_size"], variant=variant)
    assert ye.tolist() == [0] + g["inclusive"][:-1]
    # the same example through the production kernel (one tile)
    assert _roundtrip(x, "int32", False).tolist() == g["inclusive"]


def test_fig6_snapshot_premise(gpu):
    g = read_golden("decoupled_lookback_fig6.txt")
    p, s = g["partitions"], g["partition_sum"]
    rng = np.random.default_rng(6)
    parts = [np.diff(np.concatenate([[0], np.sort(rng.integers(0, s + 1, size=4)), [s]])) for _ in range(p)]
    x = np.concatenate(parts).astype(np.int32)
    for delay_every in (0, 2, 3):
        note(f"fig6 delay_every={delay_every}")
        y, desc = _debug(x, "int32", False, 5, delay_every=delay_every, delay_phase=1 if delay_every else 0,
                         delay_ticks=200_000)
        check(x, y, "int32", False)
        _, status, value = decode_desc(desc)
        assert status.tolist() == [2] * p
        assert value.view(np.int32).tolist() == [s * (t + 1) for t in range(p)]


# ---------------------------------------------------------------------------
# look-back protocol under stress: many small tiles, delayed publications
# ---------------------------------------------------------------------------
STRESS = [
    # (tile_elems, n, delay_every, delay_phase, delay_ticks)
    (1, 70_001, 0, 0, 0),
    (3, 200_003, 0, 0, 0),
    (64, 1_000_000, 0, 0, 0),
    (7, 100_000, 97, 13, 20_000),     # 0.2 ms stalls before publishing A
    (64, 640_000, 1001, 0, 200_000),  # tile 0 and every 1001st stall 2 ms
    (2, 40_000, 5, 4, 2_000),
]


@pytest.mark.parametrize("variant", [dws.SINGLE_PASS, dws.CHAINED], ids=["lookback", "chained"])
@pytest.mark.parametrize("dtype", ["uint32", "float32"])
def test_lookback_protocol_stress(gpu, dtype, variant):
    for tile_elems, n, every, phase, ticks in STRESS:
        if variant == dws.CHAINED and ticks * max(1, n // max(every, 1) // tile_elems) > 50_000_000:
            continue  # a serial chain would sum every stall; keep the case short
        for exclusive in (False, True):
            note(f"stress dtype={dtype} variant={variant} tile={tile_elems} n={n} delay={every}/{phase}/{ticks}")
            x = wl.random_input(dtype, n, seed=tile_elems * 7 + n)
            y, desc = _debug(x, dtype, exclusive, tile_elems, variant=variant, delay_every=every,
                             delay_phase=phase, delay_ticks=ticks)
            check(x, y, dtype, exclusive, label=f"stress tile={tile_elems} n={n}")
            epoch, status, value = decode_desc(desc)
            num_tiles = -(-n // tile_elems)
            assert status.size == num_tiles
            assert np.all(status == 2), "every tile must end with an inclusive prefix (P)"
            assert np.all(epoch == epoch[0]) and epoch[0] > 0
            ends = np.minimum(np.arange(1, num_tiles + 1) * tile_elems, n) - 1
            if dtype == "uint32":
                ref = oracle.scan_u32(x)
                assert np.array_equal(value, ref[ends])
            else:
                ref, sabs = oracle.scan_f32(x)
                got = value.view(np.float32).astype(np.float64)
                assert np.all(np.abs(got - ref[ends]) <= 1e-4 * sabs[ends] + 1e-6)


# ---------------------------------------------------------------------------
# repeated calls (epochs), several streams, determinism, special values
# ---------------------------------------------------------------------------
def test_repeated_calls_same_stream(gpu):
    import torch
    rng = np.random.default_rng(42)
    sizes = [int(v) for v in rng.integers(1, 40 * TILE, size=30)] + [TILE + 1] * 5 + [1 << 20] * 3
    for k, n in enumerate(sizes):
        dtype = DTYPES[k % 3]
        exclusive = bool(k & 1)
        note(f"repeat k={k} n={n} dtype={dtype}")
        x = wl.random_input(dtype, n, seed=k)
        y = _roundtrip(x, dtype, exclusive, in_place=(k % 4 == 0))
        check(x, y, dtype, exclusive, label=f"call {k}")
    # many back-to-back calls without host synchronisation in between
    x = wl.random_input("int32", 9 * TILE + 1, seed=5)
    _, xd = to_device(x)
    outs = [torch.empty_like(xd) for _ in range(50)]
    for o in outs:
        run(xd, o, x.size, "int32", False)
    ref = oracle.scan_i32(x)
    for o in outs:
        assert np.array_equal(from_device(o, "int32"), ref)


def test_concurrent_streams(gpu):
    import torch
    streams = [torch.cuda.Stream() for _ in range(4)]
    cases = []
    for k, s in enumerate(streams):
        n = (k + 1) * 37 * TILE + k
        x = wl.random_input("uint32", n, seed=200 + k)
        _, xd = to_device(x)
        out = torch.empty_like(xd)
        cases.append((x, xd, out, s))
    torch.cuda.synchronize()
    note("concurrent streams")
    for rep in range(3):
        for x, xd, out, s in cases:
            with torch.cuda.stream(s):
                run(xd, out, x.size, "uint32", rep == 1)
        torch.cuda.synchronize()
        for x, xd, out, s in cases:
            check(x, from_device(out, "uint32"), "uint32", rep == 1, label="stream")


def test_integer_results_are_deterministic(gpu):
    n = 1 << 24
    x = wl.random_input("int32", n, seed=8)
    a = _roundtrip(x, "int32", True)
    b = _roundtrip(x, "int32", True)
    assert np.array_equal(a, b)
    check(x, a, "int32", True)


def test_special_values(gpu):
    n = 3 * TILE + 11
    cases = [
        ("int32", np.full(n, 2**31 - 1, dtype=np.int32)),          # wraps every other element
        ("uint32", np.full(n, 0xFFFFFFFF, dtype=np.uint32)),        # y[i] = -(i+1) mod 2^32
        ("int32", np.full(n, -1, dtype=np.int32)),
        ("float32", np.zeros(n, dtype=np.float32)),
        ("float32", np.ones(n, dtype=np.float32)),
        ("float32", wl.generate("f32_normal", 1 << 20, 3) * np.float32(1e3)),
        ("float32", np.full(n, -0.25, dtype=np.float32)),
    ]
    for dtype, x in cases:
        for exclusive in (False, True):
            note(f"special dtype={dtype} excl={exclusive} first={x[0]!r}")
            y = _roundtrip(x, dtype, exclusive)
            check(x, y, dtype, exclusive)
    # closed forms, exactly
    ones = np.ones(n, dtype=np.float32)
    assert np.array_equal(_roundtrip(ones, "float32", False), np.arange(1, n + 1, dtype=np.float32))
    assert np.array_equal(_roundtrip(ones, "float32", True), np.arange(n, dtype=np.float32))
    y = _roundtrip(np.full(n, 0xFFFFFFFF, dtype=np.uint32), "uint32", False)
    assert np.array_equal(y.astype(np.int64), (-(np.arange(1, n + 1, dtype=np.int64))) & 0xFFFFFFFF)


def test_errors_enqueue_nothing(gpu):
    import torch
    x = torch.arange(1000, dtype=torch.int32, device="cuda")
    before = x.clone()
    st = dws.scan_inclusive_ptr(x.data_ptr(), x.data_ptr() + 4, 999, dws.INT32,
                                torch.cuda.current_stream().cuda_stream)
    assert st == dws.ERR_OVERLAP
    torch.cuda.synchronize()
    assert torch.equal(x, before)
    with pytest.raises(dws.ScanError):
        dws.scan_ex(x, variant=7)


# ---------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the benchmark
# times (default options through scan_inclusive / scan_exclusive)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["i32_4096_incl", "f32_2p20_incl", "u32_2p26_incl", "f32_2p28_excl_inplace", "flags_2p30m12345_excl"])
def test_workload_full_size(gpu, name):
    import torch
    w = wl.WORKLOADS[name]
    note(f"workload {name}: {w.description}")
    x = wl.generate_workload(w)
    store, xd = to_device(x)
    out = xd if w.in_place else torch.empty_like(xd)
    if w.dtype == "uint32":
        run(xd, out, x.size, "uint32", w.exclusive)
    else:
        (dws.scan_exclusive if w.exclusive else dws.scan_inclusive)(xd, out=out)
    torch.cuda.synchronize()
    y = from_device(out, w.dtype)
    del store, xd, out
    worst = check_chunked(x, y, w.dtype, w.exclusive, label=name)
    note(f"workload {name}: parity ok, max fp32 tolerance ratio {worst:.3g}")
    if name == "flags_2p30m12345_excl":
        # stream-compaction offsets: the exclusive scan of 0/1 flags ends at
        # popcount - last flag
        assert int(y[-1]) + int(x[-1]) == int(x.sum(dtype=np.int64))


@pytest.mark.parametrize("n", [5, (1 << 20) + 3, (1 << 24) + 77])
def test_profiled_scan(gpu, n):
    import torch
    for dtype in ("int32", "float32"):
        for exclusive in (False, True):
            note(f"profiled dtype={dtype} excl={exclusive} n={n}")
            x = wl.random_input(dtype, n, seed=n + 3)
            _, xd = to_device(x)
            out, stamps = dws.scan_profiled(xd, exclusive=exclusive)
            torch.cuda.synchronize()
            check(x, from_device(out, dtype), dtype, exclusive, label="profiled")
            st = stamps.cpu().numpy()
            assert st.shape == (dws.profiled_num_tiles(n), 5)
            assert np.all(st > 0), "every tile writes its stamps"
            assert np.all(np.diff(st, axis=1) >= 0), "phases are in order within a tile"


def test_profiled_scan_nontemporal(gpu):
    # from 2^28 elements the automatic choice loads with non-temporal loads;
    # the instrumented kernel the benchmark's phase stamps come from is that one
    import torch
    n = (1 << 28) + 5
    note(f"profiled fp32 exclusive n={n} (non-temporal loads)")
    x = wl.random_input("float32", n, seed=29)
    _, xd = to_device(x)
    out, stamps = dws.scan_profiled(xd, exclusive=True)
    torch.cuda.synchronize()
    check_chunked(x, from_device(out, "float32"), "float32", True, label="profiled non-temporal")
    st = stamps.cpu().numpy()
    assert st.shape == (dws.profiled_num_tiles(n), 5)
    assert np.all(st > 0) and np.all(np.diff(st, axis=1) >= 0)


# ---------------------------------------------------------------------------
# stream compaction (select by flags) fused with the single-pass scan
# ---------------------------------------------------------------------------
SEL_TILE_LARGE = 32768    # from 2^22 elements
SELECT_SIZES = [0, 1, 2, 63, 64, 65, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, 1_000_003,
                (1 << 22) - 1, 1 << 22, (1 << 22) + 1, (1 << 22) + SEL_TILE_LARGE + 5, 129 * SEL_TILE_LARGE - 3]
DENSITIES = [0.0, 0.01, 0.5, 0.99, 1.0]
SENTINEL = -0x21524111   # 0xdeadbeef as int32


def _select(x, flags, in_place=False, offset=0):
    """Run dws_select_flagged; returns (out as numpy over all n, count)."""
    import torch
    n = x.size
    _, xd = to_device(x, extra_front=offset)
    _, fd = to_device(flags, extra_front=offset)
    if in_place:
        out = xd
    else:
        ostore = torch.full((n + offset,), SENTINEL, dtype=torch.int32, device="cuda")
        out = ostore[offset:]
    count = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = dws.select_flagged_ptr(xd.data_ptr(), fd.data_ptr(), out.data_ptr(), n, dws.INT32,
                                count.data_ptr(), stream)
    assert st == dws.OK, dws.status_string(st)
    return from_device(out, "int32"), int(count.item())


def _check_select(x, flags, got, cnt, in_place, label):
    want = oracle.select_flagged(x, flags)
    assert cnt == want.size, f"{label}: count {cnt} != {want.size}"
    if not np.array_equal(got[:cnt], want):
        i = int(np.flatnonzero(got[:cnt] != want)[0])
        raise AssertionError(f"{label}: mismatch at {i}/{cnt}: gpu {got[i]} ref {want[i]}")
    # past the count the output is untouched: the sentinel, or (in place) the input
    rest = x[cnt:] if in_place else np.full(x.size - cnt, SENTINEL, dtype=np.int32)
    assert np.array_equal(got[cnt:], rest), f"{label}: output changed past the count"


@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
@pytest.mark.parametrize("density", DENSITIES)
def test_select_sizes_and_densities(gpu, density, in_place):
    for n in SELECT_SIZES:
        note(f"select n={n} density={density} in_place={in_place}")
        x = wl.generate("i32_full", n, seed=n + 1)
        flags = wl.selection_flags(n, density, seed=n + 2, any_nonzero=(n % 2 == 1))
        got, cnt = _select(x, flags, in_place=in_place)
        _check_select(x, flags, got, cnt, in_place, f"n={n} d={density}")


def test_select_nontemporal_tiles(gpu):
    # the large tiles with non-temporal loads (from 2^23): either side of the
    # threshold, and sizes past 2^25 and 2^27 with a ragged last tile, in and
    # out of place
    for n in ((1 << 23) - 1, (1 << 23) + SEL_TILE_LARGE + 5, (1 << 25) + SEL_TILE_LARGE + 5,
              (1 << 27) + SEL_TILE_LARGE + 5):
        x = wl.generate("i32_full", n, seed=n + 1)
        flags = wl.selection_flags(n, 0.5, seed=n + 2, any_nonzero=True)
        for in_place in (False, True):
            note(f"select n={n} in_place={in_place}")
            got, cnt = _select(x, flags, in_place=in_place)
            _check_select(x, flags, got, cnt, in_place, f"n={n} in_place={in_place}")


def test_select_unaligned(gpu):
    for off in (1, 3):
        for n in (TILE - 1, 5 * TILE + 7, (1 << 22) + 9):
            for in_place in (False, True):
                note(f"select unaligned off={off} n={n} in_place={in_place}")
                x = wl.generate("i32_full", n, seed=n + off)
                flags = wl.selection_flags(n, 0.3, seed=n + off + 1)
                got, cnt = _select(x, flags, in_place=in_place, offset=off)
                _check_select(x, flags, got, cnt, in_place, f"offset {off} n={n}")


def test_select_flags_are_the_input(gpu):
    # d_flags == d_in: keeps the non-zero words
    import torch
    n = 3 * SEL_TILE_LARGE + 11 + (1 << 22)
    note(f"select flags=input n={n}")
    x = wl.generate("flags_half", n, seed=9) * wl.generate("i32_full", n, seed=10)
    _, xd = to_device(x)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, cnt = dws.select_flagged(xd, xd, out=out, count=cnt)
    c = int(cnt.item())
    assert np.array_equal(from_device(out, "int32")[:c], x[x != 0])


def test_select_float_bits_and_binding(gpu):
    import torch
    n = 50_001
    note(f"select float bits n={n}")
    x = wl.generate("f32_normal", n, seed=12)
    x[::7] = -0.0
    x[5] = np.inf
    x[6] = np.nan
    flags = wl.selection_flags(n, 0.5, seed=13)
    xd = torch.from_numpy(x).cuda()
    fd = torch.from_numpy(flags).cuda()
    out, cnt = dws.select_flagged(xd, fd)
    c = int(cnt.item())
    want = oracle.select_flagged(x, flags)
    assert c == want.size
    assert np.array_equal(out[:c].cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_select_repeated_and_streams(gpu):
    # the descriptor epoch protocol is shared with the scans: interleave them
    import torch
    n = (1 << 22) + 77
    x = wl.generate("i32_full", n, seed=21)
    flags = wl.selection_flags(n, 0.5, seed=22)
    want = oracle.select_flagged(x, flags)
    _, xd = to_device(x)
    _, fd = to_device(flags)
    s2 = torch.cuda.Stream()
    for rep in range(6):
        note(f"select repeat {rep}")
        out = torch.empty_like(xd)
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        stream = s2 if rep % 2 else None
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                dws.select_flagged(xd, fd, out=out, count=cnt)
                y = dws.scan_exclusive(fd)
            torch.cuda.current_stream().wait_stream(stream)
        else:
            dws.select_flagged(xd, fd, out=out, count=cnt)
            y = dws.scan_exclusive(fd)
        torch.cuda.synchronize()
        c = int(cnt.item())
        assert c == want.size
        assert np.array_equal(out[:c].cpu().numpy(), want)
        check(flags, from_device(y, "int32"), "int32", True, label=f"interleaved scan {rep}")


def test_select_full_size(gpu):
    # the 2^30 - 12345 0/1 flags select from uniform int32 values, in place
    w = wl.WORKLOADS["flags_2p30m12345_excl"]
    note(f"select full size n={w.n}")
    flags = wl.generate_workload(w)
    x = wl.generate("i32_full", w.n, seed=wl.SELECT_VALUE_SEED)
    got, cnt = _select(x, flags, in_place=True)
    want = oracle.select_flagged(x, flags)
    assert cnt == want.size
    for s in range(0, cnt, 1 << 26):
        e = slice(s, min(s + (1 << 26), cnt))
        assert np.array_equal(got[e], want[e]), f"mismatch in [{s}, {e.stop})"
    assert np.array_equal(got[cnt:], x[cnt:])


def test_random_sizes(gpu):
    # 64 log-uniform sizes from 1 to 2^24 with random dtype, kind, in place
    # and pointer offset (seeded), through the default entry points
    rng = np.random.default_rng(2024)
    for case in range(64):
        n = int(np.exp(rng.uniform(0.0, np.log(1 << 24))))
        dtype = DTYPES[int(rng.integers(0, 3))]
        exclusive = bool(rng.integers(0, 2))
        in_place = bool(rng.integers(0, 2))
        offset = int(rng.integers(0, 4)) if rng.random() < 0.25 else 0
        note(f"random case {case}: n={n} dtype={dtype} excl={exclusive} in_place={in_place} offset={offset}")
        x = wl.random_input(dtype, n, seed=case)
        y = _roundtrip(x, dtype, exclusive, in_place=in_place, offset=offset)
        check(x, y, dtype, exclusive, label=f"random case {case} n={n}")


@pytest.mark.parametrize("n", [(1 << 22) + 7, (1 << 27) + 3], ids=["mid", "large"])
def test_graph_replays(gpu, n):
    # a captured call replays with the arguments it was captured with; the
    # descriptor epoch comes from the workspace, so every replay still sees
    # only its own descriptors, and a drawn-index scan's last draw puts the
    # tile counter back for the next one. Eager work (new inputs, an
    # uncaptured scan on the same stream) runs between replays, and every
    # replay is checked.
    import torch
    s = torch.cuda.Stream()
    x = torch.empty(n, dtype=torch.int32, device="cuda")
    out = torch.empty_like(x)
    flags = torch.empty_like(x)
    sel = torch.empty_like(x)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    pairs = torch.empty((n, 2), dtype=torch.int32, device="cuda")
    pout = torch.empty_like(pairs)
    dout = torch.empty_like(x)
    dws.reserve(n, stream=s.cuda_stream)
    with torch.cuda.stream(s):          # warm-up outside the capture
        dws.scan_exclusive(x, out)
        dws.scan_opts(x, dout, tile_index=dws.TILE_DRAWN)
        dws.select_flagged(x, flags, out=sel, count=cnt)
        dws.scan_op(pairs, dws.OP_AFFINE, dws.PAIR_U32, out=pout)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dws.scan_exclusive(x, out)
        dws.scan_opts(x, dout, tile_index=dws.TILE_DRAWN)
        dws.select_flagged(x, flags, out=sel, count=cnt)
        dws.scan_op(pairs, dws.OP_AFFINE, dws.PAIR_U32, out=pout)
    for rep in range(4):
        note(f"graph replay n={n} rep={rep}")
        data = wl.random_input("int32", n, seed=100 + rep)
        fl = wl.selection_flags(n, 0.5, seed=200 + rep)
        pr = wl.op_input("affine_u32", n, seed=300 + rep)
        x.copy_(torch.from_numpy(data))
        flags.copy_(torch.from_numpy(fl))
        pairs.copy_(torch.from_numpy(pr.view(np.int32)))
        with torch.cuda.stream(s):        # eager launch on the workspace between replays
            dws.scan_inclusive(flags, torch.empty_like(flags))
        s.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(data, from_device(out, "int32"), "int32", True, label=f"replay {rep}")
        check(data, from_device(dout, "int32"), "int32", False, label=f"drawn replay {rep}")
        want = oracle.select_flagged(data, fl)
        assert int(cnt.item()) == want.size
        assert np.array_equal(sel[:want.size].cpu().numpy(), want)
        assert np.array_equal(pout.cpu().numpy().view(np.uint32), oracle.scan_affine_u32(pr))


def test_capture_without_workspace_is_refused(gpu):
    # a call captured on a stream whose workspace does not exist yet, or lacks
    # the scan-then-propagate scratch, is refused before it allocates or
    # synchronises anything, so the capture itself stays valid; the same
    # stream then works eagerly
    import torch
    n = (1 << 20) + 3
    s = torch.cuda.Stream()
    data = wl.random_input("int32", n, seed=41)
    x = torch.from_numpy(data).cuda()
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    note("capture on a stream with no workspace")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(dws.ScanError) as err:
            dws.scan_exclusive(x, out)
    assert err.value.status == dws.ERR_UNSUPPORTED
    del g
    # a workspace reserved for a small n holds 1,024 scan-then-propagate tile
    # sums; 2^23 + 5 elements need more, so capturing that call must grow it
    s2 = torch.cuda.Stream()
    dws.reserve(4097, stream=s2.cuda_stream)
    n2 = (1 << 23) + 5
    data2 = wl.random_input("int32", n2, seed=43)
    x2 = torch.from_numpy(data2).cuda()
    out2 = torch.empty_like(x2)
    torch.cuda.synchronize()
    note("capture that would grow the scan-then-propagate scratch")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s2):
        with pytest.raises(dws.ScanError) as err:
            dws.scan_ex(x2, out2, exclusive=True, variant=dws.SCAN_THEN_PROPAGATE)
    assert err.value.status == dws.ERR_UNSUPPORTED
    del g
    note("eager calls on the same streams after the refused captures")
    with torch.cuda.stream(s):
        dws.scan_exclusive(x, out)
    with torch.cuda.stream(s2):
        dws.scan_ex(x2, out2, exclusive=True, variant=dws.SCAN_THEN_PROPAGATE)
    torch.cuda.synchronize()
    check(data, from_device(out, "int32"), "int32", True, label="after refused capture")
    check(data2, from_device(out2, "int32"), "int32", True, label="scan-then-propagate after refused capture")


def test_zz_watchdog_never_tripped(gpu):
    assert dws.watchdog_trips() == 0

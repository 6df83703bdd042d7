"""GPU parity of the compaction family fused with the single-pass scan:
partition by flags, reduce-by-key and run-length encoding, against the CPU
oracle on the same seeded inputs. Integer outputs and counts bit-exact; fp32
run sums within 1e-4 * (sum of |value| over the run) + 1e-6."""
import numpy as np
import pytest

import device_wide_prefix_amd as dws
import oracle
import scan_workloads as wl
from gpu_util import ATOL, RTOL, note

pytestmark = pytest.mark.gpu

SENTINEL = -0x21524111


def _dev(a, offset=0):
    import torch
    a = np.ascontiguousarray(a).view(np.int32)
    store = torch.empty(a.size + offset, dtype=torch.int32, device="cuda")
    view = store[offset:]
    view.copy_(torch.from_numpy(a))
    return view


def _empty(n, offset=0):
    import torch
    store = torch.full((n + offset,), SENTINEL, dtype=torch.int32, device="cuda")
    return store[offset:]


def _count():
    import torch
    return torch.full((1,), -1, dtype=torch.int64, device="cuda")


PARTITION_SIZES = [0, 1, 2, 65, 4095, 4096, 4097, 3 * 4096 + 7, 1_000_003, (1 << 22) - 1, (1 << 22) + 32768 + 5]


@pytest.mark.parametrize("density", [0.0, 0.01, 0.5, 1.0])
def test_partition(gpu, density):
    import torch
    for n in PARTITION_SIZES:
        for off in (0, 1):
            if off and n in (0, 1, 2):
                continue
            note(f"partition n={n} density={density} offset={off}")
            x = wl.generate("i32_full", n, seed=n + 3)
            f = wl.selection_flags(n, density, seed=n + 4, any_nonzero=True)
            xd, fd, out, cnt = _dev(x, off), _dev(f, off), _empty(n, off), _count()
            st = dws.load_library().dws_partition_flagged(xd.data_ptr(), fd.data_ptr(), out.data_ptr(), n, dws.INT32,
                                                          cnt.data_ptr(), torch.cuda.current_stream().cuda_stream)
            assert st == dws.OK, dws.status_string(st)
            want, c = oracle.partition_flagged(x, f)
            assert int(cnt.item()) == c
            assert np.array_equal(out.cpu().numpy(), want), f"n={n}"


def _check_runs(name, keys, got_keys, got_aggs, got_count, vals=None):
    if vals is None:
        uk, ln = oracle.run_length_encode(keys)
        want_aggs, abs_sums = ln, None
    else:
        uk, want_aggs, abs_sums = oracle.reduce_by_key(keys, vals)
    r = uk.size
    assert got_count == r, f"{name}: {got_count} runs, oracle {r}"
    assert np.array_equal(got_keys[:r].view(np.uint32), uk.view(np.uint32)), f"{name}: keys"
    if abs_sums is None:
        assert np.array_equal(got_aggs[:r].view(np.uint32), want_aggs.view(np.uint32)), f"{name}: sums"
    else:
        g = got_aggs[:r].view(np.float32).astype(np.float64)
        err = np.abs(g - want_aggs)
        bound = RTOL * abs_sums + ATOL
        assert np.all(err <= bound), f"{name}: fp32 sum at {int(np.flatnonzero(err > bound)[0])}"
    # output elements past the runs are untouched
    assert np.all(got_keys[r:] == SENTINEL) and np.all(got_aggs[r:] == SENTINEL), f"{name}: wrote past the runs"


# around the small (4096) and large (16384 or 32768, from 2^22) tiles, a
# ragged last tile with empty wave segments, 2^25 + 5, and 2^26 + 5 where the
# look-back's long back-off is on; runs from length 1 to longer than a tile
RBK_SIZES = [1, 2, 3, 4095, 4096, 4097, 3 * 4096 + 7, 100_003, (1 << 22) - 1, (1 << 22) + 16384 + 3,
             (1 << 25) + 5, (1 << 26) + 5]
MEAN_RUNS = [1, 3, 200, 50_000]


@pytest.mark.parametrize("value_dtype", ["int32", "uint32", "float32", "rle"])
def test_reduce_by_key_and_rle(gpu, value_dtype):
    import torch
    for n in RBK_SIZES:
        for mean_run in MEAN_RUNS:
            if n > (1 << 22) + 20000 and mean_run in (3, 200):
                continue
            note(f"reduce-by-key values={value_dtype} n={n} mean_run={mean_run}")
            keys = wl.run_keys(n, mean_run, seed=n + mean_run)
            stream = torch.cuda.current_stream().cuda_stream
            kd, uk, ag, cnt = _dev(keys), _empty(n), _empty(n), _count()
            if value_dtype == "rle":
                st = dws.load_library().dws_run_length_encode(kd.data_ptr(), uk.data_ptr(), ag.data_ptr(), n,
                                                              cnt.data_ptr(), stream)
                vals = None
            else:
                vals = {"int32": lambda: wl.generate("i32_full", n, n),
                        "uint32": lambda: wl.generate("u32_full", n, n),
                        "float32": lambda: wl.generate("f32_pm1", n, n)}[value_dtype]()
                code = {"int32": dws.INT32, "uint32": dws.UINT32, "float32": dws.FLOAT32}[value_dtype]
                vd = _dev(vals)
                st = dws.load_library().dws_reduce_by_key(kd.data_ptr(), vd.data_ptr(), uk.data_ptr(), ag.data_ptr(),
                                                          n, code, cnt.data_ptr(), stream)
            assert st == dws.OK, dws.status_string(st)
            _check_runs(f"{value_dtype} n={n} run={mean_run}", keys, uk.cpu().numpy(), ag.cpu().numpy(),
                        int(cnt.item()), vals)


def _run_both(keys, vals, name):
    """Integer reduce-by-key and run-length encoding of the same keys, checked
    against the oracle."""
    import torch
    n = keys.size
    stream = torch.cuda.current_stream().cuda_stream
    kd, vd = _dev(keys), _dev(vals)
    uk, ag, cnt = _empty(n), _empty(n), _count()
    st = dws.load_library().dws_reduce_by_key(kd.data_ptr(), vd.data_ptr(), uk.data_ptr(), ag.data_ptr(), n,
                                              dws.UINT32, cnt.data_ptr(), stream)
    assert st == dws.OK, dws.status_string(st)
    _check_runs(f"{name} sums", keys, uk.cpu().numpy(), ag.cpu().numpy(), int(cnt.item()), vals)
    uk, ag, cnt = _empty(n), _empty(n), _count()
    st = dws.load_library().dws_run_length_encode(kd.data_ptr(), uk.data_ptr(), ag.data_ptr(), n, cnt.data_ptr(),
                                                  stream)
    assert st == dws.OK, dws.status_string(st)
    _check_runs(f"{name} lengths", keys, uk.cpu().numpy(), ag.cpu().numpy(), int(cnt.item()))


def test_run_boundaries(gpu):
    # Where a run's sum comes from: its own segment, the value carried in
    # through the look-back, or the segment aggregate of the array's last
    # element. From 2^22 keys wave segments hold 2,048 (sums) or 4,096 (run
    # lengths) keys and tiles 16,384 or 32,768; 4,096-key tiles below.
    big = (1 << 22) + 4096          # the array ends exactly at a segment's end
    for n in (5000, big, (1 << 22) + 4097):
        vals = wl.generate("u32_full", n, n + 7)
        for key in (0, 0xFFFFFFFF, 12345):
            note(f"run boundaries: one run of key {key:#x}, n={n}")
            _run_both(np.full(n, key, dtype=np.uint32), vals, f"one run key={key:#x} n={n}")
        for length in (2048, 4096, 16384, 32768):
            note(f"run boundaries: runs of exactly {length}, n={n}")
            keys = (np.arange(n, dtype=np.uint32) // length).astype(np.uint32) * np.uint32(2654435761)
            _run_both(keys, vals, f"runs of {length} n={n}")
        note(f"run boundaries: mean run 1 and 50,000, n={n}")
        for mean_run in (1, 50_000):
            _run_both(wl.run_keys(n, mean_run, seed=n + mean_run), vals, f"mean run {mean_run} n={n}")


def _threshold_keys(n):
    """Keys whose 4,096-element blocks (a run-length wave segment; two of
    reduce-by-key's 2,048) cycle through head counts on either side of the
    1,024 heads up to which a segment stages all of its heads before the
    look-back: exactly 1,024 heads, 1,025, about 1,365 (random runs of 1 to
    5), 4,096 (all distinct) and 1 (one run across the block, so the next
    block's first run starts elsewhere)."""
    rng = np.random.default_rng(n)
    lengths = []
    for b in range(n // 4096 + 1):
        kind = b % 5
        if kind == 0:
            lengths += [4] * 1024
        elif kind == 1:
            lengths += [4] * 1023 + [2, 2]
        elif kind == 2:
            left = 4096
            while left > 0:
                r = int(min(left, rng.integers(1, 6)))
                lengths.append(r)
                left -= r
        elif kind == 3:
            lengths += [1] * 4096
        else:
            lengths.append(4096)
    run = np.repeat(np.arange(len(lengths), dtype=np.uint64), lengths)[:n]
    return ((run * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def test_stage_threshold(gpu):
    # wave segments on both sides of the staging threshold inside the same
    # tiles, with runs that cross segments, waves and tiles; integer and fp32
    # sums and run lengths
    import torch
    for n in ((1 << 22) + 3 * 4096 + 5, (1 << 25) + 7):
        keys = _threshold_keys(n)
        note(f"staging threshold n={n}")
        _run_both(keys, wl.generate("u32_full", n, n + 11), f"threshold n={n}")
        vals = wl.generate("f32_pm1", n, n + 12)
        kd, vd, uk, ag, cnt = _dev(keys), _dev(vals), _empty(n), _empty(n), _count()
        st = dws.load_library().dws_reduce_by_key(kd.data_ptr(), vd.data_ptr(), uk.data_ptr(), ag.data_ptr(), n,
                                                  dws.FLOAT32, cnt.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == dws.OK, dws.status_string(st)
        _check_runs(f"threshold fp32 n={n}", keys, uk.cpu().numpy(), ag.cpu().numpy(), int(cnt.item()), vals)


def test_reduce_by_key_unaligned_and_special_keys(gpu):
    import torch
    # keys and values one element off 16-byte alignment (scalar-load kernel),
    # and fp32 keys compared as bit patterns (-0.0 != +0.0, equal NaNs match)
    for n in (4097, 100_003, (1 << 22) + 9):
        note(f"reduce-by-key unaligned n={n}")
        keys = wl.run_keys(n, 5, seed=n)
        vals = wl.generate("i32_full", n, n + 1)
        kd, vd = _dev(keys, 1), _dev(vals, 3)
        uk, ag, cnt = _empty(n, 1), _empty(n, 2), _count()
        st = dws.load_library().dws_reduce_by_key(kd.data_ptr(), vd.data_ptr(), uk.data_ptr(), ag.data_ptr(), n,
                                                  dws.INT32, cnt.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == dws.OK
        _check_runs(f"unaligned n={n}", keys, uk.cpu().numpy(), ag.cpu().numpy(), int(cnt.item()), vals)
    special = np.array([0.0, -0.0, -0.0, 0.0, np.nan, np.nan, 1.0], dtype=np.float32)
    keys = np.tile(special, 5000).view(np.uint32)
    note("reduce-by-key special keys")
    kd = torch.from_numpy(keys.view(np.int32)).cuda()
    uk, ln, cnt = dws.run_length_encode(kd, unique_keys=_empty(keys.size), lengths=_empty(keys.size))
    _check_runs("special keys", keys, uk.cpu().numpy(), ln.cpu().numpy(), int(cnt.item()))


def test_binding_full_size(gpu):
    # the 2^30 - 12345 0/1 flags partition 2^30 - 12345 uniform int32 values; reduce-by-key
    # over 2^27 keys in runs of mean length 32 with fp32 values
    import torch
    w = wl.WORKLOADS["flags_2p30m12345_excl"]
    note(f"partition full size n={w.n}")
    flags = wl.generate_workload(w)
    x = wl.generate("i32_full", w.n, seed=wl.SELECT_VALUE_SEED)
    out, cnt = dws.partition_flagged(torch.from_numpy(x).cuda(), torch.from_numpy(flags).cuda())
    want, c = oracle.partition_flagged(x, flags)
    assert int(cnt.item()) == c
    got = out.cpu().numpy()
    for s in range(0, w.n, 1 << 26):
        assert np.array_equal(got[s:s + (1 << 26)], want[s:s + (1 << 26)]), f"partition mismatch in block {s}"
    del out, got, want, x, flags
    torch.cuda.empty_cache()
    n = 1 << 27
    note(f"reduce-by-key full size n={n}")
    keys = wl.run_keys(n, 32, seed=9)
    vals = wl.generate("f32_pm1", n, 10)
    uk, ag, cnt = dws.reduce_by_key(torch.from_numpy(keys.view(np.int32)).cuda(), torch.from_numpy(vals).cuda())
    r = int(cnt.item())
    want_k, want_a, abs_s = oracle.reduce_by_key(keys, vals)
    assert r == want_k.size
    assert np.array_equal(uk[:r].cpu().numpy().view(np.uint32), want_k)
    g = ag[:r].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g - want_a) <= RTOL * abs_s + ATOL)

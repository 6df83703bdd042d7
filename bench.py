"""Benchmark of the device-wide + scan on one MI355X.

Default: the headline workload, an exclusive + scan in place of N = 2^28 fp32
values uniform in [0, 1) (seed 3), through scan_exclusive (the single-pass
decoupled look-back kernel). Prints ONE JSON line on stdout:
  value        scan GB/s = 2 * N * 4 bytes / mean step time
  roofline     the scan kernel against the 8 TB/s HBM peak
  memcpy       a same-run device-to-device hipMemcpyAsync of N * 4 bytes,
               counted the same way (2 * N * 4 bytes)
  cpu_baseline the sequential CPU oracle on the same input (1 host core)
  configs      every workload the metric is stated on, with its memcpy and oracle
  shard_8      one device's share of the headline split 8 ways: shard total,
               seeded scan and the per-device sequence (see --shards)

Step protocol: before every step (untimed) the input is restored from a
pristine device copy and the caches (L2, MALL) are flushed by reading a 1 GiB
buffer; a step is one scan call bracketed by HIP events on the stream the
library launches on. The call is a single kernel launch, so the event time is
the kernel's launch duration.

Options: --workload NAME (a key of scan_workloads.WORKLOADS),
--variant single_pass|reduce_then_scan|chained|scan_then_propagate,
--order relaxed|acq_rel, --tile-shape K, --nontemporal auto|on|off, --no-cpu-baseline,
--all (extra JSON lines for every workload and variant on stderr), --sweep
(N = 2^10..2^30, every variant and memcpy, cold and warm caches; stderr),
--shards G (one device's share of the headline scan split into G shards:
reduce, seeded scan and both together; stderr), --select (stream compaction on the 2^30-12345 flag workload; stderr), --ops
(generic-operator scans: max, min, {int32, fp32} pair sum, affine maps,
segmented sum, on 1 GiB inputs; stderr), --compaction (select, partition,
reduce-by-key, run-length encoding on 2^25 items, beside PyTorch; stderr).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import scan_workloads as wl  # noqa: E402

METRIC = "scan GB/s (2n·sizeof(T)/time) at N=2^28 fp32; % of HBM peak & of D2D memcpy"
HBM_PEAK_GBPS = 8000.0
FLUSH_BYTES = 1 << 30
# shader clocks of the spin kernel that precedes every timed call (~100 us)
SPIN_CYCLES = 250_000
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_scan_f32_2p28.json")
VARIANTS = {"single_pass": 0, "reduce_then_scan": 1, "chained": 2, "scan_then_propagate": 3}
ORDERS = {"relaxed": 0, "acq_rel": 1}
TILE_INDEX = {"auto": 0, "drawn": 1, "dispatch": 2}
NONTEMPORAL = {"auto": 0, "on": 1, "off": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources the fp32 single-pass kernel is compiled from
SINGLE_PASS_SOURCES = ("dws_device.hpp", "dws_protocol.h", "dws_single_pass.h", "dws_single_pass_kernel.hpp",
                       "dws_sp_f32.hip")


def strip_comments(src: str) -> str:
    """C/C++ source without its comments and with every whitespace run reduced
    to one space: what the compiler sees, as far as a fingerprint needs."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src[i] in "\"'":
            j = i + 1
            while j < n and src[j] != src[i]:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha(names=SINGLE_PASS_SOURCES) -> str:
    """Hash of the code (comments and layout left out) of the sources a kernel
    is built from, to tell whether stored counters still apply to it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "device_wide_prefix_amd", "csrc")
    for name in sorted(names):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


class Hip:
    """hipMemcpyAsync through the HIP runtime (the memcpy reference)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_int, ctypes.c_void_p]
        self.lib.hipMemcpyAsync.restype = ctypes.c_int

    def memcpy_d2d(self, dst: int, src: int, nbytes: int, stream: int):
        rc = self.lib.hipMemcpyAsync(dst, src, nbytes, 3, stream)  # hipMemcpyDeviceToDevice
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync failed ({rc})")


def time_steps(fn, prepare, steps: int, warmup: int):
    """Run warmup + steps; each step: prepare() untimed, then fn() between two
    events on the current stream. Returns per-step milliseconds.

    Between prepare() and the first event the stream runs a short spin kernel
    (about 100 us, no memory traffic), so the GPU is still busy while the host
    records the event and issues fn(): the events then time the GPU's work on
    fn() from the moment the GPU is free, not the interpreter's latency in
    issuing it. Every timed callable (scans, memcpy, library comparisons) is
    timed this way."""
    import torch
    times = []
    for i in range(warmup + steps):
        prepare()
        torch.cuda._sleep(SPIN_CYCLES)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        if i >= warmup:
            times.append(a.elapsed_time(b))
    torch.cuda.synchronize()
    return times


def run_workload(w: wl.Workload, variant: int, order: int, shape: int, nt: int, steps: int, warmup: int,
                 with_memcpy: bool, x_host=None, instrument: bool = True, flush_caches: bool = True,
                 tile_index: int = 0, with_library: bool = True):
    import torch
    import device_wide_prefix_amd as dws

    x = wl.generate_workload(w) if x_host is None else x_host
    tdtype = torch.float32 if w.dtype == "float32" else torch.int32
    host = torch.from_numpy(x if w.dtype != "uint32" else x.view(np.int32))
    pristine = host.to("cuda")
    work = torch.empty_like(pristine)
    out = work if w.in_place else torch.empty_like(pristine)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    code = {"int32": dws.INT32, "uint32": dws.UINT32, "float32": dws.FLOAT32}[w.dtype]
    stream = torch.cuda.current_stream().cuda_stream
    dws.reserve(w.n)
    opt = dws.DwsOptions(variant, order, shape, int(nt), tile_index)
    default = variant == 0 and order == 0 and shape == 0 and nt == 0 and tile_index == 0
    entry = dws.scan_exclusive_ptr if w.exclusive else dws.scan_inclusive_ptr

    def prepare():
        work.copy_(pristine)
        if flush_caches:
            flush.sum()    # read-only flush: leaves clean lines, no write-back later

    def scan():
        if default:
            st = entry(work.data_ptr(), out.data_ptr(), w.n, code, stream)
        else:
            st = dws.scan_opts_ptr(work.data_ptr(), out.data_ptr(), w.n, code, w.exclusive, opt, stream)
        if st != dws.OK:
            raise RuntimeError(f"scan failed: {dws.status_string(st)}")

    launch = None
    if variant in (0, 2):
        # what the library resolves the options to for these buffers
        st, plan = dws.scan_plan_ptr(work.data_ptr(), out.data_ptr(), w.n, code, w.exclusive, opt)
        if st != dws.OK:
            raise RuntimeError(f"scan plan failed: {dws.status_string(st)}")
        launch = {"threads": plan.threads, "tile_elems": plan.tile_elems, "num_tiles": plan.num_tiles,
                  "tile_index": "drawn" if plan.tile_index == dws.TILE_DRAWN else "dispatch",
                  "nontemporal": bool(plan.nontemporal), "pause_units": plan.pause_units}

    trips_before = dws.watchdog_trips()
    times = time_steps(scan, prepare, steps, warmup)
    # a look-back wait that timed out leaves wrong output behind a DWS_OK
    # status: count the trips of the timed steps and fail the check on any
    trips = dws.watchdog_trips() - trips_before
    result = {"times_ms": times, "watchdog_trips": int(trips), "launch": launch}

    # property checks that hold at any size (no oracle here)
    y = out.cpu().numpy()
    if w.dtype == "uint32":
        y = y.view(np.uint32)
    if w.dtype == "float32":
        tot = float(np.sum(x, dtype=np.float64))
        last = float(y[-1]) + (float(x[-1]) if w.exclusive else 0.0)
        sabs = float(np.sum(np.abs(x), dtype=np.float64))
        ok = abs(last - tot) <= 1e-4 * sabs + 1e-6
        if w.exclusive:
            ok = ok and float(y[0]) == 0.0
        # (no monotonicity check: fp32 prefixes reached through different
        # rounding paths may step back by an ulp where x[i] is below the ulp)
    else:
        # integers: the whole output, exactly. Adjacent outputs differ by one
        # input element modulo 2^32 (x[i] inclusive, x[i-1] exclusive), and the
        # first output is x[0] (inclusive) or 0 (exclusive).
        yu, xu = y.view(np.uint32), x.view(np.uint32)
        step = yu[1:] - yu[:-1]          # uint32 arithmetic wraps modulo 2^32
        ok = bool(np.array_equal(step, xu[:-1] if w.exclusive else xu[1:]))
        ok = ok and int(yu[0]) == (0 if w.exclusive else int(xu[0]))
        del step
    result["property_check"] = bool(ok) and trips == 0

    if instrument and w.dtype != "uint32" and default:
        # one instrumented run: where a tile's time goes (100 MHz stamps)
        prepare()
        torch.cuda.synchronize()
        _, st = dws.scan_profiled(work, out=out, exclusive=w.exclusive)
        torch.cuda.synchronize()
        st = st.cpu().numpy().astype(np.int64)
        life = (st[:, 4] - st[:, 0]).astype(np.float64)
        phases = {"tile_index": st[:, 1] - st[:, 0], "load_and_local_scan": st[:, 2] - st[:, 1],
                  "lookback": st[:, 3] - st[:, 2], "finish_and_store_issue": st[:, 4] - st[:, 3]}
        result["lookback_stall_share"] = float((st[:, 3] - st[:, 2]).sum() / life.sum())
        result["phase_mean_us"] = {k: round(float(v.mean()) * 0.01, 3) for k, v in phases.items()}
        result["tiles"] = int(st.shape[0])

    if with_memcpy:
        hip = Hip()
        dst = torch.empty_like(pristine)
        nbytes = w.n * 4

        def memcpy():
            hip.memcpy_d2d(dst.data_ptr(), work.data_ptr(), nbytes, stream)

        result["memcpy_times_ms"] = time_steps(memcpy, prepare, steps, warmup)
        # the vendor library's device-wide scan on the same input, out of
        # place: torch.cumsum of a 1-D GPU tensor runs hipCUB's inclusive
        # scan (rocPRIM's look-back scan) on ROCm
        if w.dtype != "uint32" and with_library:
            result["torch_cumsum_times_ms"] = time_steps(lambda: torch.cumsum(work, 0, dtype=work.dtype, out=dst),
                                                         prepare, steps,
                                                         warmup)
        del dst
    del pristine, work, out, flush
    torch.cuda.empty_cache()
    return result


SWEEP_EXPONENTS = range(10, 31)


def run_sweep(steps: int, warmup: int):
    """Exclusive in-place fp32 scan (the headline workload's kind) at N = 2^10 ..
    2^30, every variant, against a same-size device-to-device memcpy; cold
    (caches flushed before each step) and warm (no flush). Inputs are prefixes
    of one seeded draw. One JSON line per (N, variant, cache state) on stderr."""
    w_big = wl.WORKLOADS["f32_2p28_excl_inplace"]
    x_all = wl.generate(w_big.dist, 1 << max(SWEEP_EXPONENTS), w_big.seed)
    rows = []
    for k in SWEEP_EXPONENTS:
        n = 1 << k
        w = wl.Workload(f"sweep_2^{k}", n, "float32", w_big.dist, w_big.seed, True, True,
                        f"exclusive + scan in place, N=2^{k} fp32 uniform [0,1) (prefix of the seed-3 draw)")
        x = x_all[:n]
        for cold in (True, False):
            for vname, v in VARIANTS.items():
                r = run_workload(w, v, 0, 0, 0, steps, warmup, with_memcpy=(v == 0), x_host=x,
                                 instrument=False, flush_caches=cold)
                row = summarize(w, r, vname, None)
                row["cache"] = "cold" if cold else "warm"
                row["n"] = n
                log("SWEEP " + json.dumps(row))
                rows.append(row)
    return rows


ORACLE_SAMPLE = 1 << 26   # elements of a large input the oracle is timed on


def run_select(steps: int, warmup: int, in_place: bool, with_oracle: bool = True):
    """Stream compaction: the 2^30 - 12345 0/1 flags (Bernoulli 0.5, seed 4) select from
    uniform int32 values (seed 5). Algorithmic bytes = read values and flags
    (8 n) + write the selected values (4 count). Also times torch.masked_select
    on the same data (its output size needs a host synchronisation)."""
    import torch
    import device_wide_prefix_amd as dws
    w = wl.WORKLOADS["flags_2p30m12345_excl"]
    n = w.n
    flags_h = wl.generate_workload(w)
    vals_h = wl.generate("i32_full", n, wl.SELECT_VALUE_SEED)
    flags = torch.from_numpy(flags_h).to("cuda")
    vals = torch.from_numpy(vals_h).to("cuda")
    work = torch.empty_like(vals)
    out = work if in_place else torch.empty_like(vals)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    dws.reserve(n)

    def prepare():
        work.copy_(vals)
        flush.sum()

    def select():
        st = dws.select_flagged_ptr(work.data_ptr(), flags.data_ptr(), out.data_ptr(), n, dws.INT32,
                                    cnt.data_ptr(), stream)
        if st != dws.OK:
            raise RuntimeError(f"select failed: {dws.status_string(st)}")

    times = time_steps(select, prepare, steps, warmup)
    count = int(cnt.item())
    mask = flags != 0
    ok = count == int(mask.sum().item())
    ok = ok and bool(torch.equal(out[:count], vals[mask]))
    algo = 8 * n + 4 * count
    mean = float(np.mean(times))
    row = {"op": "select_flagged", "n": n, "in_place": in_place, "count": count, "ms_mean": mean,
           "ms_min": float(np.min(times)), "gbps": algo / (mean * 1e-3) / 1e9,
           "frac_hbm_peak": algo / (mean * 1e-3) / 1e9 / HBM_PEAK_GBPS, "property_check": ok}

    # select-if on the same values by a predicate (x < 0, about half of
    # uniform int32 values): the selection comes from the values, so the
    # kernel reads 4 n bytes instead of 8 n
    cnt_if = torch.zeros(1, dtype=torch.int64, device="cuda")
    zero = np.zeros(1, dtype=np.int32)

    def select_if():
        st = dws.load_library().dws_select_if(work.data_ptr(), out.data_ptr(), n, dws.INT32, dws.PRED_LT,
                                              zero.ctypes.data, cnt_if.data_ptr(), stream)
        if st != dws.OK:
            raise RuntimeError(f"select_if failed: {dws.status_string(st)}")

    ti = time_steps(select_if, prepare, steps, warmup)
    count_if = int(cnt_if.item())
    neg = vals < 0
    ok_if = count_if == int(neg.sum().item()) and bool(torch.equal(out[:count_if], vals[neg]))
    mean_if = float(np.mean(ti))
    algo_if = 4 * n + 4 * count_if
    row.update({"select_if_lt0_count": count_if, "select_if_lt0_ms_mean": mean_if,
                "select_if_lt0_gbps": algo_if / (mean_if * 1e-3) / 1e9,
                "select_if_lt0_frac_hbm_peak": algo_if / (mean_if * 1e-3) / 1e9 / HBM_PEAK_GBPS})
    row["property_check"] = bool(row["property_check"] and ok_if)
    del neg

    def torch_select():
        torch.masked_select(work, mask)

    tt = time_steps(torch_select, prepare, max(3, steps // 2), 2)
    row["torch_masked_select_ms_mean"] = float(np.mean(tt))
    row["speedup_vs_torch_masked_select"] = float(np.mean(tt)) / mean
    if with_oracle:
        import oracle
        m = min(n, ORACLE_SAMPLE)
        fs, vs = flags_h[:m], vals_h[:m]
        sel = int(np.count_nonzero(fs))
        row["cpu_baseline"] = oracle_rate(lambda: oracle.select_flagged(vs, fs), 8 * m + 4 * sel,
                                        f"first {m} values and flags of the same input")
    del flags, vals, work, out, flush, mask, flags_h, vals_h
    torch.cuda.empty_cache()
    return row


# name: (op, dtype, input kind, element bytes); every case reads and writes 1 GiB
OP_CASES = {
    "max_i32": (0x1, 0, "i32_full", 4),
    "min_u32": (0x2, 1, "u32_full", 4),
    "sum_pair_i32_f32": (0x0, 3, "pair_i32_f32", 8),
    "affine_u32": (0x3, 4, "affine_u32", 8),
    "segsum_i32_f32": (0x4, 3, "segsum_i32_f32", 8),
}
OP_BYTES = 1 << 31


def _op_oracle():
    """Operator name -> the oracle's inclusive scan for it (CPU baseline only)."""
    import oracle
    return {
        "max_i32": lambda x: oracle.scan_minmax(x, True),
        "min_u32": lambda x: oracle.scan_minmax(x, False),
        "sum_pair_i32_f32": lambda x: oracle.scan_pair_sum_i32_f32(x),
        "affine_u32": lambda x: oracle.scan_affine_u32(x),
        "segsum_i32_f32": lambda x: oracle.scan_segsum_i32_f32(x),
    }


def op_property_check(name: str, x: np.ndarray, y: np.ndarray) -> bool:
    """Checks that hold at any size (no oracle here)."""
    if name == "max_i32":
        return bool(np.all(np.diff(y.view(np.int32).astype(np.int64)) >= 0) and y.view(np.int32)[-1] == x.max())
    if name == "min_u32":
        return bool(np.all(np.diff(y.astype(np.int64)) <= 0) and y[-1] == x.min())
    if name == "sum_pair_i32_f32":
        tot_i = int(np.sum(x[:, 0].view(np.int32).astype(np.int64))) & 0xFFFFFFFF
        f = x[:, 1].view(np.float32).astype(np.float64)
        tot_f = float(f.sum())
        return bool(int(y[-1, 0]) == tot_i and abs(float(y[-1:, 1].view(np.float32)[0]) - tot_f)
                    <= 1e-4 * float(np.abs(f).sum()) + 1e-6)
    if name == "affine_u32":
        v, s = 7, 7
        for i in range(2000):   # the recurrence, run directly, from start value 7
            v = (int(x[i, 0]) * v + int(x[i, 1])) & 0xFFFFFFFF
            if v != (int(y[i, 0]) * s + int(y[i, 1])) & 0xFFFFFFFF:
                return False
        return True
    if name == "segsum_i32_f32":
        heads = np.flatnonzero(x[:, 0] != 0)
        return bool(np.array_equal(y[heads, 1], x[heads, 1]))   # a head restarts with its own value
    return False


def run_ops(steps: int, warmup: int, with_oracle: bool = True):
    """Generic-operator scans of 1 GiB of input (2^28 32-bit or 2^27 pair
    elements), out of place, cold caches; GB/s counts 2 x the input bytes,
    like the + scan, against a same-size memcpy; and the reduction of the same
    input under the operator (dws_reduce_op; GB/s counts the input bytes once).
    One OPS line per operator."""
    import torch
    import device_wide_prefix_amd as dws
    rows = []
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()
    OP_ORACLE = _op_oracle() if with_oracle else {}
    for name, (op, dtype, kind, esize) in OP_CASES.items():
        n = (OP_BYTES // 2) // esize
        x = wl.op_input(kind, n, seed=11)
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int32).reshape(-1)).to("cuda")
        out = torch.empty_like(xd)
        dws.reserve(n)

        def prepare():
            flush.sum()

        def scan():
            st = dws.scan_op_ptr(xd.data_ptr(), out.data_ptr(), n, dtype, op, False, stream)
            if st != dws.OK:
                raise RuntimeError(f"{name}: {dws.status_string(st)}")

        times = time_steps(scan, prepare, steps, warmup)
        y = out.cpu().numpy().view(np.uint32).reshape(x.shape)
        ok = op_property_check(name, x, y)
        # the same input's total under the operator (dws_reduce_op, n * esize
        # bytes read): the inclusive scan's last element, fp32 parts within
        # the scans' bar
        total = torch.zeros(esize // 4, dtype=torch.int32, device="cuda")

        def reduce():
            st = dws.reduce_op_ptr(xd.data_ptr(), n, dtype, op, total.data_ptr(), stream)
            if st != dws.OK:
                raise RuntimeError(f"{name} reduce: {dws.status_string(st)}")

        rtimes = time_steps(reduce, prepare, steps, warmup)
        tw = total.cpu().numpy().view(np.uint32)
        last = y.reshape(n, -1)[-1]
        if name in ("sum_pair_i32_f32", "segsum_i32_f32"):
            xs = x.reshape(n, -1)[:, 1].view(np.float32).astype(np.float64)
            scale = float(np.abs(xs).sum())
            ok = ok and tw[0] == last[0] and abs(float(tw[1:2].view(np.float32)[0])
                                               - float(last[1:2].view(np.float32)[0])) <= 2e-4 * scale + 1e-6
        else:
            ok = ok and np.array_equal(tw, last)
        mc = time_steps(lambda: hip.memcpy_d2d(out.data_ptr(), xd.data_ptr(), n * esize, stream), prepare,
                        steps, warmup)
        mean, mcm = float(np.mean(times)), float(np.mean(mc))
        row = {"op": name, "n": n, "element_bytes": esize, "ms_mean": mean, "ms_min": float(np.min(times)),
               "gbps": 2 * n * esize / (mean * 1e-3) / 1e9, "memcpy_gbps": 2 * n * esize / (mcm * 1e-3) / 1e9,
               "frac_memcpy": mcm / mean, "frac_hbm_peak": 2 * n * esize / (mean * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               "reduce_ms_mean": float(np.mean(rtimes)),
               "reduce_gbps": n * esize / (float(np.mean(rtimes)) * 1e-3) / 1e9,
               "property_check": ok}
        if with_oracle:
            m = min(n, ORACLE_SAMPLE // 4)
            xs = np.ascontiguousarray(x[:m])
            row["cpu_baseline"] = oracle_rate(lambda: OP_ORACLE[name](xs), 2 * m * esize,
                                              f"first {m} elements of the same input")
        log("OPS " + json.dumps(row))
        rows.append(row)
        del xd, out
        torch.cuda.empty_cache()
    return rows


def run_shards(steps: int, warmup: int, shards: int, x_host=None):
    """One device's share of the headline scan split into `shards` contiguous
    shards (2^28 / shards fp32 elements, exclusive, in place), cold caches:
      reduce     the shard's total (dws_reduce; 4 bytes per element read)
      seeded     the shard's scan seeded with a device element (8 bytes)
      unseeded   scan_exclusive of the same shard, for comparison
      sequence   reduce, exclusive scan of the `shards` totals, seeded scan:
                 what each device runs besides the exchange of the totals
                 (12 bytes per element, ~3n/G per device)
      torch_sum  torch.sum of the shard (the library reduction), for comparison
    One SHARD line on stderr."""
    import torch
    import device_wide_prefix_amd as dws
    w = wl.WORKLOADS["f32_2p28_excl_inplace"]
    m = w.n // shards
    x = (wl.generate_workload(w) if x_host is None else x_host)[:m].copy()
    pristine = torch.from_numpy(x).to("cuda")
    work = torch.empty_like(pristine)
    totals = torch.zeros(shards, dtype=torch.float32, device="cuda")
    offsets = torch.zeros_like(totals)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    dws.reserve(m)

    def prepare():
        work.copy_(pristine)
        flush.sum()

    def ok(st):
        if st != dws.OK:
            raise RuntimeError(dws.status_string(st))

    def reduce():
        ok(dws.reduce_ptr(work.data_ptr(), m, dws.FLOAT32, totals.data_ptr(), stream))

    def seeded():
        ok(dws.scan_seeded_ptr(work.data_ptr(), work.data_ptr(), m, dws.FLOAT32, True, offsets.data_ptr(), stream))

    def unseeded():
        ok(dws.scan_exclusive_ptr(work.data_ptr(), work.data_ptr(), m, dws.FLOAT32, stream))

    def sequence():
        reduce()
        ok(dws.scan_exclusive_ptr(totals.data_ptr(), offsets.data_ptr(), shards, dws.FLOAT32, stream))
        seeded()

    def torch_sum():
        torch.sum(work, 0, out=totals[:1].view(()))

    row = {"workload": f"{w.description}, one of {shards} shards", "shards": shards, "n": m}
    trips = dws.watchdog_trips()
    for name, fn, per_elem in (("reduce", reduce, 4), ("seeded", seeded, 8), ("unseeded", unseeded, 8),
                               ("torch_sum", torch_sum, 4), ("sequence", sequence, 12)):
        times = time_steps(fn, prepare, steps, warmup)
        mean = float(np.mean(times))
        gbps = per_elem * m / (mean * 1e-3) / 1e9
        row[name] = {"us_mean": round(mean * 1e3, 3), "us_min": round(float(np.min(times)) * 1e3, 3),
                     "bytes_per_element": per_elem, "gbps": round(gbps, 1),
                     "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    # the last timed step ran the whole sequence on the shard: its total and
    # the ends of its seeded scan agree with a float64 sum (offsets[0], the
    # seed of the first shard, is 0)
    sequence_out = work.cpu().numpy()
    total = float(totals[0].item())
    ref = float(np.sum(x, dtype=np.float64))
    bound = 1e-4 * float(np.sum(np.abs(x), dtype=np.float64)) + 1e-6
    seed0 = float(offsets[0].item())
    row["property_check"] = bool(abs(total - ref) <= bound and seed0 == 0.0 and sequence_out[0] == 0.0
                                 and abs(float(sequence_out[-1]) + float(x[-1]) - ref) <= bound)
    row["watchdog_trips"] = int(dws.watchdog_trips() - trips)
    log("SHARD " + json.dumps(row))
    del pristine, work, flush
    torch.cuda.empty_cache()
    return row


COMPACTION_N = 1 << 25   # the 32M-item size the pages measure the compaction family on


def run_compaction(steps: int, warmup: int, with_oracle: bool = True):
    """Select, partition, reduce-by-key (int32 and fp32 values) and run-length
    encoding on 2^25 items, cold caches, each beside the nearest PyTorch
    equivalent on the same data. GB/s counts the algorithmic bytes: select
    8n + 4 count, partition 12n, reduce-by-key 8n + 8 runs, run-length encoding
    4n + 8 runs. One COMPACTION line per case on stderr."""
    import torch
    import device_wide_prefix_amd as dws
    n = COMPACTION_N
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    dws.reserve(n)
    lib = dws.load_library()

    def prepare():
        flush.sum()

    def emit(name, ms, algo_bytes, torch_ms, ok, extra, oracle_call=None):
        row = {"op": name, "n": n, "ms_mean": ms, "gbps": algo_bytes / (ms * 1e-3) / 1e9,
               "frac_hbm_peak": algo_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "torch_ms_mean": torch_ms,
               "speedup_vs_torch": (torch_ms / ms) if torch_ms else None, "property_check": bool(ok), **extra}
        if with_oracle and oracle_call is not None:
            row["cpu_baseline"] = oracle_rate(oracle_call, algo_bytes, "the same input, whole")
        log("COMPACTION " + json.dumps(row))

    if with_oracle:
        import oracle
    x_h = wl.generate("i32_full", n, 21)
    flags_h = wl.generate("flags_half", n, 22)
    x = torch.from_numpy(x_h).cuda()
    flags = torch.from_numpy(flags_h).cuda()
    mask = flags != 0
    out = torch.empty_like(x)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    for name, fn in (("select_flagged", lib.dws_select_flagged), ("partition_flagged", lib.dws_partition_flagged)):
        def run(fn=fn):
            st = fn(x.data_ptr(), flags.data_ptr(), out.data_ptr(), n, dws.INT32, cnt.data_ptr(), stream)
            if st != dws.OK:
                raise RuntimeError(f"{name}: {dws.status_string(st)}")
        ms = float(np.mean(time_steps(run, prepare, steps, warmup)))
        c = int(cnt.item())
        ok = c == int(mask.sum().item()) and torch.equal(out[:c], x[mask])
        if name == "partition_flagged":
            ok = ok and torch.equal(out[c:], x[~mask].flip(0))
            t = float(np.mean(time_steps(lambda: torch.cat((x[mask], x[~mask].flip(0))), prepare, steps, warmup)))
            emit(name, ms, 12 * n, t, ok, {"selected": c, "torch": "cat(x[mask], x[~mask].flip(0))"},
                 (lambda: oracle.partition_flagged(x_h, flags_h)) if with_oracle else None)
        else:
            t = float(np.mean(time_steps(lambda: torch.masked_select(x, mask), prepare, steps, warmup)))
            emit(name, ms, 8 * n + 4 * c, t, ok, {"selected": c, "torch": "masked_select"},
                 (lambda: oracle.select_flagged(x_h, flags_h)) if with_oracle else None)
    del x, flags, mask, out, x_h, flags_h
    vals_h = wl.generate("i32_full", n, 23)
    fvals_h = wl.generate("f32_pm1", n, 25)
    vals = torch.from_numpy(vals_h).cuda()
    fvals = torch.from_numpy(fvals_h).cuda()
    uk = torch.empty(n, dtype=torch.int32, device="cuda")
    ag = torch.empty(n, dtype=torch.int32, device="cuda")
    for mean_run in (1, 16):
        keys_h = wl.run_keys(n, mean_run, 24)
        keys = torch.from_numpy(keys_h.view(np.int32)).cuda()
        ref_keys, inverse, counts = torch.unique_consecutive(keys, return_inverse=True, return_counts=True)
        runs = ref_keys.numel()

        def rbk():
            st = lib.dws_reduce_by_key(keys.data_ptr(), vals.data_ptr(), uk.data_ptr(), ag.data_ptr(), n,
                                       dws.INT32, cnt.data_ptr(), stream)
            if st != dws.OK:
                raise RuntimeError(dws.status_string(st))

        def rle():
            st = lib.dws_run_length_encode(keys.data_ptr(), uk.data_ptr(), ag.data_ptr(), n, cnt.data_ptr(), stream)
            if st != dws.OK:
                raise RuntimeError(dws.status_string(st))

        def torch_rbk():
            k, inv = torch.unique_consecutive(keys, return_inverse=True)
            torch.zeros(k.numel(), dtype=torch.int64, device="cuda").index_add_(0, inv, vals.long())

        ms = float(np.mean(time_steps(rbk, prepare, steps, warmup)))
        want = torch.zeros(runs, dtype=torch.int64, device="cuda").index_add_(0, inverse, vals.long())
        want = (want & 0xFFFFFFFF).to(torch.int64)
        ok = int(cnt.item()) == runs and torch.equal(uk[:runs], ref_keys) and \
            torch.equal(ag[:runs].to(torch.int64) & 0xFFFFFFFF, want)
        t = float(np.mean(time_steps(torch_rbk, prepare, steps, warmup)))
        emit("reduce_by_key", ms, 8 * n + 8 * runs, t, ok,
             {"mean_run": mean_run, "runs": runs, "torch": "unique_consecutive + index_add_"},
             (lambda: oracle.reduce_by_key(keys_h, vals_h)) if with_oracle else None)

        def rbk_f32():
            st = lib.dws_reduce_by_key(keys.data_ptr(), fvals.data_ptr(), uk.data_ptr(), ag.data_ptr(), n,
                                       dws.FLOAT32, cnt.data_ptr(), stream)
            if st != dws.OK:
                raise RuntimeError(dws.status_string(st))

        def torch_rbk_f32():
            k, inv = torch.unique_consecutive(keys, return_inverse=True)
            torch.zeros(k.numel(), dtype=torch.float32, device="cuda").index_add_(0, inv, fvals)

        ms = float(np.mean(time_steps(rbk_f32, prepare, steps, warmup)))
        # fp32 sums within 1e-4 * (sum of |value| over the run) + 1e-6 of the fp64 sums
        want = torch.zeros(runs, dtype=torch.float64, device="cuda").index_add_(0, inverse, fvals.double())
        scale = torch.zeros(runs, dtype=torch.float64, device="cuda").index_add_(0, inverse, fvals.double().abs())
        got = ag[:runs].view(torch.float32).double()
        ok = int(cnt.item()) == runs and torch.equal(uk[:runs], ref_keys) and \
            bool(((got - want).abs() <= 1e-4 * scale + 1e-6).all())
        t = float(np.mean(time_steps(torch_rbk_f32, prepare, steps, warmup)))
        emit("reduce_by_key_f32", ms, 8 * n + 8 * runs, t, ok,
             {"mean_run": mean_run, "runs": runs, "torch": "unique_consecutive + index_add_ (fp32)"},
             (lambda: oracle.reduce_by_key(keys_h, fvals_h)) if with_oracle else None)
        del want, scale, got
        ms = float(np.mean(time_steps(rle, prepare, steps, warmup)))
        ok = int(cnt.item()) == runs and torch.equal(uk[:runs], ref_keys) and \
            torch.equal(ag[:runs].to(torch.int64), counts)
        t = float(np.mean(time_steps(lambda: torch.unique_consecutive(keys, return_counts=True), prepare, steps,
                                     warmup)))
        emit("run_length_encode", ms, 4 * n + 8 * runs, t, ok,
             {"mean_run": mean_run, "runs": runs, "torch": "unique_consecutive(return_counts=True)"},
             (lambda: oracle.run_length_encode(keys_h)) if with_oracle else None)
        del keys, ref_keys, inverse, counts, keys_h
    del vals, fvals, uk, ag, flush, vals_h, fvals_h
    torch.cuda.empty_cache()


def device_info():
    """Name, compute units, memory clock and bus width as the runtime reports
    them, and the bandwidth those imply, beside the published 8 TB/s used as
    the roofline peak. HBM3E moves 4 bits per pin per reported memory clock
    (8 Gb/s per pin at 2 GHz), so the implied figure is 4 x clock x width."""
    import torch
    import device_wide_prefix_amd as dws
    m = dws.device_memory_info()
    implied = 4.0 * m["memory_clock_khz"] * 1e3 * m["memory_bus_width_bits"] / 8 / 1e9
    return {"name": torch.cuda.get_device_properties(0).name, "arch": torch.cuda.get_device_properties(0).gcnArchName,
            **m, "implied_peak_gbps": round(implied, 1), "roofline_peak_gbps": HBM_PEAK_GBPS}


def cpu_model() -> str:
    """The host CPU's model name as the kernel reports it, or "unknown"."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: wl.Workload, x: np.ndarray, budget_s: float = 10.0):
    """The sequential oracle on the same input, timed on one host core, repeated
    until about budget_s seconds of CPU work (the oracle is one loop: 1 thread)."""
    import oracle
    reps = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if w.dtype == "float32":
            oracle.scan_f32(x, exclusive=w.exclusive, want_sabs=False)
        else:
            oracle.scan_u32(x, exclusive=w.exclusive)
        reps.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s or len(reps) >= 50:
            break
    med = float(np.median(reps))
    return {"value": round(w.algorithmic_bytes / med / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full {w.name} input (N={w.n}), {len(reps)} repetitions, median "
                      f"{med * 1e3:.1f} ms; host has {os.cpu_count()} logical CPUs ({cpu_model()})"}


def oracle_rate(call, algo_bytes: int, sample: str, budget_s: float = 2.0):
    """The oracle's rate on one bounded sample: call() repeated until about
    budget_s seconds of CPU work (at least once), median time, the same
    algorithmic-bytes convention as the GPU row it stands beside. The oracle
    is one sequential loop, so one host core."""
    reps = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        call()
        reps.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s or len(reps) >= 20:
            break
    med = float(np.median(reps))
    return {"gbps": round(algo_bytes / med / 1e9, 3), "ms": round(med * 1e3, 2), "cores": 1, "kind": "oracle",
            "repetitions": len(reps), "sample": sample}


def traffic_for_current_kernel():
    """HBM bytes per launch from the stored rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


def summarize(w, res, variant_name, args):
    times = res["times_ms"]
    mean_ms = float(np.mean(times))
    gbps = w.algorithmic_bytes / (mean_ms * 1e-3) / 1e9
    out = {"workload": w.name, "variant": variant_name, "ms_mean": mean_ms, "ms_min": float(np.min(times)),
           "ms_median": float(np.median(times)), "gbps": gbps, "property_check": res["property_check"],
           "watchdog_trips": res["watchdog_trips"]}
    for key in ("lookback_stall_share", "phase_mean_us", "tiles", "launch"):
        if key in res:
            out[key] = res[key]
    if "memcpy_times_ms" in res:
        mc = float(np.mean(res["memcpy_times_ms"]))
        out["memcpy_ms_mean"] = mc
        out["memcpy_gbps"] = w.algorithmic_bytes / (mc * 1e-3) / 1e9
    if "torch_cumsum_times_ms" in res:
        tc = float(np.mean(res["torch_cumsum_times_ms"]))
        out["torch_cumsum_ms_mean"] = tc
        out["torch_cumsum_gbps"] = w.algorithmic_bytes / (tc * 1e-3) / 1e9
    return out


# the five workloads the metric is stated on, in order; the one that fits the
# headline metric (2^28 fp32) is the bench line's value, the others ride along
CONFIG_ORDER = ("i32_4096_incl", "f32_2p20_incl", "u32_2p26_incl", "f32_2p28_excl_inplace",
                "flags_2p30m12345_excl")


def oracle_scan_call(w: wl.Workload, x: np.ndarray):
    import oracle
    if w.dtype == "float32":
        return lambda: oracle.scan_f32(x, exclusive=w.exclusive, want_sabs=False)
    return lambda: oracle.scan_u32(x, exclusive=w.exclusive)


def config_row(w: wl.Workload, s: dict, oracle_row) -> dict:
    """One entry of the bench line's `configs`: the workload's scan through the
    default entry point, cold caches, against a same-run memcpy of the same
    bytes, with the oracle's rate beside it."""
    mean_ms = s["ms_mean"]
    gbps = w.algorithmic_bytes / (mean_ms * 1e-3) / 1e9
    row = {"workload": w.name, "description": w.description, "n": w.n, "element": w.dtype,
           "scan": "exclusive" if w.exclusive else "inclusive", "in_place": w.in_place,
           "us_mean": round(mean_ms * 1e3, 3), "us_median": round(s["ms_median"] * 1e3, 3),
           "us_min": round(s["ms_min"] * 1e3, 3), "gbps": round(gbps, 2),
           "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "memcpy_gbps": round(s["memcpy_gbps"], 2), "frac_memcpy": round(gbps / s["memcpy_gbps"], 4),
           "property_check": s["property_check"], "watchdog_trips": s["watchdog_trips"],
           "launch": s.get("launch")}
    if oracle_row is not None:
        row["oracle"] = oracle_row
    return row


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="f32_2p28_excl_inplace", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--variant", default="single_pass", choices=sorted(VARIANTS))
    ap.add_argument("--order", default="relaxed", choices=sorted(ORDERS))
    ap.add_argument("--tile-shape", type=int, default=0)
    ap.add_argument("--nontemporal", default="auto", choices=sorted(NONTEMPORAL),
                    help="non-temporal loads: the library's choice (on from 2^23 elements), on or off")
    ap.add_argument("--tile-index", default="auto", choices=sorted(TILE_INDEX))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="measure only the headline workload (no `configs` rows, no `shard_8`)")
    ap.add_argument("--all", action="store_true", help="also measure every workload and variant (stderr)")
    ap.add_argument("--sweep", action="store_true",
                    help="also sweep N = 2^10..2^30 for every variant against memcpy (stderr)")
    ap.add_argument("--select", action="store_true",
                    help="also measure stream compaction on the 2^30-12345 flag workload (stderr)")
    ap.add_argument("--ops", action="store_true",
                    help="also measure the generic-operator scans on 1 GiB inputs (stderr)")
    ap.add_argument("--shards", type=int, default=0,
                    help="also time one device's share of the headline scan split into this many shards: "
                         "reduce, seeded scan and the two together (stderr)")
    ap.add_argument("--compaction", action="store_true",
                    help="also measure select, partition, reduce-by-key and run-length encoding on 2^25 items "
                         "(stderr)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported. The scan runs on a single "
              "device; across GPUs each would scan its shard seeded by an exchange of the shard totals, "
              "which is not built here.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import device_wide_prefix_amd as dws
    dws.load_library()

    w = wl.WORKLOADS[args.workload]
    log(f"generating {w.description}")
    x = wl.generate_workload(w)
    variant = VARIANTS[args.variant]
    res = run_workload(w, variant, ORDERS[args.order], args.tile_shape, NONTEMPORAL[args.nontemporal], args.steps,
                       args.warmup, with_memcpy=True, x_host=x, tile_index=TILE_INDEX[args.tile_index])
    s = summarize(w, res, args.variant, args)
    log(json.dumps(s))
    if not s["property_check"]:
        log("WARNING: property check of the scan output failed")

    mean_ms = s["ms_mean"]
    achieved = w.algorithmic_bytes / (mean_ms * 1e-3) / 1e9
    traffic = traffic_for_current_kernel() if (variant == 0 and args.workload == "f32_2p28_excl_inplace" and args.order == "relaxed"
                                               and args.tile_shape == 0 and args.nontemporal == "auto"
                                               and args.tile_index == "auto") else None
    line = {
        "metric": METRIC,
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"float32": "f32", "int32": "int32", "uint32": "uint32"}[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.description, "n": w.n, "element": w.dtype,
                   "scan": "exclusive" if w.exclusive else "inclusive", "in_place": w.in_place,
                   "seed": w.seed, "variant": args.variant, "memory_order": args.order,
                   "tile_shape": args.tile_shape, "nontemporal": args.nontemporal,
                   "tile_index": args.tile_index,
                   "parallelism": "single GPU"},
        "frac_hbm_peak": round(achieved / HBM_PEAK_GBPS, 4),
        "memcpy_gbps": round(s["memcpy_gbps"], 2),
        "frac_memcpy": round(achieved / s["memcpy_gbps"], 4),
        "library_baseline": ({"name": "torch.cumsum (hipCUB / rocPRIM device scan, inclusive, out of place)",
                              "gbps": round(s["torch_cumsum_gbps"], 2),
                              "ms_mean": round(s["torch_cumsum_ms_mean"], 5),
                              "speedup": round(s["torch_cumsum_ms_mean"] / mean_ms, 3)}
                             if "torch_cumsum_gbps" in s else None),
        "ms_min": round(s["ms_min"], 5),
        "ms_median": round(s["ms_median"], 5),
        "property_check": s["property_check"],
        "watchdog_trips": s["watchdog_trips"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "launch": s.get("launch"),
        "lookback_stall_share": s.get("lookback_stall_share"),
        "tile_phase_mean_us": s.get("phase_mean_us"),
        "device": device_info(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(w, x)

    if not args.headline_only:
        # every configuration of the metric, each through the default entry
        # point with cold caches, its same-run memcpy and the oracle's rate
        rows = []
        for name in CONFIG_ORDER:
            wk = wl.WORKLOADS[name]
            if name == args.workload and variant == 0 and args.tile_shape == 0 and args.order == "relaxed" \
                    and args.nontemporal == "auto" and args.tile_index == "auto":
                sk, xk = s, x
            else:
                log(f"config {name}: generating")
                xk = wl.generate_workload(wk)
                rk = run_workload(wk, 0, 0, 0, 0, args.steps, args.warmup, with_memcpy=True, x_host=xk,
                                  instrument=False, with_library=False)
                sk = summarize(wk, rk, "single_pass", args)
            orow = None
            if not args.no_cpu_baseline:
                orow = oracle_rate(oracle_scan_call(wk, xk), wk.algorithmic_bytes, "the whole input",
                                   budget_s=1.0)
            rows.append(config_row(wk, sk, orow))
            log("CONFIG " + json.dumps(rows[-1]))
            del xk
        line["configs"] = rows
        line["property_check"] = bool(line["property_check"] and all(r["property_check"] for r in rows))
        # one device's share of the headline split 8 ways: the per-device steps
        # of the sharded scan (the exchange of the totals is not a device's work)
        sh = run_shards(args.steps, args.warmup, 8, x_host=x if args.workload == "f32_2p28_excl_inplace" else None)
        line["shard_8"] = sh
        line["property_check"] = bool(line["property_check"] and sh["property_check"] and sh["watchdog_trips"] == 0)

    if args.all:
        for name in ("i32_4096_incl", "f32_2p20_incl", "u32_2p26_incl", "f32_2p28_excl_inplace", "flags_2p30m12345_excl"):
            wk = wl.WORKLOADS[name]
            xk = wl.generate_workload(wk)
            for vname, v in VARIANTS.items():
                r = run_workload(wk, v, 0, 0, 0, max(5, args.steps // 2), 3, with_memcpy=(v == 0), x_host=xk)
                log("ALL " + json.dumps(summarize(wk, r, vname, args)))
            del xk

    if args.sweep:
        run_sweep(max(5, args.steps // 2), 3)
    timed_oracle = not args.no_cpu_baseline
    if args.ops:
        run_ops(args.steps, args.warmup, timed_oracle)
    if args.compaction:
        run_compaction(args.steps, args.warmup, timed_oracle)
    if args.shards and (args.headline_only or args.shards != 8):
        run_shards(args.steps, args.warmup, args.shards)
    if args.select:
        for in_place in (False, True):
            log("SELECT " + json.dumps(run_select(args.steps, args.warmup, in_place, timed_oracle and not in_place)))

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

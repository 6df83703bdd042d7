"""Host-side checks of the C ABI: the library loads, exports every function the
public header declares, and rejects bad arguments before any HIP call (so these
run without a GPU; no scan is computed here)."""
import ctypes
import os
import re

import pytest

import device_wide_prefix_amd as dws

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dws_scan.h")


def declared_functions():
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dws.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return dws.load_library()


def _prototype(text: str, name: str) -> str:
    """The declaration of `name` in the header, comments dropped and
    whitespace collapsed: 'ret name(type a, type b)'."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    m = re.search(r"^([A-Za-z_][\w \t\*]*?\b" + name + r"\s*\([^;]*\))\s*;", text, flags=re.M)
    assert m, f"{name} not declared"
    return " ".join(m.group(1).replace("(", " ( ").replace(")", " ) ").replace(",", " , ").replace("*", " * ").split())


def _enum_values(text: str, enum: str) -> dict:
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    m = re.search(r"typedef enum " + enum + r"\s*\{(.*?)\}", text, flags=re.S)
    assert m, enum
    return {k: int(v) for k, v in re.findall(r"(\w+)\s*=\s*(-?\d+)", m.group(1))}


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("scan_inclusive", "scan_exclusive", "dws_scan_ex", "dws_status_string"):
        assert required in names
    assert set(names) == set(dws.EXPORTED_SYMBOLS)


def test_header_pins_the_boundary_signatures():
    """The four calls of the boundary with the argument lists, enum values and
    status numbering they are specified with; later additions (MISALIGNED,
    the pair types) are appended after them."""
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    want = {
        "scan_inclusive": "dws_status scan_inclusive ( const void * d_in , void * d_out , size_t n , "
                          "dws_dtype dtype , hipStream_t stream )",
        "scan_exclusive": "dws_status scan_exclusive ( const void * d_in , void * d_out , size_t n , "
                          "dws_dtype dtype , hipStream_t stream )",
        "dws_scan_ex": "dws_status dws_scan_ex ( const void * d_in , void * d_out , size_t n , dws_dtype dtype , "
                       "int exclusive , int variant , hipStream_t stream )",
        "dws_status_string": "const char * dws_status_string ( dws_status status )",
    }
    for name, proto in want.items():
        assert _prototype(text, name) == proto
    st = _enum_values(text, "dws_status")
    assert [st[k] for k in ("DWS_OK", "DWS_ERR_INVALID_ARG", "DWS_ERR_UNSUPPORTED", "DWS_ERR_OVERLAP",
                            "DWS_ERR_HIP", "DWS_ERR_OOM")] == [0, 1, 2, 3, 4, 5]
    assert st["DWS_ERR_MISALIGNED"] == 6
    dt = _enum_values(text, "dws_dtype")
    assert [dt[k] for k in ("DWS_INT32", "DWS_UINT32", "DWS_FLOAT32")] == [0, 1, 2]
    var = _enum_values(text, "dws_variant")
    assert [var[k] for k in ("DWS_VARIANT_SINGLE_PASS", "DWS_VARIANT_REDUCE_THEN_SCAN",
                             "DWS_VARIANT_CHAINED")] == [0, 1, 2]
    # the binding's constants are the header's
    assert (dws.OK, dws.ERR_INVALID_ARG, dws.ERR_UNSUPPORTED, dws.ERR_OVERLAP, dws.ERR_HIP, dws.ERR_OOM,
            dws.ERR_MISALIGNED) == (0, 1, 2, 3, 4, 5, 6)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared in dws_scan.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.dws_version() == 3
    for code in range(7):
        s = dws.status_string(code)
        assert isinstance(s, str) and s
    assert dws.status_string(0) == "ok"
    assert dws.status_string(99) == "unknown status"


def test_tile_geometry(lib):
    n_opts = dws.num_tile_shapes()
    assert n_opts >= 2
    # automatic choice by n
    for n, tile, threads in ((1 << 28, 65536, 1024), (1 << 24, 65536, 1024), ((1 << 24) - 1, 32768, 1024),
                             (1 << 23, 32768, 1024), ((1 << 23) - 1, 16384, 512), (1 << 20, 16384, 512),
                             ((1 << 20) - 1, 4096, 256), (1, 4096, 256)):
        assert dws.tile_elems(0, n, True) == tile, n
        assert dws.tile_threads(0, n, True) == threads, n
    # the scalar-load kernels keep the threads of their shape and at most 16
    # elements per lane
    for n in (1, 1 << 21, 1 << 23, 1 << 28):
        t = dws.tile_threads(0, n, True)
        assert dws.tile_threads(0, n, False) == t
        assert dws.tile_elems(0, n, False) == min(dws.tile_elems(0, n, True), 16 * t)
    for s in range(1, n_opts):
        e, t = dws.tile_elems(s, 1 << 28, True), dws.tile_threads(s, 1 << 28, True)
        assert e > 0 and t % 64 == 0 and e % (t * 4) == 0
        # unaligned: the scalar-load version of the forced shape, or of the
        # automatic shape when the forced one has none
        assert dws.tile_elems(s, 1 << 28, False) in (min(e, 16 * t), dws.tile_elems(0, 1 << 28, False))
    assert dws.tile_elems(n_opts, 100, True) == 0
    assert dws.tile_elems(-1, 100, True) == 0


FAKE = 0x10000  # never dereferenced: validation fails or passes before any HIP call


@pytest.mark.parametrize("fn", ["scan_inclusive", "scan_exclusive"])
def test_validation(lib, fn):
    f = getattr(lib, fn)
    # n == 0 is a no-op, even with null pointers
    assert f(None, None, 0, dws.INT32, None) == dws.OK
    assert f(None, FAKE, 10, dws.INT32, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, None, 10, dws.FLOAT32, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4096, 10, 7, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4096, 10, -1, None) == dws.ERR_INVALID_ARG
    assert f(FAKE + 2, FAKE + 4096, 10, dws.UINT32, None) == dws.ERR_MISALIGNED
    assert f(FAKE, FAKE + 4097, 10, dws.UINT32, None) == dws.ERR_MISALIGNED
    # partial overlap in either direction; exact aliasing is allowed (not run here)
    assert f(FAKE, FAKE + 4, 10, dws.INT32, None) == dws.ERR_OVERLAP
    assert f(FAKE + 36, FAKE, 10, dws.INT32, None) == dws.ERR_OVERLAP
    # too large
    assert f(FAKE, FAKE + (1 << 40), (1 << 35) + 1, dws.INT32, None) == dws.ERR_UNSUPPORTED
    # address range wraps around
    assert f(2**64 - 16, FAKE, 100, dws.INT32, None) == dws.ERR_INVALID_ARG


def test_option_validation(lib):
    def call(**kw):
        o = dws.DwsOptions(kw.get("variant", 0), kw.get("order", 0), kw.get("shape", 0), kw.get("nt", 0),
                           kw.get("tile_index", 0))
        return lib.dws_scan_opts(FAKE, FAKE + (1 << 20), 1 << 16, dws.FLOAT32, 1, ctypes.byref(o), None)
    assert call(variant=4) == dws.ERR_INVALID_ARG
    assert call(variant=-1) == dws.ERR_INVALID_ARG
    assert call(order=2) == dws.ERR_INVALID_ARG
    assert call(shape=dws.num_tile_shapes()) == dws.ERR_INVALID_ARG
    assert call(shape=-1) == dws.ERR_INVALID_ARG
    assert call(nt=3) == dws.ERR_INVALID_ARG
    assert call(nt=-1) == dws.ERR_INVALID_ARG
    # combinations that are not built
    # forced shapes 2 (256 x 32) and 4 (1024 x 16) are built for the relaxed
    # single pass only
    assert call(shape=2, order=dws.ORDER_ACQ_REL) == dws.ERR_UNSUPPORTED
    assert call(variant=dws.CHAINED, shape=4) == dws.ERR_UNSUPPORTED
    assert call(shape=4, nt=1) == dws.ERR_UNSUPPORTED
    assert call(variant=dws.REDUCE_THEN_SCAN, shape=1) == dws.ERR_UNSUPPORTED
    assert call(variant=dws.REDUCE_THEN_SCAN, nt=1) == dws.ERR_UNSUPPORTED
    assert call(variant=dws.SCAN_THEN_PROPAGATE, shape=1) == dws.ERR_UNSUPPORTED
    assert call(variant=dws.SCAN_THEN_PROPAGATE, nt=1) == dws.ERR_UNSUPPORTED
    # nontemporal 0 (the library's choice) and 2 (off) are valid everywhere;
    # with an unbuilt combination they still fail before any HIP call
    assert call(variant=dws.REDUCE_THEN_SCAN, nt=2, shape=1) == dws.ERR_UNSUPPORTED
    # tile index source: 0..2; dispatch order is built for the relaxed single
    # pass without non-temporal access
    assert call(tile_index=3) == dws.ERR_INVALID_ARG
    assert call(tile_index=-1) == dws.ERR_INVALID_ARG
    assert call(variant=dws.REDUCE_THEN_SCAN, tile_index=dws.TILE_DRAWN) == dws.ERR_UNSUPPORTED
    assert call(variant=dws.SCAN_THEN_PROPAGATE, tile_index=dws.TILE_DISPATCH) == dws.ERR_UNSUPPORTED
    assert call(variant=dws.CHAINED, tile_index=dws.TILE_DISPATCH) == dws.ERR_UNSUPPORTED
    assert call(tile_index=dws.TILE_DISPATCH, order=dws.ORDER_ACQ_REL) == dws.ERR_UNSUPPORTED
    assert call(tile_index=dws.TILE_DISPATCH, nt=1) == dws.ERR_UNSUPPORTED
    # options are validated before the arguments: n == 0 with bad options
    o = dws.DwsOptions(9, 0, 0, 0)
    assert lib.dws_scan_opts(None, None, 0, dws.INT32, 0, ctypes.byref(o), None) == dws.ERR_INVALID_ARG
    assert lib.dws_scan_opts(None, None, 0, dws.INT32, 0, None, None) == dws.OK


def test_variant_validation(lib):
    """dws_scan_ex takes the variant as a plain int: unknown values are
    rejected before any HIP call, known ones pass to argument validation."""
    f = lib.dws_scan_ex
    for bad in (4, -1, 1 << 20):
        assert f(FAKE, FAKE + (1 << 20), 1 << 16, dws.FLOAT32, 1, bad, None) == dws.ERR_INVALID_ARG
        assert f(None, None, 0, dws.INT32, 0, bad, None) == dws.ERR_INVALID_ARG
    for v in (dws.SINGLE_PASS, dws.REDUCE_THEN_SCAN, dws.CHAINED, dws.SCAN_THEN_PROPAGATE):
        assert f(None, None, 0, dws.INT32, 0, v, None) == dws.OK
        assert f(FAKE, FAKE + 4, 10, dws.INT32, 0, v, None) == dws.ERR_OVERLAP
        assert f(FAKE + 2, FAKE + 4096, 10, dws.UINT32, 1, v, None) == dws.ERR_MISALIGNED
        assert f(FAKE, FAKE + 4096, 10, 9, 1, v, None) == dws.ERR_INVALID_ARG


def test_debug_and_selftest_validation(lib):
    d = lib.dws_scan_debug
    assert d(FAKE, FAKE + 4096, 16, dws.INT32, 0, 0, 0, 0, 0, 0, None, None) == dws.ERR_INVALID_ARG
    assert d(FAKE, FAKE + 4096, 16, dws.INT32, 0, 0, 65, 0, 0, 0, None, None) == dws.ERR_INVALID_ARG
    assert d(FAKE, FAKE + 4096, 16, dws.INT32, 0, 1, 4, 0, 0, 0, None, None) == dws.ERR_INVALID_ARG
    assert d(FAKE, FAKE + 4096, 16, dws.INT32, 0, 0, 4, 3, 3, 0, None, None) == dws.ERR_INVALID_ARG
    assert d(FAKE, FAKE + 4096, 16, dws.INT32, 0, 0, 4, 0, 0, 10**9, None, None) == dws.ERR_INVALID_ARG
    assert d(FAKE, FAKE + 4, 16, dws.INT32, 0, 0, 4, 0, 0, 0, None, None) == dws.ERR_OVERLAP
    assert d(None, None, 0, dws.INT32, 0, 0, 4, 0, 0, 0, None, None) == dws.OK
    s = lib.dws_selftest_wave
    assert s(None, None, None, 0, dws.INT32, None) == dws.OK
    assert s(None, FAKE, FAKE, 1, dws.INT32, None) == dws.ERR_INVALID_ARG
    assert s(FAKE, FAKE, FAKE, 1, 5, None) == dws.ERR_INVALID_ARG
    assert lib.dws_watchdog_trips(None) == dws.ERR_INVALID_ARG
    assert lib.dws_device_memory_info(None, None, None) == dws.ERR_INVALID_ARG
    assert lib.dws_reserve((1 << 35) + 1, None) == dws.ERR_UNSUPPORTED


def test_profiled_size_query_and_validation(lib):
    # size query: no pointers, no HIP call
    assert dws.profiled_num_tiles(0) == 0
    assert dws.profiled_num_tiles(1) == 1
    assert dws.profiled_num_tiles(1 << 28) == (1 << 28) // dws.tile_elems(0, 1 << 28, True)
    assert dws.profiled_num_tiles((1 << 28) + 1) == (1 << 28) // dws.tile_elems(0, 1 << 28, True) + 1
    f = lib.dws_scan_profiled
    t = ctypes.c_uint(0)
    assert f(FAKE, FAKE + (1 << 20), 1 << 16, 9, 0, None, 0, ctypes.byref(t), None) == dws.ERR_INVALID_ARG
    # too small a stamp buffer, misaligned stamps, overlap, unaligned data
    tiles = dws.profiled_num_tiles(1 << 16)
    assert f(FAKE, FAKE + (1 << 20), 1 << 16, dws.INT32, 0, FAKE + (1 << 24), 5 * tiles - 1, None, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + (1 << 20), 1 << 16, dws.INT32, 0, FAKE + (1 << 24) + 4, 5 * tiles, None, None) == dws.ERR_MISALIGNED
    assert f(FAKE, FAKE + 4, 1 << 16, dws.INT32, 0, FAKE + (1 << 24), 5 * tiles, None, None) == dws.ERR_OVERLAP
    assert f(FAKE + 4, FAKE + (1 << 20), 1 << 16, dws.INT32, 0, FAKE + (1 << 24), 5 * tiles, None, None) == dws.ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    x = torch.arange(10, dtype=torch.int32)
    with pytest.raises(TypeError):
        dws.scan_inclusive(x)
    with pytest.raises(TypeError):
        dws.scan_exclusive(x.float())


def test_select_validation(lib):
    f = lib.dws_select_flagged
    cnt = FAKE + (1 << 24)
    n = 1000
    # bad dtype, missing or misaligned count word
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, 9, cnt, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, None, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, cnt + 4, None) == dws.ERR_MISALIGNED
    # null data pointers, misaligned elements
    assert f(None, FAKE + 8192, FAKE + 16384, n, dws.INT32, cnt, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, None, FAKE + 16384, n, dws.INT32, cnt, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 8192, None, n, dws.INT32, cnt, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 8194, FAKE + 16384, n, dws.INT32, cnt, None) == dws.ERR_MISALIGNED
    # flags overlapping the output (the flags must survive the writes)
    assert f(FAKE, FAKE + 8192, FAKE + 8192, n, dws.INT32, cnt, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + 8192, FAKE + 8192 + 400, n, dws.INT32, cnt, None) == dws.ERR_OVERLAP
    # partial overlap of input and output
    assert f(FAKE, FAKE + 16384, FAKE + 4, n, dws.INT32, cnt, None) == dws.ERR_OVERLAP
    # the count word inside the input, the flags or the output
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, FAKE + 8, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, FAKE + 8192 + 8, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, FAKE + 16384 + 3992, None) == dws.ERR_OVERLAP
    # counts travel in 32-bit descriptor values
    assert f(FAKE, FAKE + (1 << 36), FAKE + (2 << 36), 1 << 32, dws.INT32, cnt, None) == dws.ERR_UNSUPPORTED


def test_select_binding_checks_flags(lib):
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        dws.select_flagged(torch.arange(10, dtype=torch.int32), torch.ones(10, dtype=torch.int32))


def test_scan_op_validation(lib):
    f = lib.dws_scan_op
    big = FAKE + (1 << 24)
    # bad enums
    assert f(FAKE, big, 10, 5, dws.OP_MAX, 0, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, big, 10, -1, dws.OP_MAX, 0, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, big, 10, dws.INT32, 5, 0, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, big, 10, dws.INT32, -1, 0, None) == dws.ERR_INVALID_ARG
    # combinations that are not built
    assert f(FAKE, big, 10, dws.FLOAT32, dws.OP_MAX, 0, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE, big, 10, dws.PAIR_U32, dws.OP_MIN, 0, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE, big, 10, dws.INT32, dws.OP_AFFINE, 0, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE, big, 10, dws.PAIR_I32_F32, dws.OP_AFFINE, 0, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE, big, 10, dws.FLOAT32, dws.OP_SEGMENTED_SUM, 0, None) == dws.ERR_UNSUPPORTED
    # pointers: null, alignment to the element size, overlap, empty
    assert f(None, big, 10, dws.PAIR_U32, dws.OP_AFFINE, 0, None) == dws.ERR_INVALID_ARG
    assert f(FAKE + 4, big, 10, dws.PAIR_U32, dws.OP_AFFINE, 0, None) == dws.ERR_MISALIGNED
    assert f(FAKE, big + 4, 10, dws.PAIR_I32_F32, dws.OP_SUM, 0, None) == dws.ERR_MISALIGNED
    assert f(FAKE + 2, big, 10, dws.INT32, dws.OP_MAX, 0, None) == dws.ERR_MISALIGNED
    assert f(FAKE, FAKE + 8, 10, dws.PAIR_U32, dws.OP_SEGMENTED_SUM, 0, None) == dws.ERR_OVERLAP
    assert f(FAKE + 72, FAKE, 10, dws.PAIR_U32, dws.OP_SEGMENTED_SUM, 0, None) == dws.ERR_OVERLAP
    assert f(None, None, 0, dws.PAIR_U32, dws.OP_AFFINE, 1, None) == dws.OK
    assert f(FAKE, big, (1 << 35) + 1, dws.PAIR_U32, dws.OP_AFFINE, 0, None) == dws.ERR_UNSUPPORTED
    # + on the 32-bit types is the plain scan, with its checks
    assert f(FAKE, FAKE + 4, 10, dws.INT32, dws.OP_SUM, 0, None) == dws.ERR_OVERLAP
    assert f(None, None, 0, dws.FLOAT32, dws.OP_SUM, 0, None) == dws.OK


def test_scan_op_binding_checks(lib):
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        dws.scan_op(torch.zeros((4, 2), dtype=torch.int32), dws.OP_AFFINE, dws.PAIR_U32)


def test_partition_validation(lib):
    f = lib.dws_partition_flagged
    cnt = FAKE + (1 << 24)
    n = 1000
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, 9, cnt, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, None, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, cnt + 4, None) == dws.ERR_MISALIGNED
    # never in place: the output must not overlap the input
    assert f(FAKE, FAKE + 8192, FAKE, n, dws.INT32, cnt, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + 8192, FAKE + 16384, n, dws.INT32, FAKE + 16384 + 8, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + 8192, FAKE + 8192, n, dws.INT32, cnt, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + (1 << 36), FAKE + (2 << 36), 1 << 32, dws.INT32, cnt, None) == dws.ERR_UNSUPPORTED


def test_reduce_by_key_and_rle_validation(lib):
    r = lib.dws_reduce_by_key
    e = lib.dws_run_length_encode
    K, V, UK, AG, C = FAKE, FAKE + 8192, FAKE + 16384, FAKE + 24576, FAKE + (1 << 24)
    n = 1000
    assert r(K, V, UK, AG, n, 7, C, None) == dws.ERR_INVALID_ARG
    assert r(K, V, UK, AG, n, dws.INT32, None, None) == dws.ERR_INVALID_ARG
    assert r(K, V, UK, AG, n, dws.INT32, C + 4, None) == dws.ERR_MISALIGNED
    assert r(None, V, UK, AG, n, dws.INT32, C, None) == dws.ERR_INVALID_ARG
    assert r(K, V, UK, None, n, dws.FLOAT32, C, None) == dws.ERR_INVALID_ARG
    assert r(K + 2, V, UK, AG, n, dws.INT32, C, None) == dws.ERR_MISALIGNED
    # no output may overlap an input, the other output or the count word
    assert r(K, V, K, AG, n, dws.INT32, C, None) == dws.ERR_OVERLAP
    assert r(K, V, UK, V + 400, n, dws.INT32, C, None) == dws.ERR_OVERLAP
    assert r(K, V, UK, UK + 40, n, dws.INT32, C, None) == dws.ERR_OVERLAP
    assert r(K, V, UK, AG, n, dws.INT32, UK + 8, None) == dws.ERR_OVERLAP
    assert r(K, V, UK, AG, n, dws.INT32, K + 8, None) == dws.ERR_OVERLAP
    assert r(K, V, UK, AG, 1 << 32, dws.INT32, C + (1 << 40), None) == dws.ERR_UNSUPPORTED
    assert e(K, UK, AG, n, None, None) == dws.ERR_INVALID_ARG
    assert e(K, K + 3996, AG, n, C, None) == dws.ERR_OVERLAP
    assert e(K, UK, UK, n, C, None) == dws.ERR_OVERLAP
    assert e(K + 1, UK, AG, n, C, None) == dws.ERR_MISALIGNED


def test_noalloc_validation_and_limit(lib):
    """dws_scan_noalloc: the scans' argument checks, and the size limit of its
    fixed array, all before any HIP call."""
    f = lib.dws_scan_noalloc
    assert f(None, None, 0, dws.INT32, 0, None) == dws.OK
    assert f(None, FAKE, 10, dws.INT32, 1, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4096, 10, 7, 0, None) == dws.ERR_INVALID_ARG
    assert f(FAKE + 2, FAKE + 4096, 10, dws.UINT32, 0, None) == dws.ERR_MISALIGNED
    assert f(FAKE, FAKE + 4, 10, dws.INT32, 0, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + (1 << 40), (1 << 35) + 1, dws.INT32, 0, None) == dws.ERR_UNSUPPORTED
    # one descriptor per tile, DWS_NOALLOC_MAX_TILES of them: 65,536-element
    # tiles with 16-byte aligned pointers, 16,384 otherwise
    max_tiles = 65536
    big = FAKE + (1 << 36)
    assert dws.tile_elems(0, max_tiles * 65536, True) == 65536
    assert f(FAKE, big, max_tiles * 65536 + 1, dws.FLOAT32, 1, None) == dws.ERR_UNSUPPORTED
    assert dws.tile_elems(0, max_tiles * 16384, False) == 16384
    assert f(FAKE + 4, big, max_tiles * 16384 + 1, dws.FLOAT32, 1, None) == dws.ERR_UNSUPPORTED


def test_scan_seeded_validation(lib):
    """dws_scan_seeded: the scans' argument checks, then the seed's, all before
    any HIP call."""
    f = lib.dws_scan_seeded
    seed = FAKE + (1 << 41)
    # n == 0 is a no-op that reads nothing, even the seed
    assert f(None, None, 0, dws.INT32, 0, None, None) == dws.OK
    assert f(None, FAKE, 10, dws.INT32, 0, seed, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4096, 10, 7, 1, seed, None) == dws.ERR_INVALID_ARG
    assert f(FAKE + 2, FAKE + 4096, 10, dws.UINT32, 0, seed, None) == dws.ERR_MISALIGNED
    assert f(FAKE, FAKE + 4, 10, dws.INT32, 0, seed, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE + (1 << 40), (1 << 35) + 1, dws.INT32, 0, seed, None) == dws.ERR_UNSUPPORTED
    # the seed itself
    assert f(FAKE, FAKE + 4096, 10, dws.FLOAT32, 0, None, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4096, 10, dws.FLOAT32, 1, seed + 2, None) == dws.ERR_MISALIGNED
    # inside the output's n elements (first, last), in place or not
    out = FAKE + 4096
    assert f(FAKE, out, 10, dws.INT32, 0, out, None) == dws.ERR_OVERLAP
    assert f(FAKE, out, 10, dws.INT32, 0, out + 36, None) == dws.ERR_OVERLAP
    assert f(FAKE, FAKE, 10, dws.INT32, 1, FAKE + 8, None) == dws.ERR_OVERLAP
    # (a seed just outside the output, or inside an input that is not the
    # output, passes these checks: the GPU tests run such calls)


def test_scan_op_seeded_validation(lib):
    """dws_scan_op_seeded: dws_scan_op's checks, then the seed's, before any
    HIP call; + on a 32-bit scalar is dws_scan_seeded."""
    f = lib.dws_scan_op_seeded
    seed = FAKE + (1 << 41)
    assert f(None, None, 0, dws.PAIR_U32, dws.OP_AFFINE, 0, None, None) == dws.OK
    assert f(FAKE, FAKE + 4096, 10, 9, dws.OP_MAX, 0, seed, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4096, 10, dws.INT32, 7, 0, seed, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4096, 10, dws.FLOAT32, dws.OP_MAX, 0, seed, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE, FAKE + 4096, 10, dws.INT32, dws.OP_AFFINE, 0, seed, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE + 4, FAKE + 4096, 10, dws.PAIR_U32, dws.OP_AFFINE, 0, seed, None) == dws.ERR_MISALIGNED
    assert f(FAKE, FAKE + 8, 10, dws.PAIR_U32, dws.OP_AFFINE, 0, seed, None) == dws.ERR_OVERLAP
    for op, dt in ((dws.OP_MAX, dws.INT32), (dws.OP_SEGMENTED_SUM, dws.PAIR_I32_F32), (dws.OP_SUM, dws.UINT32)):
        esize = 4 if dt in (dws.INT32, dws.UINT32) else 8
        out = FAKE + 4096
        assert f(FAKE, out, 10, dt, op, 1, None, None) == dws.ERR_INVALID_ARG
        assert f(FAKE, out, 10, dt, op, 1, seed + 2, None) == dws.ERR_MISALIGNED
        # inside the output's 10 elements: first and last element
        assert f(FAKE, out, 10, dt, op, 0, out, None) == dws.ERR_OVERLAP
        assert f(FAKE, out, 10, dt, op, 0, out + 9 * esize, None) == dws.ERR_OVERLAP
        # an 8-byte seed that straddles the output's first byte
        if esize == 8:
            assert f(FAKE, out, 10, dt, op, 0, out - 4, None) == dws.ERR_OVERLAP


def test_reduce_op_validation(lib):
    """dws_reduce_op: argument checks before any HIP call; + on a 32-bit
    scalar is dws_reduce."""
    f = lib.dws_reduce_op
    total = FAKE + (1 << 41)
    assert f(FAKE, 10, 9, dws.OP_MAX, total, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, 10, dws.INT32, 7, total, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, 10, dws.FLOAT32, dws.OP_MAX, total, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE, 10, dws.UINT32, dws.OP_AFFINE, total, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE, 10, dws.PAIR_U32, dws.OP_AFFINE, None, None) == dws.ERR_INVALID_ARG
    assert f(None, 10, dws.PAIR_U32, dws.OP_AFFINE, total, None) == dws.ERR_INVALID_ARG
    assert f(None, 0, dws.PAIR_U32, dws.OP_AFFINE, None, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, (1 << 35) + 1, dws.PAIR_U32, dws.OP_SEGMENTED_SUM, total, None) == dws.ERR_UNSUPPORTED
    assert f(FAKE + 4, 10, dws.PAIR_U32, dws.OP_AFFINE, total, None) == dws.ERR_MISALIGNED
    assert f(FAKE, 10, dws.PAIR_I32_F32, dws.OP_SUM, total + 2, None) == dws.ERR_MISALIGNED
    assert f(FAKE + 2, 10, dws.INT32, dws.OP_MIN, total, None) == dws.ERR_MISALIGNED
    # the total inside the input's n elements (8-byte elements: 80 bytes)
    assert f(FAKE, 10, dws.PAIR_U32, dws.OP_AFFINE, FAKE + 72, None) == dws.ERR_OVERLAP
    assert f(FAKE, 10, dws.PAIR_U32, dws.OP_AFFINE, FAKE - 4, None) == dws.ERR_OVERLAP
    assert f(FAKE, 10, dws.INT32, dws.OP_SUM, FAKE + 36, None) == dws.ERR_OVERLAP


def test_select_if_validation(lib):
    """dws_select_if / dws_partition_if: the predicate and threshold checks,
    then those of the flagged calls, before any HIP call."""
    import numpy as np
    t = np.array([3], dtype=np.int32)
    tp = t.ctypes.data
    cnt = FAKE + (1 << 24)
    for f in (lib.dws_select_if, lib.dws_partition_if):
        assert f(FAKE, FAKE + 8192, 100, dws.INT32, 6, tp, cnt, None) == dws.ERR_INVALID_ARG
        assert f(FAKE, FAKE + 8192, 100, dws.INT32, -1, tp, cnt, None) == dws.ERR_INVALID_ARG
        assert f(FAKE, FAKE + 8192, 100, dws.INT32, dws.PRED_LT, None, cnt, None) == dws.ERR_INVALID_ARG
        assert f(FAKE, FAKE + 8192, 100, 7, dws.PRED_LT, tp, cnt, None) == dws.ERR_INVALID_ARG
        assert f(FAKE, FAKE + 8192, 100, dws.INT32, dws.PRED_LT, tp, None, None) == dws.ERR_INVALID_ARG
        assert f(FAKE, FAKE + 8192, 100, dws.INT32, dws.PRED_LT, tp, cnt + 4, None) == dws.ERR_MISALIGNED
        assert f(FAKE + 2, FAKE + 8192, 100, dws.FLOAT32, dws.PRED_GE, tp, cnt, None) == dws.ERR_MISALIGNED
        assert f(FAKE, FAKE + 4, 100, dws.UINT32, dws.PRED_EQ, tp, cnt, None) == dws.ERR_OVERLAP
        assert f(FAKE, FAKE + 8192, (1 << 32), dws.INT32, dws.PRED_NE, tp, cnt, None) == dws.ERR_UNSUPPORTED
        assert f(FAKE, FAKE + 8192, 100, dws.INT32, dws.PRED_NE, tp, FAKE + 200, None) == dws.ERR_OVERLAP
    # a partition is never in place
    assert lib.dws_partition_if(FAKE, FAKE, 100, dws.INT32, dws.PRED_LT, tp, cnt, None) == dws.ERR_OVERLAP


def test_reduce_validation(lib):
    """dws_reduce: argument checks before any HIP call."""
    f = lib.dws_reduce
    total = FAKE + (1 << 41)
    assert f(FAKE, 10, 7, total, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, 10, -1, total, None) == dws.ERR_INVALID_ARG
    assert f(FAKE, 10, dws.INT32, None, None) == dws.ERR_INVALID_ARG
    assert f(None, 10, dws.INT32, total, None) == dws.ERR_INVALID_ARG
    assert f(None, 0, dws.INT32, None, None) == dws.ERR_INVALID_ARG   # the total is written even for n == 0
    assert f(FAKE + 2, 10, dws.FLOAT32, total, None) == dws.ERR_MISALIGNED
    assert f(FAKE, 10, dws.FLOAT32, total + 1, None) == dws.ERR_MISALIGNED
    assert f(FAKE, (1 << 35) + 1, dws.UINT32, total, None) == dws.ERR_UNSUPPORTED
    # the total inside the input's n elements
    assert f(FAKE, 10, dws.INT32, FAKE, None) == dws.ERR_OVERLAP
    assert f(FAKE, 10, dws.INT32, FAKE + 36, None) == dws.ERR_OVERLAP
    # an input range that wraps the address space
    assert f(2**64 - 16, 100, dws.INT32, total, None) == dws.ERR_INVALID_ARG


def test_seeded_and_reduce_bindings_refuse_cpu_tensors(lib):
    import torch
    x = torch.zeros(8, dtype=torch.float32)
    with pytest.raises(TypeError):
        dws.reduce(x)
    with pytest.raises(TypeError):
        dws.scan_seeded(x, torch.zeros(1))


# ---------------------------------------------------------------------------
# the launch the library chooses (dws_scan_plan: no HIP call, no launch)
# ---------------------------------------------------------------------------
def _plan(lib, n, dtype=dws.FLOAT32, in_place=False, offset=0, exclusive=False, **kw):
    d_in = FAKE + offset
    d_out = d_in if in_place else d_in + (1 << 40)
    o = dws.DwsOptions(kw.get("variant", 0), kw.get("order", 0), kw.get("shape", 0), kw.get("nt", 0),
                       kw.get("tile_index", 0))
    return dws.scan_plan_ptr(d_in, d_out, n, dtype, exclusive, o)


def _auto_tile(n):
    """The automatic tile: (threads, elements) by n."""
    if n >= 1 << 24:
        return 1024, 65536
    if n >= 1 << 23:
        return 1024, 32768
    if n >= 1 << 20:
        return 512, 16384
    return 256, 4096


@pytest.mark.parametrize("in_place", [False, True], ids=["out_of_place", "in_place"])
def test_plan_automatic_policy(lib, in_place):
    # every size takes the workgroup index and the short pause; non-temporal
    # loads from 2^23 elements, in place or not
    for n in (1, 4096, 4097, (1 << 20) - 1, 1 << 20, (1 << 23) - 1, 1 << 23, (1 << 24) - 3, 1 << 24,
              (1 << 27) + 1, 1 << 28, (1 << 30) - 12345, 1 << 32):
        st, p = _plan(lib, n, in_place=in_place)
        assert st == dws.OK, n
        threads, tile = _auto_tile(n)
        assert (p.threads, p.tile_elems) == (threads, tile), n
        assert p.num_tiles == -(-n // tile), n
        assert p.tile_index == dws.TILE_DISPATCH, n
        assert p.nontemporal == (1 if n >= 1 << 23 else 0), n
        assert p.pause_units == 1, n


def test_plan_explicit_choices(lib):
    big = 1 << 28
    # a drawn index: the 64-unit back-off from 2^27, the short pause below it
    st, p = _plan(lib, big, tile_index=dws.TILE_DRAWN)
    assert st == dws.OK and (p.tile_index, p.nontemporal, p.pause_units) == (dws.TILE_DRAWN, 1, 64)
    st, p = _plan(lib, 1 << 26, tile_index=dws.TILE_DRAWN)
    assert st == dws.OK and (p.tile_index, p.nontemporal, p.pause_units) == (dws.TILE_DRAWN, 1, 1)
    # the chained scan and release/acquire descriptors always draw, without
    # non-temporal loads unless asked for
    for kw in (dict(variant=dws.CHAINED), dict(order=dws.ORDER_ACQ_REL)):
        st, p = _plan(lib, big, **kw)
        assert st == dws.OK and (p.tile_index, p.nontemporal) == (dws.TILE_DRAWN, 0), kw
    # non-temporal loads off; on for a small automatic shape (only its drawn
    # kernel has them); on with the workgroup index where it has them
    st, p = _plan(lib, big, nt=2)
    assert st == dws.OK and (p.tile_index, p.nontemporal) == (dws.TILE_DISPATCH, 0)
    st, p = _plan(lib, 1 << 16, nt=1)
    assert st == dws.OK and (p.tile_index, p.nontemporal, p.tile_elems) == (dws.TILE_DRAWN, 1, 4096)
    st, p = _plan(lib, 1 << 24, nt=1, tile_index=dws.TILE_DISPATCH)
    assert st == dws.OK and (p.tile_index, p.nontemporal) == (dws.TILE_DISPATCH, 1)
    assert _plan(lib, 1 << 16, nt=1, tile_index=dws.TILE_DISPATCH)[0] == dws.ERR_UNSUPPORTED
    # a forced shape does not take the automatic non-temporal loads
    st, p = _plan(lib, big, shape=5)
    assert st == dws.OK and (p.tile_elems, p.nontemporal, p.tile_index) == (32768, 0, dws.TILE_DISPATCH)
    # pointers that are not 16-byte aligned: scalar loads, 16 per lane, no
    # non-temporal loads
    st, p = _plan(lib, big, offset=4)
    assert st == dws.OK and (p.threads, p.tile_elems, p.nontemporal) == (1024, 16384, 0)


def test_plan_validation(lib):
    o = dws.DwsOptions(0, 0, 0, 0, 0)
    f = lib.dws_scan_plan
    assert f(FAKE, FAKE + (1 << 20), 100, dws.FLOAT32, 0, ctypes.byref(o), None) == dws.ERR_INVALID_ARG
    st, p = _plan(lib, 0)
    assert st == dws.OK and p.num_tiles == 0
    assert _plan(lib, 100, dtype=9)[0] == dws.ERR_INVALID_ARG
    assert _plan(lib, 100, offset=2)[0] == dws.ERR_MISALIGNED
    assert _plan(lib, 1 << 20, variant=dws.REDUCE_THEN_SCAN)[0] == dws.ERR_UNSUPPORTED
    assert _plan(lib, 1 << 20, variant=dws.SCAN_THEN_PROPAGATE)[0] == dws.ERR_UNSUPPORTED
    assert _plan(lib, 1 << 20, variant=7)[0] == dws.ERR_INVALID_ARG
    st = dws.scan_plan_ptr(FAKE, FAKE + 4, 100, dws.INT32, False)[0]
    assert st == dws.ERR_OVERLAP


def test_plan_agrees_with_the_profiled_scan(lib):
    # the instrumented scan sizes its stamp buffer by its own tile count
    for n in (5, 4097, (1 << 20) + 3, (1 << 23) + 1, (1 << 24) + 77, (1 << 28) + 5):
        st, p = _plan(lib, n)
        assert st == dws.OK
        assert p.num_tiles == dws.profiled_num_tiles(n), n

/*
 * Host sanitizer driver for the scan library's C ABI: tests/test_sanitizers.py
 * builds the library's host code with AddressSanitizer and
 * UndefinedBehaviorSanitizer (device code unchanged) and links this driver to
 * it. Every call here is answered on the host before any HIP call: argument
 * validation of each entry point (null pointers, bad enums and options,
 * misalignment, overlaps, sizes past the limits, n == 0), the status strings
 * and the tile-geometry queries. No GPU is needed and no memory is touched at
 * the fake addresses. A failed check or any sanitizer report fails the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dws_scan.h"

static int g_bad = 0;

#define CHECK(call, want)                                                                  \
    do {                                                                                   \
        const int got_ = (int)(call);                                                      \
        if (got_ != (int)(want)) {                                                         \
            fprintf(stderr, "FAIL line %d: %s = %d, want %d\n", __LINE__, #call, got_,      \
                    (int)(want));                                                          \
            g_bad = 1;                                                                     \
        }                                                                                  \
    } while (0)

static void* at(uint64_t addr) { return (void*)(uintptr_t)addr; }

#define FAKE 0x10000ull

static void status_and_geometry(void)
{
    CHECK(dws_version(), DWS_VERSION);
    for (int s = -3; s < 12; ++s) {
        const char* str = dws_status_string((dws_status)s);
        if (str == NULL || str[0] == '\0') {
            fprintf(stderr, "FAIL empty status string for %d\n", s);
            g_bad = 1;
        }
    }
    CHECK(strcmp(dws_status_string(DWS_OK), "ok"), 0);
    const int shapes = dws_num_tile_shapes();
    if (shapes < 2) g_bad = 1;
    const size_t sizes[] = {0, 1, 4095, 4096, 4097, (size_t)1 << 20, ((size_t)1 << 24) - 1, (size_t)1 << 28,
                            DWS_MAX_ELEMENTS, DWS_MAX_ELEMENTS + 1, SIZE_MAX};
    for (int s = -2; s <= shapes + 1; ++s)
        for (size_t k = 0; k < sizeof(sizes) / sizeof(sizes[0]); ++k)
            for (int al = 0; al < 2; ++al) {
                const unsigned e = dws_tile_elems(s, sizes[k], al);
                const unsigned t = dws_tile_threads(s, sizes[k], al);
                if ((s < 0 || s >= shapes) && (e != 0u || t != 0u)) {
                    fprintf(stderr, "FAIL shape %d gives a tile\n", s);
                    g_bad = 1;
                }
                if (s >= 0 && s < shapes && (e == 0u || t == 0u || t % 64u != 0u || e % t != 0u)) {
                    fprintf(stderr, "FAIL shape %d n %zu aligned %d: %u elements, %u threads\n", s, sizes[k],
                            al, e, t);
                    g_bad = 1;
                }
            }
}

static void scans(void)
{
    CHECK(scan_inclusive(NULL, NULL, 0, DWS_INT32, NULL), DWS_OK);
    CHECK(scan_exclusive(NULL, NULL, 0, DWS_FLOAT32, NULL), DWS_OK);
    CHECK(scan_inclusive(NULL, at(FAKE), 10, DWS_INT32, NULL), DWS_ERR_INVALID_ARG);
    CHECK(scan_exclusive(at(FAKE), NULL, 10, DWS_FLOAT32, NULL), DWS_ERR_INVALID_ARG);
    CHECK(scan_inclusive(at(FAKE), at(FAKE + 4096), 10, (dws_dtype)7, NULL), DWS_ERR_INVALID_ARG);
    CHECK(scan_inclusive(at(FAKE), at(FAKE + 4096), 10, (dws_dtype)-1, NULL), DWS_ERR_INVALID_ARG);
    CHECK(scan_inclusive(at(FAKE + 2), at(FAKE + 4096), 10, DWS_UINT32, NULL), DWS_ERR_MISALIGNED);
    CHECK(scan_exclusive(at(FAKE), at(FAKE + 4), 10, DWS_INT32, NULL), DWS_ERR_OVERLAP);
    CHECK(scan_exclusive(at(FAKE + 36), at(FAKE), 10, DWS_INT32, NULL), DWS_ERR_OVERLAP);
    CHECK(scan_inclusive(at(FAKE), at(FAKE + (1ull << 40)), DWS_MAX_ELEMENTS + 1, DWS_INT32, NULL),
          DWS_ERR_UNSUPPORTED);
    CHECK(scan_inclusive(at(UINT64_MAX - 15), at(FAKE), 100, DWS_INT32, NULL), DWS_ERR_INVALID_ARG);
    CHECK(scan_inclusive(at(FAKE), at(FAKE + 4096), SIZE_MAX, DWS_INT32, NULL), DWS_ERR_UNSUPPORTED);

    dws_options o;
    const int bad_opts[][5] = {{4, 0, 0, 0, 0}, {-1, 0, 0, 0, 0}, {0, 2, 0, 0, 0}, {0, 0, -1, 0, 0},
                               {0, 0, 0, 3, 0}, {0, 0, 0, -1, 0}, {0, 0, 0, 0, 3}, {0, 0, 0, 0, -1}};
    for (size_t k = 0; k < sizeof(bad_opts) / sizeof(bad_opts[0]); ++k) {
        o.variant = bad_opts[k][0];
        o.memory_order = bad_opts[k][1];
        o.tile_shape = bad_opts[k][2];
        o.nontemporal = bad_opts[k][3];
        o.tile_index = bad_opts[k][4];
        CHECK(dws_scan_opts(at(FAKE), at(FAKE + (1 << 20)), 1 << 16, DWS_FLOAT32, 1, &o, NULL), DWS_ERR_INVALID_ARG);
        CHECK(dws_scan_opts(NULL, NULL, 0, DWS_INT32, 0, &o, NULL), DWS_ERR_INVALID_ARG);
    }
    o.variant = 0;
    o.memory_order = 0;
    o.tile_shape = dws_num_tile_shapes();
    o.nontemporal = 0;
    o.tile_index = 0;
    CHECK(dws_scan_opts(at(FAKE), at(FAKE + (1 << 20)), 1 << 16, DWS_FLOAT32, 1, &o, NULL), DWS_ERR_INVALID_ARG);
    o.tile_shape = 0;
    o.variant = DWS_VARIANT_CHAINED;
    o.tile_index = DWS_TILE_DISPATCH;
    CHECK(dws_scan_opts(at(FAKE), at(FAKE + (1 << 20)), 1 << 16, DWS_FLOAT32, 1, &o, NULL), DWS_ERR_UNSUPPORTED);
    CHECK(dws_scan_opts(NULL, NULL, 0, DWS_INT32, 0, NULL, NULL), DWS_OK);
    /* the variant as a plain int */
    CHECK(dws_scan_ex(at(FAKE), at(FAKE + (1 << 20)), 1 << 16, DWS_FLOAT32, 1, 4, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_ex(at(FAKE), at(FAKE + (1 << 20)), 1 << 16, DWS_FLOAT32, 1, -1, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_ex(NULL, NULL, 0, DWS_INT32, 0, DWS_VARIANT_CHAINED, NULL), DWS_OK);
    CHECK(dws_scan_ex(at(FAKE), at(FAKE + 4), 10, DWS_INT32, 0, DWS_VARIANT_REDUCE_THEN_SCAN, NULL), DWS_ERR_OVERLAP);
}

static void compaction(void)
{
    const uint64_t cnt = FAKE + (1 << 24);
    const size_t n = 1000;
    CHECK(dws_select_flagged(at(FAKE), at(FAKE + 8192), at(FAKE + 16384), n, (dws_dtype)9, at(cnt), NULL),
          DWS_ERR_INVALID_ARG);
    CHECK(dws_select_flagged(at(FAKE), at(FAKE + 8192), at(FAKE + 16384), n, DWS_INT32, NULL, NULL),
          DWS_ERR_INVALID_ARG);
    CHECK(dws_select_flagged(at(FAKE), at(FAKE + 8192), at(FAKE + 16384), n, DWS_INT32, at(cnt + 4), NULL),
          DWS_ERR_MISALIGNED);
    CHECK(dws_select_flagged(at(FAKE), at(FAKE + 8192), at(FAKE + 8192 + 400), n, DWS_INT32, at(cnt), NULL),
          DWS_ERR_OVERLAP);
    CHECK(dws_select_flagged(at(FAKE), at(FAKE + 8192), at(FAKE + 16384), n, DWS_INT32, at(FAKE + 8), NULL),
          DWS_ERR_OVERLAP);
    CHECK(dws_select_flagged(at(FAKE), at(FAKE + (1ull << 36)), at(FAKE + (2ull << 36)), (size_t)1 << 32,
                             DWS_INT32, at(cnt), NULL),
          DWS_ERR_UNSUPPORTED);
    CHECK(dws_partition_flagged(at(FAKE), at(FAKE + 8192), at(FAKE), n, DWS_INT32, at(cnt), NULL),
          DWS_ERR_OVERLAP);
    CHECK(dws_partition_flagged(at(FAKE), at(FAKE + 8192), at(FAKE + 16384), n, DWS_INT32, NULL, NULL),
          DWS_ERR_INVALID_ARG);

    const uint64_t K = FAKE, V = FAKE + 8192, UK = FAKE + 16384, AG = FAKE + 24576, C = FAKE + (1 << 24);
    CHECK(dws_reduce_by_key(at(K), at(V), at(UK), at(AG), n, (dws_dtype)7, at(C), NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_reduce_by_key(at(K), at(V), at(UK), NULL, n, DWS_FLOAT32, at(C), NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_reduce_by_key(at(K + 2), at(V), at(UK), at(AG), n, DWS_INT32, at(C), NULL), DWS_ERR_MISALIGNED);
    CHECK(dws_reduce_by_key(at(K), at(V), at(UK), at(V + 400), n, DWS_INT32, at(C), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_reduce_by_key(at(K), at(V), at(UK), at(AG), n, DWS_INT32, at(UK + 8), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_reduce_by_key(at(K), at(V), at(UK), at(AG), (size_t)1 << 32, DWS_INT32, at(C + (1ull << 40)), NULL),
          DWS_ERR_UNSUPPORTED);
    CHECK(dws_run_length_encode(at(K), at(UK), at(AG), n, NULL, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_run_length_encode(at(K), at(K + 3996), at(AG), n, at(C), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_run_length_encode(at(K + 1), at(UK), at(AG), n, at(C), NULL), DWS_ERR_MISALIGNED);
}

static void operators(void)
{
    const uint64_t big = FAKE + (1 << 24);
    CHECK(dws_scan_op(at(FAKE), at(big), 10, (dws_dtype)5, DWS_OP_MAX, 0, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_op(at(FAKE), at(big), 10, DWS_INT32, (dws_op)5, 0, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_op(at(FAKE), at(big), 10, DWS_INT32, (dws_op)-1, 0, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_op(at(FAKE), at(big), 10, DWS_FLOAT32, DWS_OP_MAX, 0, NULL), DWS_ERR_UNSUPPORTED);
    CHECK(dws_scan_op(at(FAKE), at(big), 10, DWS_INT32, DWS_OP_AFFINE, 0, NULL), DWS_ERR_UNSUPPORTED);
    CHECK(dws_scan_op(at(FAKE + 4), at(big), 10, DWS_PAIR_U32, DWS_OP_AFFINE, 0, NULL), DWS_ERR_MISALIGNED);
    CHECK(dws_scan_op(at(FAKE), at(FAKE + 8), 10, DWS_PAIR_U32, DWS_OP_SEGMENTED_SUM, 0, NULL), DWS_ERR_OVERLAP);
    CHECK(dws_scan_op(NULL, NULL, 0, DWS_PAIR_U32, DWS_OP_AFFINE, 1, NULL), DWS_OK);
    CHECK(dws_scan_op(at(FAKE), at(big), DWS_MAX_ELEMENTS + 1, DWS_PAIR_U32, DWS_OP_AFFINE, 0, NULL),
          DWS_ERR_UNSUPPORTED);
}

static void sharded_steps(void)
{
    const uint64_t seed = FAKE + (1ull << 41);
    /* dws_scan_seeded: the scans' checks, then the seed's */
    CHECK(dws_scan_seeded(NULL, NULL, 0, DWS_INT32, 0, NULL, NULL), DWS_OK);
    CHECK(dws_scan_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_INT32, 0, NULL, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_seeded(at(FAKE), at(FAKE + 4096), 10, (dws_dtype)5, 0, at(seed), NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_FLOAT32, 1, at(seed + 2), NULL), DWS_ERR_MISALIGNED);
    CHECK(dws_scan_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_INT32, 0, at(FAKE + 4096 + 36), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_scan_seeded(at(FAKE), at(FAKE), 10, DWS_INT32, 1, at(FAKE), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_scan_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_INT32, 0, at(UINT64_MAX - 1), NULL), DWS_ERR_MISALIGNED);
    /* dws_reduce */
    CHECK(dws_reduce(NULL, 0, DWS_INT32, NULL, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_reduce(NULL, 10, DWS_INT32, at(seed), NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_reduce(at(FAKE), 10, (dws_dtype)-2, at(seed), NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_reduce(at(FAKE), 10, DWS_FLOAT32, at(seed + 1), NULL), DWS_ERR_MISALIGNED);
    CHECK(dws_reduce(at(FAKE), DWS_MAX_ELEMENTS + 1, DWS_UINT32, at(seed), NULL), DWS_ERR_UNSUPPORTED);
    CHECK(dws_reduce(at(FAKE), 10, DWS_INT32, at(FAKE + 36), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_reduce(at(UINT64_MAX - 15), 100, DWS_INT32, at(seed), NULL), DWS_ERR_INVALID_ARG);
    /* under the generic operators */
    CHECK(dws_scan_op_seeded(NULL, NULL, 0, DWS_PAIR_U32, DWS_OP_AFFINE, 0, NULL, NULL), DWS_OK);
    CHECK(dws_scan_op_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_PAIR_U32, (dws_op)9, 0, at(seed), NULL),
          DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_op_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_FLOAT32, DWS_OP_MAX, 0, at(seed), NULL),
          DWS_ERR_UNSUPPORTED);
    CHECK(dws_scan_op_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_PAIR_U32, DWS_OP_AFFINE, 1, NULL, NULL),
          DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_op_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_PAIR_U32, DWS_OP_AFFINE, 1, at(FAKE + 4092), NULL),
          DWS_ERR_OVERLAP);
    CHECK(dws_scan_op_seeded(at(FAKE), at(FAKE + 4096), 10, DWS_PAIR_I32_F32, DWS_OP_SEGMENTED_SUM, 0,
                             at(FAKE + 4096 + 72), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_reduce_op(at(FAKE), 10, DWS_PAIR_U32, DWS_OP_AFFINE, NULL, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_reduce_op(at(FAKE), 10, DWS_INT32, DWS_OP_AFFINE, at(seed), NULL), DWS_ERR_UNSUPPORTED);
    CHECK(dws_reduce_op(at(FAKE + 4), 10, DWS_PAIR_U32, DWS_OP_SUM, at(seed), NULL), DWS_ERR_MISALIGNED);
    CHECK(dws_reduce_op(at(FAKE), 10, DWS_PAIR_U32, DWS_OP_SUM, at(FAKE + 76), NULL), DWS_ERR_OVERLAP);
    CHECK(dws_reduce_op(at(FAKE), DWS_MAX_ELEMENTS + 1, DWS_INT32, DWS_OP_MAX, at(seed), NULL), DWS_ERR_UNSUPPORTED);
    CHECK(dws_reduce_op(at(UINT64_MAX - 7), 10, DWS_PAIR_U32, DWS_OP_AFFINE, at(seed), NULL), DWS_ERR_INVALID_ARG);
}

static void diagnostics(void)
{
    CHECK(dws_scan_debug(at(FAKE), at(FAKE + 4096), 16, DWS_INT32, 0, 0, 0, 0, 0, 0, NULL, NULL),
          DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_debug(at(FAKE), at(FAKE + 4096), 16, DWS_INT32, 0, 0, 65, 0, 0, 0, NULL, NULL),
          DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_debug(at(FAKE), at(FAKE + 4), 16, DWS_INT32, 0, 0, 4, 0, 0, 0, NULL, NULL), DWS_ERR_OVERLAP);
    CHECK(dws_scan_debug(NULL, NULL, 0, DWS_INT32, 0, 0, 4, 0, 0, 0, NULL, NULL), DWS_OK);
    unsigned tiles = 0;
    CHECK(dws_scan_profiled(at(FAKE), at(FAKE + (1 << 20)), 1 << 16, (dws_dtype)9, 0, NULL, 0, &tiles, NULL),
          DWS_ERR_INVALID_ARG);
    CHECK(dws_scan_profiled(at(FAKE), at(FAKE + 4), 1 << 16, DWS_INT32, 0, at(FAKE + (1 << 24)), 1 << 20, NULL,
                            NULL),
          DWS_ERR_OVERLAP);
    CHECK(dws_selftest_wave(NULL, NULL, NULL, 0, DWS_INT32, NULL), DWS_OK);
    CHECK(dws_selftest_wave(NULL, at(FAKE), at(FAKE), 1, DWS_INT32, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_watchdog_trips(NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_device_memory_info(NULL, NULL, NULL), DWS_ERR_INVALID_ARG);
    CHECK(dws_reserve(DWS_MAX_ELEMENTS + 1, NULL), DWS_ERR_UNSUPPORTED);
}

int main(void)
{
    status_and_geometry();
    sharded_steps();
    scans();
    compaction();
    operators();
    diagnostics();
    printf(g_bad ? "abi driver: FAILED\n" : "abi driver: ok\n");
    return g_bad;
}

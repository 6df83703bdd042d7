/*
 * Host sanitizer driver for the CPU oracle (oracle/scan_oracle.c): built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py,
 * it calls every oracle function on exactly sized heap buffers, so that a read
 * or write one element past an array, a signed overflow or a bad shift aborts
 * the run. Sizes cover the empty input, one element, both sides of 64 and a
 * few hundred elements; the inputs include the extreme 32-bit values.
 * A few results are checked against closed forms on the side; the oracle's
 * correctness is pinned elsewhere, this driver is about memory and UB.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_abi_version(void);
int oracle_scan_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive);
int oracle_scan_f32(const float* x, size_t n, double* y, double* sabs, int exclusive);
size_t oracle_select_flagged(const uint32_t* x, const int32_t* flags, size_t n, uint32_t* out);
int oracle_scan_minmax(const uint32_t* x, size_t n, uint32_t* y, int is_signed, int is_max, int exclusive);
int oracle_scan_pair_sum_i32_f32(const uint32_t* x, size_t n, uint32_t* y_int, double* y_f, double* sabs,
                                 int exclusive);
int oracle_scan_pair_sum_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive);
int oracle_scan_affine_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive);
int oracle_scan_segsum_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive);
int oracle_scan_segsum_i32_f32(const uint32_t* x, size_t n, uint32_t* y_flag, double* y_f, double* sabs,
                               int exclusive);
size_t oracle_partition_flagged(const uint32_t* x, const int32_t* flags, size_t n, uint32_t* out);
size_t oracle_reduce_by_key_u32(const uint32_t* keys, const uint32_t* vals, size_t n, uint32_t* ukeys,
                                uint32_t* aggs);
size_t oracle_reduce_by_key_f32(const uint32_t* keys, const float* vals, size_t n, uint32_t* ukeys, double* aggs,
                                double* abs_sums);
size_t oracle_run_length_encode(const uint32_t* keys, size_t n, uint32_t* ukeys, uint32_t* lengths);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    /* splitmix64 step, upper half */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

/* n elements of `size` bytes, exactly; n == 0 still gives a distinct pointer */
static void* alloc(size_t n, size_t size)
{
    void* p = malloc(n == 0 ? 1 : n * size);
    if (p == NULL) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int fail(const char* what, size_t n)
{
    fprintf(stderr, "FAIL %s (n=%zu)\n", what, n);
    return 1;
}

static int run_size(size_t n)
{
    int bad = 0;
    uint32_t* x = alloc(n, 4);
    uint32_t* x2 = alloc(2 * n, 4);
    float* xf = alloc(n, 4);
    int32_t* flags = alloc(n, 4);
    uint32_t* keys = alloc(n, 4);
    uint32_t* y = alloc(n, 4);
    uint32_t* y2 = alloc(2 * n, 4);
    double* yd = alloc(n, 8);
    double* sd = alloc(n, 8);
    uint32_t* uk = alloc(n, 4);
    uint32_t* ag = alloc(n, 4);
    double* agd = alloc(n, 8);

    const uint32_t extremes[] = {0u, 1u, 0x7FFFFFFFu, 0x80000000u, 0xFFFFFFFFu};
    uint32_t key = 0u;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t r = next_u32();
        x[i] = (r & 7u) == 0u ? extremes[r % 5u] : r;
        x2[2 * i] = next_u32() & 1u;
        x2[2 * i + 1] = next_u32();
        xf[i] = (float)((int32_t)(next_u32() >> 8) - (1 << 23)) / (float)(1 << 23);
        flags[i] = (int32_t)(next_u32() & 1u);
        if ((next_u32() & 3u) == 0u) key = next_u32();
        keys[i] = key;
    }

    for (int ex = 0; ex < 2; ++ex) {
        if (oracle_scan_u32(x, n, y, ex) != 0) bad |= fail("scan_u32", n);
        if (n > 0 && ex == 0) {
            uint32_t s = 0u;
            for (size_t i = 0; i < n; ++i) s += x[i];
            if (y[n - 1] != s) bad |= fail("scan_u32 total", n);
        }
        if (oracle_scan_f32(xf, n, yd, sd, ex) != 0) bad |= fail("scan_f32", n);
        if (oracle_scan_f32(xf, n, yd, NULL, ex) != 0) bad |= fail("scan_f32 without sabs", n);
        for (int sg = 0; sg < 2; ++sg)
            for (int mx = 0; mx < 2; ++mx)
                if (oracle_scan_minmax(x, n, y, sg, mx, ex) != 0) bad |= fail("scan_minmax", n);
        if (oracle_scan_pair_sum_i32_f32(x2, n, y, yd, sd, ex) != 0) bad |= fail("pair_sum_i32_f32", n);
        if (oracle_scan_pair_sum_u32(x2, n, y2, ex) != 0) bad |= fail("pair_sum_u32", n);
        if (oracle_scan_affine_u32(x2, n, y2, ex) != 0) bad |= fail("affine_u32", n);
        if (oracle_scan_segsum_u32(x2, n, y2, ex) != 0) bad |= fail("segsum_u32", n);
        if (oracle_scan_segsum_i32_f32(x2, n, y, yd, sd, ex) != 0) bad |= fail("segsum_i32_f32", n);
        if (oracle_scan_segsum_i32_f32(x2, n, y, yd, NULL, ex) != 0) bad |= fail("segsum_i32_f32 no sabs", n);
    }

    size_t cnt = oracle_select_flagged(x, flags, n, y);
    size_t want = 0;
    for (size_t i = 0; i < n; ++i) want += flags[i] != 0;
    if (cnt != want) bad |= fail("select count", n);
    if (oracle_partition_flagged(x, flags, n, y) != want) bad |= fail("partition count", n);
    const size_t runs = oracle_run_length_encode(keys, n, uk, ag);
    size_t total = 0;
    for (size_t r = 0; r < runs; ++r) total += ag[r];
    if (total != n) bad |= fail("run lengths sum to n", n);
    if (oracle_reduce_by_key_u32(keys, x, n, uk, ag) != runs) bad |= fail("reduce_by_key_u32 runs", n);
    if (oracle_reduce_by_key_f32(keys, xf, n, uk, agd, yd) != runs) bad |= fail("reduce_by_key_f32 runs", n);

    free(x); free(x2); free(xf); free(flags); free(keys); free(y); free(y2);
    free(yd); free(sd); free(uk); free(ag); free(agd);
    return bad;
}

int main(void)
{
    const size_t sizes[] = {0, 1, 2, 3, 63, 64, 65, 127, 128, 129, 1000, 4097};
    int bad = 0;
    if (oracle_abi_version() < 1) bad |= fail("abi version", 0);
    for (size_t k = 0; k < sizeof(sizes) / sizeof(sizes[0]); ++k) bad |= run_size(sizes[k]);
    /* null outputs with n > 0 are refused, not dereferenced */
    uint32_t one = 1u;
    if (oracle_scan_u32(&one, 1, NULL, 0) == 0) bad |= fail("scan_u32 refuses a null output", 1);
    if (oracle_scan_pair_sum_u32(&one, 1, NULL, 0) == 0) bad |= fail("pair_sum refuses a null output", 1);
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}

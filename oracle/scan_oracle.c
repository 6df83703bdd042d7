/*
 * Sequential CPU oracle for the device-wide + prefix scan.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it (through oracle/__init__.py). It shares no header, table
 * or helper with the HIP path.
 *
 * What it computes is the plain definition of a prefix sum, one element at a
 * time, in input order:
 *   inclusive  y[i] = x[0] + x[1] + ... + x[i]
 *              (CUDA-Operators-6-Cumsum, section 1 "Cumsum theory": the
 *               definition and its one-loop CPU routine; the same definition is
 *               restated in the RTX 4090 scan notes at smarter.xin, section
 *               "three implementations", problem statement);
 *   exclusive  y[0] = 0 (the identity of +), y[i] = x[0] + ... + x[i-1]
 *              (smarter.xin RTX 4090 scan notes, section on converting between
 *               inclusive and exclusive scans).
 * The serial chain is the minimum-size scan network, n-1 operator applications
 * (Merrill & Garland, "Single-pass Parallel Prefix Scan with Decoupled
 * Look-back", section A3, serial scan of Fig 1a).
 *
 * Readings where the pages are silent:
 *   - 32-bit integers: the pages do not say what happens on overflow. The
 *     accumulator is uint32_t, so every addition wraps modulo 2^32; int32 data
 *     is scanned as its two's-complement bit pattern, which gives the same bits
 *     as wrapping signed addition and avoids signed-overflow undefined
 *     behaviour.
 *   - fp32: the pages say floating-point results of the single-pass method vary
 *     from run to run (section A6 of the Merrill & Garland notes), so there is
 *     no bit pattern to reproduce. The oracle accumulates in fp64 and returns
 *     fp64 sums; alongside it returns the running absolute sum
 *     s[i] = |x[0]| + ... + |x[i]| (fp64), which scales the fp32 tolerance.
 *
 * Pins (tests/test_oracle_pins.py): the 16-element worked examples printed in
 * the PMPP 11.3 and 11.2 notes (tests/golden/), closed forms (constant and
 * arithmetic inputs), modular wrap cases, an fp64-accumulation witness,
 * O(n^2) brute force on small n and numpy's cumsum as an independent library
 * routine. The compaction is pinned by closed forms (all, none, every other),
 * brute force against a list comprehension, the scatter to exclusive prefix
 * offsets and numpy's boolean-mask indexing.
 */
#include <stddef.h>
#include <stdint.h>
#include <math.h>

#define ORACLE_ABI_VERSION 1

int oracle_abi_version(void) { return ORACLE_ABI_VERSION; }

/*
 * 32-bit integer scan, modulo 2^32. x and y may be the same buffer (each x[i]
 * is read before y[i] is written). Returns 0, or -1 on a null pointer with
 * n > 0.
 */
int oracle_scan_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y == NULL) return -1;
    uint32_t running = 0u;
    for (size_t i = 0; i < n; ++i) {
        uint32_t xi = x[i];
        if (exclusive) {
            y[i] = running;
            running += xi;
        } else {
            running += xi;
            y[i] = running;
        }
    }
    return 0;
}

/*
 * fp32 scan accumulated in fp64. y receives the fp64 prefix sums; sabs (may be
 * NULL) receives the fp64 running absolute sums up to and including element i,
 * for both the inclusive and the exclusive scan. Returns 0, or -1 on a null
 * pointer with n > 0.
 */
int oracle_scan_f32(const float* x, size_t n, double* y, double* sabs, int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y == NULL) return -1;
    double running = 0.0;
    double running_abs = 0.0;
    for (size_t i = 0; i < n; ++i) {
        double xi = (double)x[i];
        if (exclusive) {
            y[i] = running;
            running += xi;
        } else {
            running += xi;
            y[i] = running;
        }
        if (sabs != NULL) {
            running_abs += fabs(xi);
            sabs[i] = running_abs;
        }
    }
    return 0;
}

/*
 * Stream compaction by flags: appends, in input order, every x[i] whose flag
 * is non-zero to out and returns how many were appended. This is the plain
 * definition of the select operation that Merrill & Garland (section 4.4,
 * in-place compaction) build from a prefix sum of 0/1 flags: selected element
 * i lands at the number of selected elements before it. out may be x itself
 * (the write index never passes the read index).
 */
size_t oracle_select_flagged(const uint32_t* x, const int32_t* flags, size_t n, uint32_t* out)
{
    size_t count = 0;
    for (size_t i = 0; i < n; ++i) {
        if (flags[i] != 0) {
            out[count] = x[i];
            ++count;
        }
    }
    return count;
}

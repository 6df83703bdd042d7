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
 * offsets and numpy's boolean-mask indexing. The generic operators are pinned
 * by numpy's maximum/minimum.accumulate and per-column cumsum, by running the
 * affine recurrence directly from several start values, by brute-force
 * segmented sums and by closed forms (a = 1, b = 0; all heads, no heads).
 * Partition, reduce-by-key and run-length encoding are pinned by numpy's
 * boolean masks, itertools.groupby, numpy's add.reduceat and diff over the run
 * starts, and closed forms (one run, all distinct, keys as bit patterns).
 */
#include <stddef.h>
#include <stdint.h>
#include <math.h>
#include <string.h>

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

/*
 * Generic associative operators (Merrill & Garland, section 4.2: the method
 * only ever combines contiguous inputs or contiguous partial reductions, so
 * the operator need not be commutative; section A4: 32-bit integers and
 * {int32, fp32} pairs). Each function below is one sequential loop that folds
 * the operator left to right, x[0] first, and writes the running value after
 * (inclusive) or before (exclusive, identity first) element i. Pairs are two
 * 32-bit words per element, interleaved: x[2i] first component, x[2i+1]
 * second.
 */

/* Running max or min of 32-bit integers, signed or unsigned. The exclusive
 * identity is the smallest (max) or largest (min) value of the type. */
int oracle_scan_minmax(const uint32_t* x, size_t n, uint32_t* y, int is_signed, int is_max, int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y == NULL) return -1;
    uint32_t running;
    if (is_max) running = is_signed ? 0x80000000u : 0u;
    else running = is_signed ? 0x7fffffffu : 0xffffffffu;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t xi = x[i];
        int take;
        if (is_signed) take = is_max ? ((int32_t)xi > (int32_t)running) : ((int32_t)xi < (int32_t)running);
        else take = is_max ? (xi > running) : (xi < running);
        if (exclusive) y[i] = running;
        if (take) running = xi;
        if (!exclusive) y[i] = running;
    }
    return 0;
}

static float word_as_float(uint32_t w)
{
    float f;
    memcpy(&f, &w, sizeof f);
    return f;
}

/* Componentwise + on {int32, fp32} pairs: the integer part wraps modulo 2^32,
 * the fp32 part is accumulated in fp64 (returned as y_f) with the running
 * absolute sum over j <= i (sabs, may be NULL), as for the fp32 scan. */
int oracle_scan_pair_sum_i32_f32(const uint32_t* x, size_t n, uint32_t* y_int, double* y_f, double* sabs,
                                 int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y_int == NULL || y_f == NULL) return -1;
    uint32_t ri = 0u;
    double rf = 0.0, ra = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t xi = x[2 * i];
        const double xf = (double)word_as_float(x[2 * i + 1]);
        if (exclusive) {
            y_int[i] = ri;
            y_f[i] = rf;
        }
        ri += xi;
        rf += xf;
        if (!exclusive) {
            y_int[i] = ri;
            y_f[i] = rf;
        }
        ra += fabs(xf);
        if (sabs != NULL) sabs[i] = ra;
    }
    return 0;
}

/* Componentwise + on pairs of uint32, modulo 2^32. */
int oracle_scan_pair_sum_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y == NULL) return -1;
    uint32_t r0 = 0u, r1 = 0u;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t x0 = x[2 * i], x1 = x[2 * i + 1];
        if (exclusive) {
            y[2 * i] = r0;
            y[2 * i + 1] = r1;
        }
        r0 += x0;
        r1 += x1;
        if (!exclusive) {
            y[2 * i] = r0;
            y[2 * i + 1] = r1;
        }
    }
    return 0;
}

/* Composition of affine maps modulo 2^32 (a non-commutative operator).
 * Element (a, b) is the map v -> a v + b. The running value (A, B) is the
 * composition of the maps of elements 0..i, applied in order, so that for any
 * start value s the recurrence v_i = a_i v_{i-1} + b_i, v_{-1} = s, gives
 * v_i = A_i s + B_i. Folding element (a, b) into (A, B) gives (a A, a B + b);
 * the identity is (1, 0). */
int oracle_scan_affine_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y == NULL) return -1;
    uint32_t A = 1u, B = 0u;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t a = x[2 * i], b = x[2 * i + 1];
        if (exclusive) {
            y[2 * i] = A;
            y[2 * i + 1] = B;
        }
        A = a * A;
        B = a * B + b;
        if (!exclusive) {
            y[2 * i] = A;
            y[2 * i + 1] = B;
        }
    }
    return 0;
}

/* Segmented sum on (flag, value) pairs (a non-commutative operator): a
 * non-zero flag starts a new segment, whose running value restarts at the
 * element's own value; the flag part of the result is the bitwise OR of all
 * flags so far. Identity (0, 0). The value is uint32 modulo 2^32 here. */
int oracle_scan_segsum_u32(const uint32_t* x, size_t n, uint32_t* y, int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y == NULL) return -1;
    uint32_t F = 0u, V = 0u;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t f = x[2 * i], v = x[2 * i + 1];
        if (exclusive) {
            y[2 * i] = F;
            y[2 * i + 1] = V;
        }
        F |= f;
        if (f != 0u) V = v;
        else V += v;
        if (!exclusive) {
            y[2 * i] = F;
            y[2 * i + 1] = V;
        }
    }
    return 0;
}

/* Segmented sum on {int32 flag, fp32 value} pairs, the value accumulated in
 * fp64. sabs[i] (may be NULL) is the sum of |value| over exactly the elements
 * whose values make up y_f[i] (the current segment up to i, or up to i - 1 for
 * the exclusive scan), which scales the fp32 tolerance. */
int oracle_scan_segsum_i32_f32(const uint32_t* x, size_t n, uint32_t* y_flag, double* y_f, double* sabs,
                               int exclusive)
{
    if (n == 0) return 0;
    if (x == NULL || y_flag == NULL || y_f == NULL) return -1;
    uint32_t F = 0u;
    double V = 0.0, S = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t f = x[2 * i];
        const double v = (double)word_as_float(x[2 * i + 1]);
        if (exclusive) {
            y_flag[i] = F;
            y_f[i] = V;
            if (sabs != NULL) sabs[i] = S;
        }
        F |= f;
        if (f != 0u) {
            V = v;
            S = fabs(v);
        } else {
            V += v;
            S += fabs(v);
        }
        if (!exclusive) {
            y_flag[i] = F;
            y_f[i] = V;
            if (sabs != NULL) sabs[i] = S;
        }
    }
    return 0;
}

/*
 * The rest of the compaction family the single pass fuses with its scan
 * (Merrill & Garland, section 4.4 in-place compaction behaviour; section A5:
 * select-if, partition-if, reduce-by-key, run-length encoding). Plain
 * sequential definitions.
 */

/* Partition by flags: the x[i] with a non-zero flag go to out[0 .. count) in
 * input order, the others to out[count .. n) in reverse input order (the last
 * rejected element first), which is the layout a single pass can write
 * without knowing count in advance. Returns count. out must not alias x. */
size_t oracle_partition_flagged(const uint32_t* x, const int32_t* flags, size_t n, uint32_t* out)
{
    size_t sel = 0, rej = 0;
    for (size_t i = 0; i < n; ++i) {
        if (flags[i] != 0) {
            out[sel] = x[i];
            ++sel;
        } else {
            out[n - 1 - rej] = x[i];
            ++rej;
        }
    }
    return sel;
}

/* Reduce by key: each maximal run of consecutive equal keys (32-bit patterns)
 * gives one output: its key in ukeys[r] and the + of its values in aggs[r],
 * runs in input order. Returns the number of runs. uint32 values wrap modulo
 * 2^32. */
size_t oracle_reduce_by_key_u32(const uint32_t* keys, const uint32_t* vals, size_t n, uint32_t* ukeys,
                                uint32_t* aggs)
{
    size_t runs = 0;
    for (size_t i = 0; i < n; ++i) {
        if (i == 0 || keys[i] != keys[i - 1]) {
            ukeys[runs] = keys[i];
            aggs[runs] = 0u;
            ++runs;
        }
        aggs[runs - 1] += vals[i];
    }
    return runs;
}

/* The same with fp32 values, summed in fp64; abs_sums[r] (may be NULL) is the
 * sum of |value| over run r, which scales the fp32 tolerance. */
size_t oracle_reduce_by_key_f32(const uint32_t* keys, const float* vals, size_t n, uint32_t* ukeys, double* aggs,
                                double* abs_sums)
{
    size_t runs = 0;
    for (size_t i = 0; i < n; ++i) {
        if (i == 0 || keys[i] != keys[i - 1]) {
            ukeys[runs] = keys[i];
            aggs[runs] = 0.0;
            if (abs_sums != NULL) abs_sums[runs] = 0.0;
            ++runs;
        }
        aggs[runs - 1] += (double)vals[i];
        if (abs_sums != NULL) abs_sums[runs - 1] += fabs((double)vals[i]);
    }
    return runs;
}

/* Run-length encoding: each maximal run of equal keys gives its key and its
 * length. Returns the number of runs. */
size_t oracle_run_length_encode(const uint32_t* keys, size_t n, uint32_t* ukeys, uint32_t* lengths)
{
    size_t runs = 0;
    for (size_t i = 0; i < n; ++i) {
        if (i == 0 || keys[i] != keys[i - 1]) {
            ukeys[runs] = keys[i];
            lengths[runs] = 0u;
            ++runs;
        }
        lengths[runs - 1] += 1u;
    }
    return runs;
}

/*
 * dws_scan.h — device-wide + prefix scan (inclusive / exclusive) for AMD
 * Instinct MI355X (gfx950), single pass with decoupled look-back.
 *
 * What is computed (the plain definition of a prefix sum):
 *   inclusive  y[i] = x[0] + ... + x[i]
 *   exclusive  y[0] = 0,  y[i] = x[0] + ... + x[i-1]
 * Definition: CUDA-Operators-6-Cumsum, section 1 (Cumsum theory); the
 * exclusive form and its identity first element: the smarter.xin RTX 4090 scan
 * notes, section on converting between inclusive and exclusive scans.
 * How: one kernel launch in which every workgroup scans one tile, publishes its
 * aggregate, then determines its exclusive prefix by looking back over
 * predecessor tiles' descriptors (Merrill & Garland, "Single-pass Parallel
 * Prefix Scan with Decoupled Look-back", sections 4.1 and 4.4). It moves about
 * 2n elements through memory (section A1 of the same notes).
 *
 * Element types and arithmetic:
 *   DWS_INT32, DWS_UINT32  wrap modulo 2^32 (int32 is two's complement, so both
 *                          give identical bits); results are deterministic.
 *   DWS_FLOAT32            IEEE fp32 additions, round to nearest even; the order
 *                          of additions depends on run-time scheduling, so bits
 *                          may differ from run to run (section A6 of the same
 *                          notes) while staying within a few ulps of the exact
 *                          prefix relative to the running sum of |x|.
 *
 * Pointers: d_in and d_out are DEVICE pointers on the current HIP device, owned
 * by the caller, each holding n contiguous 4-byte elements. d_out == d_in
 * (in place) is allowed; any other overlap is rejected. Pointers must be 4-byte
 * aligned; 16-byte alignment of both selects the vector (dwordx4) path, other
 * alignments a scalar-load path with the same results.
 *
 * Streams and ownership: every call is asynchronous on `stream` (0 = the
 * default stream of the current device) and returns after enqueue. The library
 * keeps one small workspace per (device, stream): descriptors (8 bytes per
 * tile and 32-bit element word), a tile counter, a partials array for the
 * reduce-then-scan variant and, allocated on its first use, the tile sums of
 * the scan-then-propagate variant (about n / 4095 elements). It is allocated
 * and cleared on the first multi-tile call on that stream (which therefore
 * must not be under graph capture; dws_reserve can create it ahead of time)
 * and reused by later calls, which the stream orders; a call that needs more
 * descriptors than the workspace holds synchronises the stream and grows it.
 *
 * Graphs: once the workspace of the stream covers n (a first call, or
 * dws_reserve), calls on that stream allocate nothing and may be captured
 * into a HIP graph. A call captured before that, which would have to create
 * or grow the workspace, returns DWS_ERR_UNSUPPORTED without allocating,
 * synchronising or enqueuing anything, so the capture stays valid. Replays stay correct: each launch (the
 * reductions dws_reduce and dws_reduce_op included, whose partials are
 * descriptors of the same workspace) takes its descriptor epoch from a device
 * word that the launch itself advances. The host clears
 * the descriptors before its own calls could wrap the 30-bit epoch, but
 * replays advance it unseen: after about 2^30 launches on one workspace,
 * replays included, call dws_release_workspaces (and capture again) so that
 * no epoch is reused.
 * Calls on different streams never share a workspace. Host threads may call
 * concurrently. dws_release_workspaces frees every workspace.
 * Workspaces are keyed by the stream handle and outlive the stream: destroying
 * a stream frees nothing, and a stream created later may receive the same
 * handle and then reuses that workspace. So synchronise a stream that has
 * called the library before destroying it (a call still running on it would
 * otherwise share its descriptors and tile counter with the new stream's
 * calls), and call dws_release_workspaces to free the workspaces of streams
 * that are gone.
 *
 * Errors: argument checks run before any HIP call and enqueue nothing. No C++
 * exception crosses this interface.
 */
#ifndef DWS_SCAN_H
#define DWS_SCAN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DWS_VERSION 3

typedef enum dws_status {
    DWS_OK = 0,
    DWS_ERR_INVALID_ARG = 1,   /* null pointer with n > 0, bad enum or option */
    DWS_ERR_UNSUPPORTED = 2,   /* n above a limit, or an option, operator or
                                  type combination that is not built */
    DWS_ERR_OVERLAP = 3,       /* d_in and d_out overlap without being equal */
    DWS_ERR_HIP = 4,           /* a HIP runtime call failed */
    DWS_ERR_OOM = 5,           /* workspace allocation failed */
    DWS_ERR_MISALIGNED = 6     /* a pointer is not aligned to the element size */
} dws_status;

typedef enum dws_dtype {
    DWS_INT32 = 0,
    DWS_UINT32 = 1,
    DWS_FLOAT32 = 2,
    /* 8-byte pairs, for dws_scan_op only: {int32, fp32} (Merrill & Garland,
     * section A4, data types) and {uint32, uint32}; first component at the
     * lower address */
    DWS_PAIR_I32_F32 = 3,
    DWS_PAIR_U32 = 4
} dws_dtype;

/* Largest supported element count (2^35). */
#define DWS_MAX_ELEMENTS (((size_t)1) << 35)

/*
 * Inclusive + scan of n elements: d_out[i] = d_in[0] + ... + d_in[i].
 * Single-pass decoupled look-back (Merrill & Garland, section 4.1). n == 0 is a
 * no-op returning DWS_OK.
 */
dws_status scan_inclusive(const void* d_in, void* d_out, size_t n,
                          dws_dtype dtype, hipStream_t stream);

/*
 * Exclusive + scan of n elements: d_out[0] = 0, d_out[i] = d_in[0] + ... +
 * d_in[i-1] (smarter.xin RTX 4090 scan notes, inclusive/exclusive section). The
 * exclusive values are produced directly, not by subtracting x from an
 * inclusive result. Same contract as scan_inclusive.
 */
dws_status scan_exclusive(const void* d_in, void* d_out, size_t n,
                          dws_dtype dtype, hipStream_t stream);

/* Global strategy: the variant argument of dws_scan_ex, or dws_options.variant. */
typedef enum dws_variant {
    /* one pass, decoupled look-back: ~2n traffic (Merrill & Garland, 4.1) */
    DWS_VARIANT_SINGLE_PASS = 0,
    /* three kernels: reduce G chunks, scan the G partials, seeded scan of
     * each chunk: ~3n traffic (same notes, section 3.2, Fig 3; G is the
     * number of co-resident workgroups, CUDA-Operators-6-Cumsum section 1.2) */
    DWS_VARIANT_REDUCE_THEN_SCAN = 1,
    /* one pass, each tile waits for its immediate predecessor's inclusive
     * prefix: ~2n traffic, serial signal chain (same notes, section 3.2,
     * Fig 4; PMPP 11.3 notes, single-pass domino scan with adjacent
     * synchronisation) */
    DWS_VARIANT_CHAINED = 2,
    /* three steps, recursively: scan every tile on its own, scan the tile
     * sums, add each tile's scanned predecessor sum to its elements: ~4n
     * traffic (PMPP 11.3 notes, hierarchical scan; CUDA-Operators-6-Cumsum
     * section 2, recursive form; Merrill & Garland section 3.2) */
    DWS_VARIANT_SCAN_THEN_PROPAGATE = 3
} dws_variant;

/* Ordering of descriptor stores and loads. The descriptor packs status and
 * value in one 64-bit word, so a relaxed device-scope atomic suffices for the
 * protocol (Merrill & Garland, section 4.4, fence-free descriptor updates);
 * release/acquire is available for comparison. */
typedef enum dws_memory_order {
    DWS_ORDER_RELAXED = 0,
    DWS_ORDER_ACQ_REL = 1
} dws_memory_order;

/* Where a tile's index comes from in the single-pass and chained kernels. */
typedef enum dws_tile_index {
    /* the library's choice: DWS_TILE_DISPATCH for the relaxed single pass
     * (non-temporal loads asked for on a shape whose workgroup-index kernel
     * has none take DWS_TILE_DRAWN), DWS_TILE_DRAWN for the chained scan and
     * release/acquire descriptors */
    DWS_TILE_AUTO = 0,
    /* one atomic add on a device-wide counter per workgroup, in the order the
     * workgroups start (PMPP 11.3 notes, dynamic block index; Merrill &
     * Garland, section 4.4): a tile only ever waits on tiles whose
     * workgroups are running, whatever order the hardware starts them in */
    DWS_TILE_DRAWN = 1,
    /* the workgroup index itself: no atomic per tile, relying on the GPU
     * starting the workgroups of each XCD in index order. A look-back wait
     * that still outlives the watchdog (about two seconds) ends and is
     * counted by dws_watchdog_trips() */
    DWS_TILE_DISPATCH = 2
} dws_tile_index;

typedef struct dws_options {
    int variant;        /* dws_variant; default DWS_VARIANT_SINGLE_PASS */
    int memory_order;   /* dws_memory_order; default DWS_ORDER_RELAXED */
    int tile_shape;     /* 0 = automatic (by n: 65536-element tiles from
                           2^24 elements, 32768 from 2^23, 16384 from 2^20,
                           else 4096);
                           1 .. dws_num_tile_shapes()-1 force one shape of
                           the single-pass kernel, for sweeps */
    int nontemporal;    /* non-temporal (streaming) loads of the input:
                           0 = the library's choice (for the automatic
                           relaxed single pass: on from 2^23 elements,
                           in place or not),
                           1 = on, 2 = off; stores are never
                           non-temporal */
    int tile_index;     /* dws_tile_index; default DWS_TILE_AUTO */
} dws_options;

/*
 * Scan by a chosen global strategy: exclusive != 0 selects the exclusive scan,
 * variant is a dws_variant (DWS_VARIANT_SINGLE_PASS is exactly scan_inclusive
 * / scan_exclusive; the others are the comparison strategies). Every other
 * choice is the library's automatic one. An unknown variant gives
 * DWS_ERR_INVALID_ARG. Same contract as scan_inclusive.
 */
dws_status dws_scan_ex(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                       int exclusive, int variant, hipStream_t stream);

/*
 * Scan with explicit options, for measurements and sweeps. opt == NULL (or a
 * zeroed struct) means all defaults; exclusive != 0 selects the exclusive
 * scan. Unknown values give DWS_ERR_INVALID_ARG. Built combinations (others
 * give DWS_ERR_UNSUPPORTED):
 *   single pass: every tile_shape with relaxed order; the automatically
 *                chosen shapes also with release/acquire and with
 *                nontemporal 1 (relaxed);
 *   chained:     the automatically chosen shapes, either order;
 *   reduce-then-scan, scan-then-propagate: tile_shape 0, nontemporal 0
 *                or 2, tile_index 0 (memory_order ignored);
 *   DWS_TILE_DISPATCH: single pass with relaxed order, every tile_shape,
 *                nontemporal 0 or 2; nontemporal 1 with the automatic
 *                32768- and 65536-element shapes.
 * Pointers that are not both 16-byte aligned use scalar loads; a forced
 * shape without a scalar-load kernel then falls back to the automatic one,
 * and nontemporal is ignored.
 */
dws_status dws_scan_opts(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                         int exclusive, const dws_options* opt, hipStream_t stream);

/* The launch a single-pass or chained dws_scan_opts call with the same
 * arguments would make. */
typedef struct dws_launch_plan {
    unsigned threads;      /* threads per workgroup */
    unsigned tile_elems;   /* elements per tile (one workgroup each) */
    unsigned num_tiles;    /* workgroups launched (0 when n == 0) */
    int tile_index;        /* DWS_TILE_DRAWN or DWS_TILE_DISPATCH */
    int nontemporal;       /* 1: the input is read with non-temporal loads */
    int pause_units;       /* sleep between blocked look-back polls after the
                              first re-poll, in units of 64 clocks (1: the
                              short pause) */
} dws_launch_plan;

/*
 * Describe, without launching anything or making any HIP call, what
 * dws_scan_opts(d_in, d_out, n, dtype, exclusive, opt, ...) would launch for
 * the single pass or the chained scan: the tile shape, the tile index source
 * (the dynamic index of the PMPP 11.3 notes and section 4.4 of the Merrill &
 * Garland notes, or the workgroup index), non-temporal loads and the
 * look-back's back-off, as the library chooses them. d_in and
 * d_out are only compared and checked for alignment, never dereferenced.
 * Validation and status codes are those of dws_scan_opts; the other variants
 * give DWS_ERR_UNSUPPORTED, plan == NULL gives DWS_ERR_INVALID_ARG. The
 * caller owns *plan, which is written only on DWS_OK.
 */
dws_status dws_scan_plan(const void* d_in, const void* d_out, size_t n, dws_dtype dtype,
                         int exclusive, const dws_options* opt, dws_launch_plan* plan);

/*
 * Seeded scan: the single-pass scan of d_in with the DEVICE element *d_seed
 * (one element of dtype, 4-byte aligned) as the prefix of the whole array:
 *   inclusive (exclusive == 0): d_out[i] = *d_seed + x[0] + ... + x[i]
 *   exclusive (exclusive != 0): d_out[i] = *d_seed + x[0] + ... + x[i-1],
 *                               so d_out[0] = *d_seed
 * that is, the scan of the sequence *d_seed, x[0], ..., x[n-1] without its
 * first (inclusive) or last (exclusive) element. It is the last stage of a
 * reduce-then-scan decomposition taken one level up (Merrill & Garland,
 * section 3.2 and Fig 3: each block's downsweep scan starts from the scanned
 * block aggregates): a scan split into contiguous shards scans each shard
 * seeded with the + of the shards before it (dws_reduce gives each shard's
 * total). The seed enters as the prefix of tile 0, which reads it while its
 * loads are in flight; the other tiles receive it through the look-back, so
 * the call costs what scan_inclusive / scan_exclusive cost. int32 / uint32
 * wrap mod 2^32; fp32 adds in fp32 (the seed is added to tile 0's aggregate
 * first). Same validation, kernels and workspace as scan_inclusive; in
 * addition d_seed == NULL gives DWS_ERR_INVALID_ARG, a d_seed that is not
 * 4-byte aligned DWS_ERR_MISALIGNED, and a d_seed inside d_out's n elements
 * DWS_ERR_OVERLAP (it may lie inside d_in when d_out != d_in). n == 0 is a
 * no-op that does not read *d_seed. The seed is read on `stream` in order
 * with the caller's earlier work there, so it may be written by a kernel
 * enqueued just before (dws_reduce, or a scan of shard totals).
 */
dws_status dws_scan_seeded(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                           int exclusive, const void* d_seed, hipStream_t stream);

/*
 * Device-wide + reduction: writes x[0] + ... + x[n-1] to the DEVICE element
 * *d_total (one element of dtype, 4-byte aligned; 0 when n == 0). The first
 * stage of the reduce-then-scan decomposition (Merrill & Garland, section 3.2
 * and Fig 3, block-wide reduction), used one level up to give each shard of a
 * split scan its total. One kernel launch reading the input once (4 bytes per
 * element): at most 1,024 workgroups each add a contiguous run of
 * 16,384-element tiles, and the workgroup with the highest index then adds
 * their partials in index order. int32 / uint32 wrap mod 2^32; fp32 adds in fp32 in an order
 * fixed by n and by whether d_in is 16-byte aligned, so repeated calls give
 * the same bits. Validation before any HIP call: an invalid dtype, d_total ==
 * NULL, d_in == NULL with n > 0 or an input range that wraps the address
 * space give DWS_ERR_INVALID_ARG; pointers that are
 * not 4-byte aligned DWS_ERR_MISALIGNED; n above DWS_MAX_ELEMENTS
 * DWS_ERR_UNSUPPORTED; d_total inside d_in's n elements DWS_ERR_OVERLAP. Each
 * workgroup publishes its partial as a look-back descriptor of the
 * per-(device, stream) workspace of the scans, so calls in order on one
 * stream are safe. Only the highest-indexed workgroup waits, and only on
 * workgroups that never wait; the wait is bounded like a look-back wait and
 * counts in dws_watchdog_trips when it expires (the total is then wrong).
 * Asynchronous on `stream`.
 */
dws_status dws_reduce(const void* d_in, size_t n, dws_dtype dtype, void* d_total, hipStream_t stream);

/* Tiles the fixed device array of dws_scan_noalloc has descriptors for (64
 * bytes each), so n may be up to 2^32 elements when both pointers are 16-byte
 * aligned (65,536-element tiles) and up to 2^30 otherwise (16,384). */
#define DWS_NOALLOC_MAX_TILES 65536

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * scan as scan_inclusive (exclusive == 0) or scan_exclusive (exclusive != 0),
 * with the same kernels, arguments, validation and results, but the call
 * allocates nothing. The look-back state the scans otherwise keep in a
 * per-stream workspace (a 256-byte control block and one 64-byte descriptor
 * slot per tile) lives in a fixed array of the library in device memory,
 * 256 B + DWS_NOALLOC_MAX_TILES x 64 B (4 MiB) per GPU, held until the
 * process ends.
 *
 * Limit: a call whose tile count would exceed DWS_NOALLOC_MAX_TILES returns
 * DWS_ERR_UNSUPPORTED before any HIP call (see DWS_NOALLOC_MAX_TILES for the
 * element counts).
 *
 * Set-up: the first call on a device with more than one tile (n above 4,096
 * elements) finds the array's address on that device and clears it with a
 * kernel on `stream`. That first call must not be under graph capture: there
 * it returns DWS_ERR_UNSUPPORTED without enqueuing anything. Later calls,
 * captured or not, need nothing more.
 *
 * Sharing: every call on one GPU uses that GPU's one array, which keeps the
 * last call's contents. Calls that overlap in time on one GPU (on different
 * streams, or from host threads with nothing ordering them) race on it and
 * give wrong results; calls in order on one stream are safe. Asynchronous on
 * `stream`, like scan_inclusive; look-back timeouts count in
 * dws_watchdog_trips like those of the other calls.
 */
dws_status dws_scan_noalloc(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                            int exclusive, hipStream_t stream);

/*
 * Stream compaction (select by flags), fused with the single-pass scan
 * (Merrill & Garland, section 4.4, in-place compaction; section A5): copies,
 * in order, every d_in[i] whose flag d_flags[i] (32-bit integer) is non-zero
 * to d_out[0 .. count) and writes count to the DEVICE word *d_count (64-bit,
 * 8-byte aligned). The values are moved as 32-bit words whatever dtype says
 * (dtype is checked, not used). d_out == d_in (in place) is allowed: a tile
 * writes only after every earlier tile has read its input. d_flags may equal
 * d_in when d_out does not (selects the non-zero words); the flags, the count
 * word and the output must not overlap otherwise (DWS_ERR_OVERLAP). d_out
 * elements at and past count are left unchanged. n must be below 2^32
 * (DWS_ERR_UNSUPPORTED): counts travel in 32-bit descriptor values. n == 0
 * writes count 0. Asynchronous on `stream`; same workspace as the scans.
 */
dws_status dws_select_flagged(const void* d_in, const void* d_flags, void* d_out, size_t n,
                              dws_dtype dtype, unsigned long long* d_count,
                              hipStream_t stream);

/*
 * Partition by flags (Merrill & Garland, section A5, partition-if), fused with
 * the single-pass scan like dws_select_flagged: the d_in[i] with a non-zero
 * 32-bit flag go to d_out[0 .. count) in input order, the others to
 * d_out[count .. n) in reverse input order (the last rejected element at
 * d_out[count]), a layout one pass writes without knowing count in advance.
 * count goes to the DEVICE word *d_num_selected (64-bit, 8-byte aligned).
 * d_out must not overlap d_in or d_flags (DWS_ERR_OVERLAP): rejected elements
 * land at the back before later tiles have read it. Other rules as for
 * dws_select_flagged (n below 2^32, values moved as 32-bit words).
 */
dws_status dws_partition_flagged(const void* d_in, const void* d_flags, void* d_out, size_t n,
                                 dws_dtype dtype, unsigned long long* d_num_selected,
                                 hipStream_t stream);

/* Predicates of dws_select_if / dws_partition_if: x[i] compared with a
 * threshold t in the element type's order (int32 signed, uint32 unsigned,
 * fp32 IEEE: a NaN on either side satisfies only DWS_PRED_NE, and -0.0 equals
 * +0.0). */
typedef enum dws_pred {
    DWS_PRED_EQ = 0,   /* x == t */
    DWS_PRED_NE = 1,   /* x != t */
    DWS_PRED_LT = 2,   /* x <  t */
    DWS_PRED_LE = 3,   /* x <= t */
    DWS_PRED_GT = 4,   /* x >  t */
    DWS_PRED_GE = 5    /* x >= t */
} dws_pred;

/*
 * Select-if (Merrill & Garland, section A5, select-if): dws_select_flagged
 * with the selection computed from the values themselves, x[i] `pred` t,
 * where t is the element the HOST pointer h_threshold points to (one element
 * of dtype, read during the call). The same single-pass kernel reads only the
 * values (4 bytes per element instead of 8): no flags array is materialised.
 * Results, in-place use (d_out == d_in allowed: a tile's count needs its values,
 * so every earlier tile has read its input before any write), the count word,
 * limits and errors are those of dws_select_flagged (d_flags aside); in
 * addition an unknown pred or h_threshold == NULL gives DWS_ERR_INVALID_ARG.
 */
dws_status dws_select_if(const void* d_in, void* d_out, size_t n, dws_dtype dtype, dws_pred pred,
                         const void* h_threshold, unsigned long long* d_count, hipStream_t stream);

/*
 * Partition-if (Merrill & Garland, section A5, partition-if):
 * dws_partition_flagged with the selection x[i] `pred` t computed from the
 * values, as dws_select_if. The selected elements go to the front in input
 * order, the others to the back in reverse input order; *d_num_selected is
 * their count. Never in place (DWS_ERR_OVERLAP), as dws_partition_flagged.
 */
dws_status dws_partition_if(const void* d_in, void* d_out, size_t n, dws_dtype dtype, dws_pred pred,
                            const void* h_threshold, unsigned long long* d_num_selected,
                            hipStream_t stream);

/*
 * Reduce by key (Merrill & Garland, section A5, reduce-by-key), one
 * single-pass launch: every maximal run of consecutive equal keys (compared
 * as 32-bit patterns, so +0.0 and -0.0 differ) gives its key in
 * d_unique_keys[r] and the + of its values in d_aggregates[r], runs in input
 * order; the number of runs goes to the DEVICE word *d_num_runs (64-bit,
 * 8-byte aligned). value_dtype DWS_INT32 / DWS_UINT32 sums wrap modulo 2^32,
 * DWS_FLOAT32 sums in fp32 (rounding order depends on scheduling). Arrays hold
 * n 4-byte elements (outputs need room for n); outputs must not overlap the
 * inputs, each other or the count word. n below 2^32. Elements of the outputs
 * at and past the number of runs are left unchanged.
 */
dws_status dws_reduce_by_key(const void* d_keys, const void* d_values, void* d_unique_keys,
                             void* d_aggregates, size_t n, dws_dtype value_dtype,
                             unsigned long long* d_num_runs, hipStream_t stream);

/*
 * Run-length encoding (Merrill & Garland, section A5, run-length-encode):
 * reduce-by-key with every value 1. d_lengths receives uint32 run lengths.
 * Same rules as dws_reduce_by_key.
 */
dws_status dws_run_length_encode(const void* d_keys, void* d_unique_keys, void* d_lengths, size_t n,
                                 unsigned long long* d_num_runs, hipStream_t stream);

/* Associative operators of dws_scan_op. The single pass only ever combines
 * contiguous inputs or contiguous partial results, earlier operand first, so
 * an operator need not be commutative (Merrill & Garland, section 4.2). */
typedef enum dws_op {
    /* +: int32/uint32 modulo 2^32 and fp32 (the scans above), and
     * componentwise on both pair types */
    DWS_OP_SUM = 0,
    /* max / min: DWS_INT32 (signed order) and DWS_UINT32 (unsigned order);
     * the exclusive scan starts with the type's lowest (max) or highest (min)
     * value */
    DWS_OP_MAX = 1,
    DWS_OP_MIN = 2,
    /* DWS_PAIR_U32 (a, b) is the map v -> a v + b modulo 2^32; element i of
     * the inclusive result is (A, B) with v_i = A s + B for the recurrence
     * v_i = a_i v_{i-1} + b_i, v_{-1} = s. Not commutative. Identity (1, 0). */
    DWS_OP_AFFINE = 3,
    /* (flag, value) pairs, DWS_PAIR_U32 or DWS_PAIR_I32_F32: a non-zero flag
     * starts a new segment, the value part sums within the segment, the flag
     * part is the OR of all flags so far. Not commutative. Identity (0, 0). */
    DWS_OP_SEGMENTED_SUM = 4
} dws_op;

/*
 * Inclusive (exclusive != 0: exclusive, identity first) scan of n elements of
 * `dtype` under `op`, one single-pass launch with decoupled look-back. Built
 * combinations: DWS_OP_SUM with every dtype (the 32-bit scalars take the
 * scan_inclusive / scan_exclusive path), DWS_OP_MAX / DWS_OP_MIN with
 * DWS_INT32 and DWS_UINT32, DWS_OP_AFFINE with DWS_PAIR_U32,
 * DWS_OP_SEGMENTED_SUM with both pair types; others give
 * DWS_ERR_UNSUPPORTED. Integer parts are exact; fp32 parts are rounded in an
 * order that depends on scheduling. d_out == d_in is allowed. Pointers must
 * be aligned to the element size (4 or 8 bytes); 16-byte aligned pointers
 * take the vector-load kernels. Same workspace, errors and asynchrony as
 * scan_inclusive.
 */
dws_status dws_scan_op(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                       dws_op op, int exclusive, hipStream_t stream);

/*
 * dws_scan_op with an initial value: the DEVICE element *d_seed (one element
 * of `dtype`: 4 bytes, or 8 for the pair types; 4-byte aligned) comes before
 * the whole array, as the earlier operand of every combine it enters. The
 * inclusive result is the scan of the sequence *d_seed, x[0], ..., x[n-1]
 * without its first element, the exclusive one that scan without its last
 * (so d_out[0] = *d_seed). For DWS_OP_AFFINE the seed map runs first, and for
 * DWS_OP_SEGMENTED_SUM it is the running value of a segment that x[0]
 * continues unless its flag is set. With dws_reduce_op for a shard's total,
 * it gives every operator the sharded scan that dws_reduce and
 * dws_scan_seeded give +. The seed enters as the prefix of tile
 * 0 (Merrill & Garland, section 4.2: only contiguous partial results are
 * combined, in input order); the other tiles receive it through the
 * look-back. DWS_OP_SUM with the 32-bit scalar types is dws_scan_seeded.
 * Validation and errors are those of dws_scan_op, then those of
 * dws_scan_seeded for d_seed (NULL: DWS_ERR_INVALID_ARG; not 4-byte aligned:
 * DWS_ERR_MISALIGNED; inside d_out's n elements: DWS_ERR_OVERLAP). n == 0 is a
 * no-op that does not read *d_seed. Asynchronous on `stream`.
 */
dws_status dws_scan_op_seeded(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                              dws_op op, int exclusive, const void* d_seed, hipStream_t stream);

/*
 * Reduction under `op`: writes the combination of x[0], ..., x[n-1] in input
 * order (the operator's identity when n == 0) to the DEVICE element *d_total
 * (one element of `dtype`, 4-byte aligned), the last element an inclusive
 * dws_scan_op would give. The first stage of the reduce-then-scan
 * decomposition (Merrill & Garland, section 3.2 and Fig 3) under any
 * associative operator (section 4.2): with dws_scan_op_seeded it shards every
 * operator's scan as dws_reduce and dws_scan_seeded shard +. One launch
 * reading the input once: the grid and the partials of dws_reduce, and every
 * combine in input order (within a wave segment, across a tile's waves,
 * along a workgroup's tiles and over the partials), so non-commutative
 * operators are exact; fp32 parts are added in an order fixed by n and the
 * input's alignment. Built combinations are those of dws_scan_op; DWS_OP_SUM
 * with the 32-bit scalar types is dws_reduce. Validation before any HIP call:
 * an unknown dtype or op, d_total == NULL, d_in == NULL with n > 0 or an
 * input range that wraps the address space give DWS_ERR_INVALID_ARG; other combinations, or n above DWS_MAX_ELEMENTS,
 * DWS_ERR_UNSUPPORTED; d_in not aligned to the element size or d_total not
 * 4-byte aligned DWS_ERR_MISALIGNED; d_total inside d_in's n elements
 * DWS_ERR_OVERLAP. Workspace, watchdog and asynchrony as dws_reduce.
 */
dws_status dws_reduce_op(const void* d_in, size_t n, dws_dtype dtype, dws_op op, void* d_total,
                         hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* dws_status_string(dws_status status);

/* Library version (DWS_VERSION). */
int dws_version(void);

/* ---- tile geometry (host only, no HIP call) ---------------------------- */

/* Number of tile_shape option values (0 = automatic, then forced shapes). */
int dws_num_tile_shapes(void);

/*
 * Elements per tile the single-pass kernel uses for a tile_shape option value,
 * n elements and an alignment class (aligned != 0: both pointers 16-byte
 * aligned). Returns 0 for an unknown shape.
 */
unsigned dws_tile_elems(int tile_shape, size_t n, int aligned);

/* Threads per workgroup for the same arguments (0 for an unknown shape). */
unsigned dws_tile_threads(int tile_shape, size_t n, int aligned);

/* ---- workspace ---------------------------------------------------------- */

/*
 * Create (or grow) the workspace of `stream` on the current device so that
 * scans, compactions and generic-operator scans of up to n elements, with any
 * variant or option, need no further allocation.
 */
dws_status dws_reserve(size_t n, hipStream_t stream);

/* Synchronise every device that holds a workspace and free every workspace
 * the library holds. Not to be called while another host thread is inside a
 * call of this library: that call may still be using a workspace. */
dws_status dws_release_workspaces(void);

/* ---- diagnostics (tests and benchmarks) --------------------------------- */

/*
 * Number of look-back waits on the current device that exceeded the safety
 * limit (about two seconds) since the library was loaded, over every
 * workspace and the array of dws_scan_noalloc. A correct run keeps it at 0.
 *
 * A trip means WRONG OUTPUT that no status reports: the calls are
 * asynchronous and have already returned DWS_OK when a wait times out. Rather
 * than hang the GPU, the waiting tile goes on with an incomplete prefix, so
 * the output of the call it belongs to (a scan, compaction, partition,
 * reduce-by-key, run-length encoding or operator scan) is wrong from that
 * tile on. Check this count after results that matter.
 *
 * Synchronous: it synchronises the current device first. When the count of a
 * workspace (or of the fixed array) has grown since the last check, this call
 * also clears that look-back state, so that no descriptor left behind by the
 * timed-out call can reach a later one; call it after a trip before relying on
 * further results. The count itself is never reset.
 */
dws_status dws_watchdog_trips(unsigned long long* trips);

/*
 * Memory clock (kHz), memory bus width (bits) and compute-unit count of the
 * current device, as the HIP runtime reports them, for stating the HBM
 * roofline beside measurements. Every pointer must be non-null
 * (DWS_ERR_INVALID_ARG); a failing runtime query returns DWS_ERR_HIP.
 */
dws_status dws_device_memory_info(int* memory_clock_khz, int* memory_bus_width_bits, int* compute_units);

/*
 * Protocol inspection kernel: the same descriptor protocol and look-back as
 * the single-pass scan, but with one wavefront per tile and a run-time tile
 * size of 1..64 elements, so that small inputs exercise many tiles and
 * look-back windows. Tiles whose index t satisfies t % delay_every ==
 * delay_phase (delay_every > 0) wait delay_ticks ticks of the 100 MHz
 * real-time counter before publishing their aggregate, which forces their
 * successors to observe the X and A states. If h_desc != NULL, the call
 * synchronises the stream and copies the num_tiles = ceil(n / tile_elems)
 * final descriptor words to host memory h_desc: bits 63..34 epoch, 33..32
 * status (0 X, 1 A, 2 P), 31..0 value bits (the tile's inclusive prefix once
 * P). With variant == DWS_VARIANT_CHAINED the look-back window is one tile.
 */
dws_status dws_scan_debug(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                          int exclusive, int variant, unsigned tile_elems,
                          unsigned delay_every, unsigned delay_phase,
                          unsigned delay_ticks, unsigned long long* h_desc,
                          hipStream_t stream);

/*
 * Instrumented single-pass scan, for measuring where a tile's time goes. Same
 * result as scan_inclusive / scan_exclusive with the automatic tile shape and
 * tile index source (relaxed descriptors; both pointers must be 16-byte
 * aligned, else DWS_ERR_UNSUPPORTED). In addition, for every tile t it writes
 * five 64-bit stamps of the 100 MHz real-time counter to the DEVICE buffer
 * d_stamps[5t .. 5t+4]: workgroup start, tile index known, aggregate
 * published (tile loaded and scanned), exclusive prefix known (look-back
 * done), stores issued. *num_tiles (if not NULL) receives the tile count;
 * with d_stamps == NULL the call only reports it. stamps_capacity is the
 * number of 64-bit words at d_stamps (at least 5 per tile). Asynchronous.
 */
dws_status dws_scan_profiled(const void* d_in, void* d_out, size_t n, dws_dtype dtype,
                             int exclusive, unsigned long long* d_stamps,
                             size_t stamps_capacity, unsigned* num_tiles,
                             hipStream_t stream);

/*
 * Wavefront primitive check: for each group of 64 elements g, writes the
 * in-wave inclusive scan to d_incl and the value of the previous lane (0 in
 * lane 0) to d_shift, exactly as the scan kernels compute them.
 * n_waves groups of 64 elements; dtype DWS_UINT32/DWS_INT32/DWS_FLOAT32.
 */
dws_status dws_selftest_wave(const void* d_in, void* d_incl, void* d_shift,
                             size_t n_waves, dws_dtype dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DWS_SCAN_H */

// Host-side interface between the C ABI (dws_abi.cpp) and the kernel
// launchers (dws_kernels_*.hip). Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dws_protocol.h"
#include "dws_scan.h"
#include "dws_single_pass.h"

namespace dws {

// Look-back state a launch with more than one tile needs: descriptors, tile
// counter, watchdog word and epoch word (a workspace, or the fixed device
// array of dws_scan_noalloc).
struct LookbackState {
    uint64_t* desc;
    uint64_t desc_slots;
    unsigned long long* counter;
    unsigned int* watchdog;
    unsigned int* epoch;
};

// The single-pass kernel and arguments a validated scan call runs with
// (dws_abi.cpp). params.desc, counter, watchdog and epoch are left empty;
// launch_single_pass_plan takes them from `state` (null for one tile, which
// touches none of them).
struct SinglePassPlan {
    int cfg;                  // index into kCfgs
    bool f32;
    bool exclusive;
    SinglePassParams params;
};
dws_status status_from_hip(hipError_t e);
dws_status validate_scan_args(const void* in, const void* out, size_t n, int dtype);
dws_status plan_single_pass(const void* in, void* out, size_t n, int dtype, bool excl, int mode,
                            const dws_options& o, unsigned long long* stamps, SinglePassPlan* plan);
hipError_t launch_single_pass_plan(const SinglePassPlan& plan, const LookbackState* state, hipStream_t stream);

// Watchdog count of the no-allocation entry point's array on `device` (0
// before that device's first multi-tile call), read after the caller has
// synchronised the device. When it has grown since the last check, the array's
// look-back state is cleared (the count is kept). dws_static.hip.
hipError_t static_check_trips(int device, unsigned int* trips);

// Workspace control block layout (one 256-byte allocation per workspace):
// the tile counter and the watchdog counter sit on separate cache lines.
constexpr size_t kCtlBytes = 256;
constexpr size_t kCtlCounterOffset = 0;
constexpr size_t kCtlWatchdogOffset = 128;
constexpr size_t kCtlEpochOffset = 192;

// Shape index (into kShapes) used for an option value (0 = automatic) and n.
// Pointers that are not both 16-byte aligned use the scalar-load version of
// the shape, or of the automatic shape if that one is not built.
int resolve_shape(int option_shape, uint64_t n, bool aligned);
// Index into kCfgs of the kernel for these parameters, or -1 if not built.
int find_single_pass_cfg(int shape, bool aligned, int order, int mode, bool nontemporal,
                         int tile_index = kTileDrawn, bool instr = false);

struct RtsArgs {
    const void* in;
    void* out;
    uint64_t n;
    int kind;
    bool exclusive;
    bool aligned;
    void* partials;        // >= groups elements
    uint32_t num_tiles;
    uint32_t groups;
    uint32_t tiles_per_group;
};
constexpr uint32_t kRtsTileElems = 4096u;
hipError_t launch_rts(const RtsArgs& a, hipStream_t stream);

// Device-wide + reduction to one element (dws_reduce.hip): G workgroups of
// kReduceThreads threads, each summing tiles_per_group consecutive tiles of
// kReduceTileElems elements and publishing the partial in its descriptor; the
// highest-indexed one adds the G partials. A look-back launch of the
// workspace: it reads the epoch word and advances it.
struct ReduceArgs {
    const void* in;
    uint64_t n;
    int kind;
    bool aligned;            // in is 16-byte aligned: dwordx4 loads
    bool nontemporal;        // non-temporal loads (aligned only)
    uint64_t* desc;          // >= groups descriptor slots
    unsigned int* epoch;     // the workspace epoch word
    unsigned int* watchdog;
    void* total;             // one element
    uint32_t num_tiles;
    uint32_t groups;
    uint32_t tiles_per_group;
};
constexpr int kReduceThreads = 512;
constexpr uint32_t kReduceTileElems = 16384u;
constexpr uint32_t kReduceMaxGroups = 1024u;
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);

// Scan-then-propagate: per-tile scans, recursive scan of the tile sums,
// propagation of the scanned sums (dws_stp.hip).
struct StpArgs {
    const void* in;
    void* out;
    uint64_t n;
    int kind;
    bool exclusive;
    void* scratch;          // >= stp_scratch_elems(n) elements (16-byte aligned)
    uint64_t scratch_elems;
};
constexpr uint32_t kStpTileElems = 4096u;
uint64_t stp_scratch_elems(uint64_t n);
hipError_t launch_stp(const StpArgs& a, hipStream_t stream);

// Stream compaction by flags (dws_select.hip).
struct SelectArgs {
    const void* in;
    const void* flags;
    void* out;
    uint64_t n;
    bool aligned;            // in, flags and out all 16-byte aligned
    uint64_t* desc;
    unsigned long long* counter;
    unsigned int* watchdog;
    unsigned long long* count;
    uint32_t num_tiles;
    unsigned int* epoch;     // the workspace epoch word
    bool partition;          // also write the rejected elements, reversed, at the back
    // predicate mode (flags unused): select v when bit c of pred_mask is set,
    // c the outcome of comparing v with threshold as `kind` (0 less, 1 equal,
    // 2 greater, 3 unordered)
    bool pred;
    uint32_t pred_mask;
    uint32_t threshold;
    int kind;                // kKindU32, kKindF32 or kPredKindI32
};
// Element kind of a predicate's comparison besides kKindU32 and kKindF32:
// signed 32-bit integers.
constexpr int kPredKindI32 = 2;
constexpr uint64_t kSelectLargeMin = (uint64_t)1 << 22;   // 32768-element tiles from here
constexpr uint64_t kSelectNtMin = (uint64_t)1 << 23;      // non-temporal loads (large shape) from here
constexpr uint64_t kSelectDrawnMin = (uint64_t)1 << 25;   // in-place select: drawn tile index from here
constexpr uint64_t kSelectMaxElems = 0xffffffffull;       // counts travel in 32-bit descriptors
// pause level between blocked look-back polls of the compaction kernels: the
// short pause at every size (64 units measured 2.3% slower on 2^30 - 12,345
// flags and 3.4% at 2^25, 127 units 0.7% and 7%)
constexpr uint32_t select_backoff(uint64_t) { return kPauseShort; }
uint32_t select_tile_elems(uint64_t n, bool aligned);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

struct DebugArgs {
    const void* in;
    void* out;
    uint64_t n;
    int kind;
    bool exclusive;
    int mode;
    uint32_t tile_elems;
    uint32_t delay_every, delay_phase, delay_ticks;
    uint64_t* desc;
    unsigned long long* counter;
    unsigned int* watchdog;
    uint32_t num_tiles;
    unsigned int* epoch;     // the workspace epoch word
};
hipError_t launch_debug(const DebugArgs& a, hipStream_t stream);

// Reduce-by-key / run-length encoding (dws_rbk.hip). mode: 0 integer sums,
// 1 fp32 sums, 2 run lengths (vals unused).
struct RbkArgs {
    const void* keys;
    const void* vals;
    void* ukeys;
    void* aggs;
    uint64_t n;
    int mode;
    bool aligned;            // keys (and vals) 16-byte aligned
    uint64_t* desc;          // >= 2 * num_tiles slots
    unsigned int* watchdog;
    unsigned long long* num_runs;
    uint32_t num_tiles;
    unsigned int* epoch;     // the workspace epoch word
};
constexpr uint64_t kRbkLargeMin = (uint64_t)1 << 22;   // 16384 (32768 for run lengths) from here
constexpr uint64_t kRbkNtMin = (uint64_t)1 << 25;      // non-temporal key and value loads from here
// pause level between blocked look-back polls of the run kernels: the short
// pause at every size (sleeping 64, 127 or 190 units measured 2 to 17% slower
// at 2^25 keys and up to 7% slower at 2^28)
constexpr uint32_t rbk_backoff(uint64_t) { return kPauseShort; }
uint32_t rbk_tile_elems(uint64_t n, bool aligned, int mode);
hipError_t launch_rbk(const RbkArgs& a, hipStream_t stream);

// Scan under a generic operator (dws_op_kernel.hpp). Kinds name an
// (operator, element type) pair; pair elements are two 32-bit words.
struct OpScanParams {
    const void* in;
    void* out;
    uint64_t n;                   // elements
    uint64_t* desc;               // >= words * num_tiles slots
    unsigned int* watchdog;
    uint32_t num_tiles;
    unsigned int* epoch;     // the workspace epoch word
    uint32_t backoff;        // pause level between blocked look-back polls (kPause*)
    const void* seed;        // one element (its words): tile 0's prefix (null: the identity)
};
// Reduction under an operator (k_reduce_op in dws_op_kernel.hpp): the grid of
// the + reduction (kReduceThreads threads, at most kReduceMaxGroups groups of
// tiles_per_group consecutive tiles).
struct OpReduceParams {
    const void* in;
    uint64_t n;                   // elements
    uint32_t num_tiles;
    uint32_t tiles_per_group;
    uint32_t groups;
    uint64_t* desc;               // >= groups descriptor slots
    unsigned int* epoch;          // the workspace epoch word
    unsigned int* watchdog;
    void* total;                  // one element (its words)
};
enum OpKind : int {
    kOpMaxI32, kOpMaxU32, kOpMinI32, kOpMinU32,          // one word
    kOpSumPairIF, kOpSumPairU32, kOpAffineU32, kOpSegSumIF, kOpSegSumU32,   // two words
    kNumOpKinds
};
constexpr int op_kind_words(int kind) { return kind <= kOpMinU32 ? 1 : 2; }
// Shapes (threads x words per load x loads per lane): small 256 x 4 x 4,
// medium 512 x 4 x 8, large 1024 x 4 x 16, unaligned 256 x (one element) x 16.
constexpr int kOpShapeSmall = 0;
constexpr int kOpShapeMedium = 1;
constexpr int kOpShapeLarge = 2;
constexpr int kOpShapeUnaligned = 3;
constexpr uint64_t kOpMediumMin = (uint64_t)1 << 20;
constexpr uint64_t kOpNtMin = (uint64_t)1 << 25;       // non-temporal loads (large shape) from here
// pause level between blocked look-back polls of the generic-operator kernels:
// the short pause at every size (with the workgroup index it measured 1.3 to
// 1.6% faster than the 64-unit sleep on 1 GiB inputs)
constexpr uint32_t op_backoff(uint64_t) { return kPauseShort; }
constexpr uint64_t kOpLargeMin = (uint64_t)1 << 24;
constexpr int op_auto_shape(uint64_t n, bool aligned)
{
    return !aligned ? kOpShapeUnaligned : (n >= kOpLargeMin ? kOpShapeLarge : (n >= kOpMediumMin ? kOpShapeMedium
                                                                                                   : kOpShapeSmall));
}
constexpr uint32_t op_tile_elems(int words, int shape)
{
    return shape == kOpShapeSmall    ? 256u * (4u / words) * 4u
           : shape == kOpShapeMedium ? 512u * (4u / words) * 8u
           : shape == kOpShapeLarge  ? 1024u * (4u / words) * 16u
                                     : 256u * 16u;
}
constexpr uint32_t op_tile_threads(int shape)
{
    return shape == kOpShapeMedium ? 512u : (shape == kOpShapeLarge ? 1024u : 256u);
}
// Elements per tile of the reduction under an operator: kReduceThreads threads
// loading 4 words 8 times (16-byte aligned input) or one element 16 times.
constexpr uint32_t op_reduce_tile_elems(int words, bool aligned)
{
    return aligned ? (uint32_t)kReduceThreads * (4u / words) * 8u : (uint32_t)kReduceThreads * 16u;
}
// Reductions under the operators of each file (k_reduce_op), non-temporal
// loads as asked (aligned inputs only).
hipError_t launch_reduce_op_minmax(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream);
hipError_t launch_reduce_op_pairsum(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream);
hipError_t launch_reduce_op_affine(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream);
hipError_t launch_reduce_op_segsum(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream);
// The tile index is the workgroup index; only the large shape is built with
// non-temporal loads (used from kOpNtMin elements).
hipError_t launch_op_minmax(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                            hipStream_t stream);
hipError_t launch_op_pairsum(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                             hipStream_t stream);
hipError_t launch_op_affine(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                            hipStream_t stream);
hipError_t launch_op_segsum(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                            hipStream_t stream);

// Zero `slots` descriptors, set the counter to kCounterInit, the epoch word
// to 1 and the watchdog to 0 (each pointer may be null; a kernel, not a
// memset, so that it may sit in a graph).
hipError_t launch_workspace_init(uint64_t* desc, uint64_t slots, unsigned long long* counter,
                                 unsigned int* epoch, unsigned int* watchdog, hipStream_t stream);

hipError_t launch_wave_selftest(const void* in, void* incl, void* shift, uint64_t n_waves,
                                int kind, hipStream_t stream);

}  // namespace dws

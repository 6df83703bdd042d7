// C ABI of the scan library: argument validation, per-(device, stream)
// workspaces and dispatch to the kernel launchers. Declarations and the full
// contract are in include/dws_scan.h.
#include "dws_scan.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "dws_internal.h"

namespace {

using namespace dws;

constexpr size_t kElemBytes = 4;
constexpr uint64_t kMinDescSlots = (uint64_t)8192 * kDescStride;   // descriptors for 8,192 tiles
constexpr unsigned kMaxDebugDelayTicks = 50000000u;  // 0.5 s of the 100 MHz clock
constexpr uint64_t kMaxGridThreads = (1ull << 32) - 1ull;

struct Workspace {
    int device = 0;
    hipStream_t stream = nullptr;
    std::mutex mu;
    void* ctl = nullptr;          // counter + watchdog (kCtlBytes)
    uint64_t* desc = nullptr;     // descriptor slots
    uint64_t desc_slots = 0;
    void* partials = nullptr;     // reduce-then-scan partials (kRtsMaxGroups x 4 B)
    void* stp = nullptr;          // scan-then-propagate tile sums (all levels)
    uint64_t stp_elems = 0;
    uint32_t launches = 0;        // look-back launches issued since the descriptors were cleared
    unsigned int trips_seen = 0;  // watchdog count when dws_watchdog_trips last cleared the state

    unsigned long long* counter() const
    {
        return reinterpret_cast<unsigned long long*>(static_cast<char*>(ctl) + kCtlCounterOffset);
    }
    unsigned int* watchdog() const
    {
        return reinterpret_cast<unsigned int*>(static_cast<char*>(ctl) + kCtlWatchdogOffset);
    }
    unsigned int* epoch() const { return reinterpret_cast<unsigned int*>(static_cast<char*>(ctl) + kCtlEpochOffset); }
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Workspace>> g_workspaces;
std::map<int, int> g_cu_count;

dws_status from_hip(hipError_t e)
{
    if (e == hipSuccess) return DWS_OK;
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return DWS_ERR_OOM;
    return DWS_ERR_HIP;
}

bool valid_dtype(int d) { return d == DWS_INT32 || d == DWS_UINT32 || d == DWS_FLOAT32; }

// The value a C caller passed in an enum parameter, read from its bytes. A C
// caller may pass any int there, and in C++ reading an enum object whose value
// is outside the enum's range is undefined, so the ABI reads these parameters
// only as the int they hold. The parameter is taken by reference: copying it
// by value would itself be such a read.
template <class E>
int enum_arg(const E& e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums travel as int");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

// All checks on the data pointers that need no HIP call, for elements of
// `esize` bytes. n == 0 is accepted with any pointers.
dws_status validate_sized(const void* in, const void* out, size_t n, size_t esize)
{
    if (n == 0) return DWS_OK;
    if (in == nullptr || out == nullptr) return DWS_ERR_INVALID_ARG;
    if (n > DWS_MAX_ELEMENTS) return DWS_ERR_UNSUPPORTED;
    const uintptr_t a = reinterpret_cast<uintptr_t>(in);
    const uintptr_t b = reinterpret_cast<uintptr_t>(out);
    if ((a % esize) != 0 || (b % esize) != 0) return DWS_ERR_MISALIGNED;
    const uintptr_t bytes = (uintptr_t)n * esize;
    if (a + bytes < a || b + bytes < b) return DWS_ERR_INVALID_ARG;
    if (a != b && a < b + bytes && b < a + bytes) return DWS_ERR_OVERLAP;
    return DWS_OK;
}

dws_status validate(const void* in, const void* out, size_t n, int dtype)
{
    if (!valid_dtype(dtype)) return DWS_ERR_INVALID_ARG;
    return validate_sized(in, out, n, kElemBytes);
}

int kind_of(int dtype) { return dtype == DWS_FLOAT32 ? kKindF32 : kKindU32; }

// The seed of a seeded scan: one element of `esize` bytes, 4-byte aligned,
// outside the output's n elements (tile 0 reads it before it publishes and
// every store of the call follows that publication, but an output range that
// held the seed would still be a caller's error, so it is refused outright).
dws_status check_seed(const void* seed, const void* out, size_t n, size_t esize)
{
    if (seed == nullptr) return DWS_ERR_INVALID_ARG;
    const uintptr_t sd = reinterpret_cast<uintptr_t>(seed);
    if (sd % kElemBytes != 0) return DWS_ERR_MISALIGNED;
    const uintptr_t ob = reinterpret_cast<uintptr_t>(out);
    if (sd + esize < sd) return DWS_ERR_INVALID_ARG;
    if (sd + esize > ob && sd < ob + (uintptr_t)n * esize) return DWS_ERR_OVERLAP;
    return DWS_OK;
}

bool aligned16(const void* in, const void* out)
{
    return ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15u) == 0;
}

uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Workspace of (current device, stream), created on first use.
// True while `stream` is being captured into a graph. Nothing may be allocated
// or synchronised then, so a call that would have to create or grow a
// workspace returns DWS_ERR_UNSUPPORTED before making any such call (and the
// capture stays valid); dws_reserve ahead of the capture avoids it.
bool stream_capturing(hipStream_t stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

dws_status get_workspace(hipStream_t stream, Workspace** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e);
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = std::make_pair(dev, stream);
    auto it = g_workspaces.find(key);
    if (it != g_workspaces.end()) {
        *out = it->second.get();
        return DWS_OK;
    }
    if (stream_capturing(stream)) return DWS_ERR_UNSUPPORTED;
    auto ws = std::make_unique<Workspace>();
    ws->device = dev;
    ws->stream = stream;
    e = hipMalloc(&ws->ctl, kCtlBytes);
    if (e != hipSuccess) return from_hip(e);
    e = hipMalloc(&ws->partials, (size_t)kRtsMaxGroups * kElemBytes);
    if (e != hipSuccess) {
        (void)hipFree(ws->ctl);
        return from_hip(e);
    }
    e = launch_workspace_init(nullptr, 0, ws->counter(), ws->epoch(), ws->watchdog(), stream);
    if (e != hipSuccess) {
        (void)hipFree(ws->ctl);
        (void)hipFree(ws->partials);
        return from_hip(e);
    }
    *out = ws.get();
    g_workspaces.emplace(key, std::move(ws));
    return DWS_OK;
}

// Grow the descriptor array to at least `slots` (call with ws->mu held). A new
// array is cleared by a kernel on the workspace's stream; the old one is freed
// once the stream has drained, since kernels in flight may still use it.
dws_status ensure_desc(Workspace* ws, uint64_t slots)
{
    if (slots <= ws->desc_slots) return DWS_OK;
    if (stream_capturing(ws->stream)) return DWS_ERR_UNSUPPORTED;
    uint64_t want = std::max<uint64_t>({slots, ws->desc_slots * 2, kMinDescSlots});
    if (ws->desc != nullptr) {
        hipError_t e = hipStreamSynchronize(ws->stream);
        if (e != hipSuccess) return from_hip(e);
        (void)hipFree(ws->desc);
        ws->desc = nullptr;
        ws->desc_slots = 0;
    }
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, want * sizeof(uint64_t));
    if (e != hipSuccess) return from_hip(e);
    // fresh zeroed descriptors (all X for every epoch), a zero counter, epoch 1
    e = launch_workspace_init(static_cast<uint64_t*>(p), want, ws->counter(), ws->epoch(), nullptr, ws->stream);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return from_hip(e);
    }
    ws->desc = static_cast<uint64_t*>(p);
    ws->desc_slots = want;
    ws->launches = 0;
    return DWS_OK;
}

// Before a look-back launch on the workspace (call with ws->mu held). Every
// launch reads its descriptor epoch from the workspace's epoch word and
// advances it, so descriptors left by earlier launches read as X. The epochs
// wrap after kEpochMax launches: before that, every descriptor is cleared and
// the word goes back to 1, so no word of an old launch can carry a reused
// epoch. (Replays of a captured launch advance the word too, without passing
// here; they count towards the same limit.)
dws_status before_lookback_launch(Workspace* ws)
{
    if (ws->launches + 1u >= kEpochMax) {
        hipError_t e = launch_workspace_init(ws->desc, ws->desc_slots, ws->counter(), ws->epoch(), nullptr,
                                             ws->stream);
        if (e != hipSuccess) return from_hip(e);
        ws->launches = 0;
    }
    ++ws->launches;
    return DWS_OK;
}

int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_cu_count.find(dev);
    if (it != g_cu_count.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cu_count[dev] = cus;
    return cus;
}

}  // namespace

namespace dws {

dws_status status_from_hip(hipError_t e) { return from_hip(e); }

dws_status validate_scan_args(const void* in, const void* out, size_t n, int dtype)
{
    return validate(in, out, n, dtype);
}

dws_status plan_single_pass(const void* in, void* out, size_t n, int dtype, bool excl, int mode,
                            const dws_options& o, unsigned long long* stamps, SinglePassPlan* plan)
{
    const bool aligned = aligned16(in, out);
    // non-temporal loads are a hint, built for aligned pointers only: 1 asks
    // for them, 2 never uses them, 0 leaves it to the library, which uses them
    // on the automatic relaxed single pass from kNtLoadMin elements
    bool nt = false;
    if (o.nontemporal == 1) {
        nt = aligned;
    } else if (o.nontemporal == 0) {
        nt = aligned && n >= kNtLoadMin && o.tile_shape == 0 && mode == kModeDecoupled &&
             o.memory_order == DWS_ORDER_RELAXED;
    }
    const int shape = resolve_shape(o.tile_shape, n, aligned);
    if (shape < 0) return DWS_ERR_INVALID_ARG;
    // automatic: the workgroup index where that kernel is built (relaxed
    // decoupled look-back)
    int tile_index = o.tile_index == DWS_TILE_DISPATCH ? kTileDispatch : kTileDrawn;
    if (o.tile_index == DWS_TILE_AUTO && mode == kModeDecoupled && o.memory_order == DWS_ORDER_RELAXED)
        tile_index = auto_tile_index(n);
    const bool instr = stamps != nullptr;
    int cfg = find_single_pass_cfg(shape, aligned, o.memory_order, mode, nt, tile_index, instr);
    // the workgroup index has non-temporal kernels for the 32,768- and
    // 65,536-element tiles only: elsewhere non-temporal loads asked for with
    // the automatic tile index take the drawn index, and the library's own
    // choice with a forced workgroup index drops them
    if (cfg < 0 && nt && tile_index == kTileDispatch) {
        if (o.tile_index == DWS_TILE_AUTO) tile_index = kTileDrawn;
        else if (o.nontemporal == 0) nt = false;
        cfg = find_single_pass_cfg(shape, aligned, o.memory_order, mode, nt, tile_index, instr);
    }
    if (cfg < 0) return DWS_ERR_UNSUPPORTED;
    const TileShape ts = cfg_shape(kCfgs[cfg]);
    const uint64_t num_tiles = ceil_div(n, (uint64_t)ts.elems());
    if (num_tiles > 0xffffffffull || num_tiles * (uint64_t)ts.threads > kMaxGridThreads) return DWS_ERR_UNSUPPORTED;

    SinglePassParams p{};
    p.in = in;
    p.out = out;
    p.n = n;
    p.num_tiles = (uint32_t)num_tiles;
    p.stamps = stamps;
    p.backoff = scan_backoff(n, kCfgs[cfg].tile_index);
    plan->cfg = cfg;
    plan->f32 = kind_of(dtype) == kKindF32;
    plan->exclusive = excl;
    plan->params = p;
    return DWS_OK;
}

hipError_t launch_single_pass_plan(const SinglePassPlan& plan, const LookbackState* state, hipStream_t stream)
{
    SinglePassParams p = plan.params;
    if (state != nullptr) {
        p.desc = state->desc;
        p.counter = state->counter;
        p.watchdog = state->watchdog;
        p.epoch = state->epoch;
    }
    return plan.f32 ? launch_single_pass_typed<float>(plan.cfg, plan.exclusive, p, stream)
                    : launch_single_pass_typed<uint32_t>(plan.cfg, plan.exclusive, p, stream);
}

}  // namespace dws

namespace {

dws_status run_single_pass(const void* in, void* out, size_t n, int dtype, bool excl, int mode,
                           const dws_options& o, hipStream_t stream, unsigned long long* stamps = nullptr,
                           const void* seed = nullptr)
{
    SinglePassPlan plan{};
    dws_status s = plan_single_pass(in, out, n, dtype, excl, mode, o, stamps, &plan);
    if (s != DWS_OK) return s;
    plan.params.seed = seed;
    // one tile: no predecessors, no descriptors, no counter
    if (plan.params.num_tiles == 1) return from_hip(launch_single_pass_plan(plan, nullptr, stream));
    Workspace* ws = nullptr;
    s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    s = ensure_desc(ws, (uint64_t)plan.params.num_tiles * kDescStride);
    if (s != DWS_OK) return s;
    s = before_lookback_launch(ws);
    if (s != DWS_OK) return s;
    const LookbackState st{ws->desc, ws->desc_slots, ws->counter(), ws->watchdog(), ws->epoch()};
    return from_hip(launch_single_pass_plan(plan, &st, stream));
}

dws_status run_rts(const void* in, void* out, size_t n, int dtype, bool excl, hipStream_t stream)
{
    const bool aligned = aligned16(in, out);
    const uint64_t tile = kRtsTileElems;
    const uint64_t num_tiles = ceil_div(n, tile);
    if (num_tiles > 0xffffffffull) return DWS_ERR_UNSUPPORTED;
    uint64_t groups = std::min<uint64_t>({num_tiles, (uint64_t)cu_count() * 8u, (uint64_t)kRtsMaxGroups});
    const uint64_t tpg = ceil_div(num_tiles, groups);
    groups = ceil_div(num_tiles, tpg);
    Workspace* ws = nullptr;
    dws_status s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    RtsArgs a{};
    a.in = in;
    a.out = out;
    a.n = n;
    a.kind = kind_of(dtype);
    a.exclusive = excl;
    a.aligned = aligned;
    a.partials = ws->partials;
    a.num_tiles = (uint32_t)num_tiles;
    a.groups = (uint32_t)groups;
    a.tiles_per_group = (uint32_t)tpg;
    return from_hip(launch_rts(a, stream));
}

// Device-wide + reduction into one element (validated arguments). The grid
// depends on n only: at most kReduceMaxGroups workgroups, each summing the
// same number of consecutive tiles.
dws_status run_reduce(const void* in, size_t n, int dtype, void* total, hipStream_t stream)
{
    const uint64_t num_tiles = ceil_div(n, kReduceTileElems);
    if (num_tiles > 0xffffffffull) return DWS_ERR_UNSUPPORTED;
    uint64_t groups = std::max<uint64_t>(1u, std::min<uint64_t>(num_tiles, kReduceMaxGroups));
    const uint64_t tpg = ceil_div(num_tiles, groups);
    if (tpg > 0) groups = ceil_div(num_tiles, tpg);
    Workspace* ws = nullptr;
    dws_status s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    s = ensure_desc(ws, groups * kDescStride);
    if (s != DWS_OK) return s;
    s = before_lookback_launch(ws);
    if (s != DWS_OK) return s;
    ReduceArgs a{};
    a.in = in;
    a.n = n;
    a.kind = kind_of(dtype);
    a.aligned = (reinterpret_cast<uintptr_t>(in) & 15u) == 0;
    // each input word is read once, as in the scan's tiles
    a.nontemporal = a.aligned && n >= kNtLoadMin;
    a.desc = ws->desc;
    a.epoch = ws->epoch();
    a.watchdog = ws->watchdog();
    a.total = total;
    a.num_tiles = (uint32_t)num_tiles;
    a.groups = (uint32_t)groups;
    a.tiles_per_group = (uint32_t)tpg;
    return from_hip(launch_reduce(a, stream));
}

// Grow the scan-then-propagate scratch (call with ws->mu held).
dws_status ensure_stp(Workspace* ws, uint64_t elems)
{
    if (elems <= ws->stp_elems) return DWS_OK;
    if (stream_capturing(ws->stream)) return DWS_ERR_UNSUPPORTED;
    const uint64_t want = std::max<uint64_t>({elems, ws->stp_elems * 2, 1024});
    if (ws->stp != nullptr) {
        hipError_t e = hipStreamSynchronize(ws->stream);
        if (e != hipSuccess) return from_hip(e);
        (void)hipFree(ws->stp);
        ws->stp = nullptr;
        ws->stp_elems = 0;
    }
    hipError_t e = hipMalloc(&ws->stp, want * kElemBytes);
    if (e != hipSuccess) return from_hip(e);
    ws->stp_elems = want;
    return DWS_OK;
}

dws_status run_stp(const void* in, void* out, size_t n, int dtype, bool excl, hipStream_t stream)
{
    StpArgs a{};
    a.in = in;
    a.out = out;
    a.n = n;
    a.kind = kind_of(dtype);
    a.exclusive = excl;
    const uint64_t need = stp_scratch_elems(n);
    if (need == 0) return from_hip(launch_stp(a, stream));
    Workspace* ws = nullptr;
    dws_status s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    s = ensure_stp(ws, need);
    if (s != DWS_OK) return s;
    a.scratch = ws->stp;
    a.scratch_elems = ws->stp_elems;
    return from_hip(launch_stp(a, stream));
}

// Options checked before the arguments: unknown values are invalid, a tile
// index source other than automatic exists for the single pass and the
// chained scan only.
dws_status check_options(const dws_options& o)
{
    if (o.variant < DWS_VARIANT_SINGLE_PASS || o.variant > DWS_VARIANT_SCAN_THEN_PROPAGATE) return DWS_ERR_INVALID_ARG;
    if (o.memory_order != DWS_ORDER_RELAXED && o.memory_order != DWS_ORDER_ACQ_REL) return DWS_ERR_INVALID_ARG;
    if (o.tile_shape < 0 || o.tile_shape > kNumShapes) return DWS_ERR_INVALID_ARG;
    if (o.nontemporal < 0 || o.nontemporal > 2) return DWS_ERR_INVALID_ARG;
    if (o.tile_index < DWS_TILE_AUTO || o.tile_index > DWS_TILE_DISPATCH) return DWS_ERR_INVALID_ARG;
    if (o.tile_index != DWS_TILE_AUTO && o.variant != DWS_VARIANT_SINGLE_PASS && o.variant != DWS_VARIANT_CHAINED)
        return DWS_ERR_UNSUPPORTED;
    return DWS_OK;
}

dws_status scan_entry(const void* in, void* out, size_t n, int dtype, int exclusive, const dws_options* opt,
                      hipStream_t stream)
{
    try {
        dws_options o{};
        if (opt != nullptr) o = *opt;
        dws_status s = check_options(o);
        if (s != DWS_OK) return s;
        s = validate(in, out, n, dtype);
        if (s != DWS_OK || n == 0) return s;
        const bool excl = exclusive != 0;
        switch (o.variant) {
        case DWS_VARIANT_REDUCE_THEN_SCAN:
            if (o.tile_shape != 0 || o.nontemporal == 1) return DWS_ERR_UNSUPPORTED;
            return run_rts(in, out, n, dtype, excl, stream);
        case DWS_VARIANT_CHAINED:
            return run_single_pass(in, out, n, dtype, excl, kModeChained, o, stream);
        case DWS_VARIANT_SCAN_THEN_PROPAGATE:
            if (o.tile_shape != 0 || o.nontemporal == 1) return DWS_ERR_UNSUPPORTED;
            return run_stp(in, out, n, dtype, excl, stream);
        default:
            return run_single_pass(in, out, n, dtype, excl, kModeDecoupled, o, stream);
        }
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

// (operator, element type) -> kernel kind, or -1 where none is built.
int op_kind(int dtype, int op)
{
    switch (op) {
    case DWS_OP_MAX: return dtype == DWS_INT32 ? kOpMaxI32 : (dtype == DWS_UINT32 ? kOpMaxU32 : -1);
    case DWS_OP_MIN: return dtype == DWS_INT32 ? kOpMinI32 : (dtype == DWS_UINT32 ? kOpMinU32 : -1);
    case DWS_OP_SUM: return dtype == DWS_PAIR_I32_F32 ? kOpSumPairIF : (dtype == DWS_PAIR_U32 ? kOpSumPairU32 : -1);
    case DWS_OP_AFFINE: return dtype == DWS_PAIR_U32 ? kOpAffineU32 : -1;
    case DWS_OP_SEGMENTED_SUM:
        return dtype == DWS_PAIR_I32_F32 ? kOpSegSumIF : (dtype == DWS_PAIR_U32 ? kOpSegSumU32 : -1);
    default: return -1;
    }
}

hipError_t launch_op_kind(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p, hipStream_t stream)
{
    switch (kind) {
    case kOpMaxI32:
    case kOpMaxU32:
    case kOpMinI32:
    case kOpMinU32: return launch_op_minmax(kind, exclusive, shape, nt, p, stream);
    case kOpSumPairIF:
    case kOpSumPairU32: return launch_op_pairsum(kind, exclusive, shape, nt, p, stream);
    case kOpAffineU32: return launch_op_affine(kind, exclusive, shape, nt, p, stream);
    case kOpSegSumIF:
    case kOpSegSumU32: return launch_op_segsum(kind, exclusive, shape, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce_op_kind(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream)
{
    switch (kind) {
    case kOpMaxI32:
    case kOpMaxU32:
    case kOpMinI32:
    case kOpMinU32: return launch_reduce_op_minmax(kind, aligned, nt, p, stream);
    case kOpSumPairIF:
    case kOpSumPairU32: return launch_reduce_op_pairsum(kind, aligned, nt, p, stream);
    case kOpAffineU32: return launch_reduce_op_affine(kind, aligned, nt, p, stream);
    case kOpSegSumIF:
    case kOpSegSumU32: return launch_reduce_op_segsum(kind, aligned, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

// Reduction under an operator into one element (validated arguments): the
// grid of run_reduce, with the operator's tile size.
dws_status run_reduce_op(const void* in, size_t n, int kind, void* total, hipStream_t stream)
{
    const int words = op_kind_words(kind);
    const bool aligned = (reinterpret_cast<uintptr_t>(in) & 15u) == 0;
    const uint64_t num_tiles = ceil_div(n, op_reduce_tile_elems(words, aligned));
    if (num_tiles > 0xffffffffull) return DWS_ERR_UNSUPPORTED;
    uint64_t groups = std::max<uint64_t>(1u, std::min<uint64_t>(num_tiles, kReduceMaxGroups));
    const uint64_t tpg = ceil_div(num_tiles, groups);
    if (tpg > 0) groups = ceil_div(num_tiles, tpg);
    Workspace* ws = nullptr;
    dws_status s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    s = ensure_desc(ws, groups * kDescStride);
    if (s != DWS_OK) return s;
    s = before_lookback_launch(ws);
    if (s != DWS_OK) return s;
    OpReduceParams p{};
    p.in = in;
    p.n = n;
    p.num_tiles = (uint32_t)num_tiles;
    p.tiles_per_group = (uint32_t)tpg;
    p.groups = (uint32_t)groups;
    p.desc = ws->desc;
    p.epoch = ws->epoch();
    p.watchdog = ws->watchdog();
    p.total = total;
    // each input word is read once, as in the operator scans' tiles
    return from_hip(launch_reduce_op_kind(kind, aligned, aligned && n >= kOpNtMin, p, stream));
}

dws_status run_scan_op(const void* in, void* out, size_t n, int kind, bool excl, hipStream_t stream,
                       const void* seed = nullptr)
{
    const int words = op_kind_words(kind);
    const bool aligned = aligned16(in, out);
    const int shape = op_auto_shape(n, aligned);
    // The tile index is the workgroup index. Non-temporal loads from kOpNtMin
    // elements (the large shape): each input word is read once. With a drawn
    // index they measured 2 to 3% faster on 128 and 256 MB inputs, 4.6 to
    // 5.1% on 512 MB and 1 GiB; the workgroup index with them (and the short
    // pause) then measured 5.6 to 7.3% faster than the drawn index with them
    // on 1 GiB inputs (three alternating runs of whole library builds).
    const bool nt = shape == kOpShapeLarge && n >= kOpNtMin;
    const uint64_t num_tiles = ceil_div(n, op_tile_elems(words, shape));
    if (num_tiles > 0xffffffffull || num_tiles * op_tile_threads(shape) > kMaxGridThreads)
        return DWS_ERR_UNSUPPORTED;
    OpScanParams p{};
    p.in = in;
    p.out = out;
    p.n = n;
    p.num_tiles = (uint32_t)num_tiles;
    p.backoff = op_backoff(n);
    p.seed = seed;
    if (num_tiles == 1) return from_hip(launch_op_kind(kind, excl, shape, false, p, stream));
    Workspace* ws = nullptr;
    dws_status s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    s = ensure_desc(ws, num_tiles * kDescStride);
    if (s != DWS_OK) return s;
    s = before_lookback_launch(ws);
    if (s != DWS_OK) return s;
    p.epoch = ws->epoch();
    p.desc = ws->desc;
    p.watchdog = ws->watchdog();
    return from_hip(launch_op_kind(kind, excl, shape, nt, p, stream));
}

}  // namespace

extern "C" {

dws_status dws_scan_op(const void* d_in, void* d_out, size_t n, dws_dtype dtype, dws_op op, int exclusive,
                       hipStream_t stream)
{
    try {
        const int dt = enum_arg(dtype), o = enum_arg(op);
        if (dt < DWS_INT32 || dt > DWS_PAIR_U32) return DWS_ERR_INVALID_ARG;
        if (o < DWS_OP_SUM || o > DWS_OP_SEGMENTED_SUM) return DWS_ERR_INVALID_ARG;
        if (o == DWS_OP_SUM && valid_dtype(dt))
            return scan_entry(d_in, d_out, n, dt, exclusive, nullptr, stream);
        const int kind = op_kind(dt, o);
        if (kind < 0) return DWS_ERR_UNSUPPORTED;
        const dws_status s = validate_sized(d_in, d_out, n, 4u * (size_t)op_kind_words(kind));
        if (s != DWS_OK || n == 0) return s;
        return run_scan_op(d_in, d_out, n, kind, exclusive != 0, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status scan_inclusive(const void* d_in, void* d_out, size_t n, dws_dtype dtype, hipStream_t stream)
{
    return scan_entry(d_in, d_out, n, enum_arg(dtype), 0, nullptr, stream);
}

dws_status scan_exclusive(const void* d_in, void* d_out, size_t n, dws_dtype dtype, hipStream_t stream)
{
    return scan_entry(d_in, d_out, n, enum_arg(dtype), 1, nullptr, stream);
}

dws_status dws_scan_ex(const void* d_in, void* d_out, size_t n, dws_dtype dtype, int exclusive, int variant,
                       hipStream_t stream)
{
    dws_options o{};
    o.variant = variant;
    return scan_entry(d_in, d_out, n, enum_arg(dtype), exclusive, &o, stream);
}

dws_status dws_scan_opts(const void* d_in, void* d_out, size_t n, dws_dtype dtype, int exclusive,
                         const dws_options* opt, hipStream_t stream)
{
    return scan_entry(d_in, d_out, n, enum_arg(dtype), exclusive, opt, stream);
}

dws_status dws_scan_seeded(const void* d_in, void* d_out, size_t n, dws_dtype dtype, int exclusive,
                           const void* d_seed, hipStream_t stream)
{
    try {
        const int dt = enum_arg(dtype);
        dws_status s = validate(d_in, d_out, n, dt);
        if (s != DWS_OK || n == 0) return s;
        s = check_seed(d_seed, d_out, n, kElemBytes);
        if (s != DWS_OK) return s;
        const dws_options o{};
        return run_single_pass(d_in, d_out, n, dt, exclusive != 0, kModeDecoupled, o, stream, nullptr, d_seed);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_scan_op_seeded(const void* d_in, void* d_out, size_t n, dws_dtype dtype, dws_op op, int exclusive,
                              const void* d_seed, hipStream_t stream)
{
    try {
        const int dt = enum_arg(dtype), o = enum_arg(op);
        if (dt < DWS_INT32 || dt > DWS_PAIR_U32) return DWS_ERR_INVALID_ARG;
        if (o < DWS_OP_SUM || o > DWS_OP_SEGMENTED_SUM) return DWS_ERR_INVALID_ARG;
        if (o == DWS_OP_SUM && valid_dtype(dt))
            return dws_scan_seeded(d_in, d_out, n, dtype, exclusive, d_seed, stream);
        const int kind = op_kind(dt, o);
        if (kind < 0) return DWS_ERR_UNSUPPORTED;
        const size_t esize = 4u * (size_t)op_kind_words(kind);
        dws_status s = validate_sized(d_in, d_out, n, esize);
        if (s != DWS_OK || n == 0) return s;
        s = check_seed(d_seed, d_out, n, esize);
        if (s != DWS_OK) return s;
        return run_scan_op(d_in, d_out, n, kind, exclusive != 0, stream, d_seed);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_reduce(const void* d_in, size_t n, dws_dtype dtype, void* d_total, hipStream_t stream)
{
    try {
        const int dt = enum_arg(dtype);
        if (!valid_dtype(dt)) return DWS_ERR_INVALID_ARG;
        if (d_total == nullptr || (n > 0 && d_in == nullptr)) return DWS_ERR_INVALID_ARG;
        if (n > DWS_MAX_ELEMENTS) return DWS_ERR_UNSUPPORTED;
        const uintptr_t a = reinterpret_cast<uintptr_t>(d_in);
        const uintptr_t t = reinterpret_cast<uintptr_t>(d_total);
        if (a % kElemBytes != 0 || t % kElemBytes != 0) return DWS_ERR_MISALIGNED;
        if (a + (uintptr_t)n * kElemBytes < a || t + kElemBytes < t) return DWS_ERR_INVALID_ARG;
        if (n > 0 && t + kElemBytes > a && t < a + (uintptr_t)n * kElemBytes) return DWS_ERR_OVERLAP;
        return run_reduce(d_in, n, dt, d_total, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_reduce_op(const void* d_in, size_t n, dws_dtype dtype, dws_op op, void* d_total,
                         hipStream_t stream)
{
    try {
        const int dt = enum_arg(dtype), o = enum_arg(op);
        if (dt < DWS_INT32 || dt > DWS_PAIR_U32) return DWS_ERR_INVALID_ARG;
        if (o < DWS_OP_SUM || o > DWS_OP_SEGMENTED_SUM) return DWS_ERR_INVALID_ARG;
        if (o == DWS_OP_SUM && valid_dtype(dt)) return dws_reduce(d_in, n, dtype, d_total, stream);
        const int kind = op_kind(dt, o);
        if (kind < 0) return DWS_ERR_UNSUPPORTED;
        const size_t esize = 4u * (size_t)op_kind_words(kind);
        if (d_total == nullptr || (n > 0 && d_in == nullptr)) return DWS_ERR_INVALID_ARG;
        if (n > DWS_MAX_ELEMENTS) return DWS_ERR_UNSUPPORTED;
        const uintptr_t a = reinterpret_cast<uintptr_t>(d_in);
        const uintptr_t t = reinterpret_cast<uintptr_t>(d_total);
        if (a % esize != 0 || t % kElemBytes != 0) return DWS_ERR_MISALIGNED;
        if (a + (uintptr_t)n * esize < a || t + esize < t) return DWS_ERR_INVALID_ARG;
        if (n > 0 && t + esize > a && t < a + (uintptr_t)n * esize) return DWS_ERR_OVERLAP;
        return run_reduce_op(d_in, n, kind, d_total, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_scan_plan(const void* d_in, const void* d_out, size_t n, dws_dtype dtype, int exclusive,
                         const dws_options* opt, dws_launch_plan* plan)
{
    try {
        if (plan == nullptr) return DWS_ERR_INVALID_ARG;
        dws_options o{};
        if (opt != nullptr) o = *opt;
        dws_status s = check_options(o);
        if (s != DWS_OK) return s;
        if (o.variant != DWS_VARIANT_SINGLE_PASS && o.variant != DWS_VARIANT_CHAINED) return DWS_ERR_UNSUPPORTED;
        const int dt = enum_arg(dtype);
        s = validate(d_in, d_out, n, dt);
        if (s != DWS_OK) return s;
        dws_launch_plan out{};
        if (n > 0) {
            SinglePassPlan sp{};
            const int mode = o.variant == DWS_VARIANT_CHAINED ? kModeChained : kModeDecoupled;
            s = plan_single_pass(d_in, const_cast<void*>(d_out), n, dt, exclusive != 0, mode, o, nullptr, &sp);
            if (s != DWS_OK) return s;
            const KernelCfg& c = kCfgs[sp.cfg];
            const TileShape ts = cfg_shape(c);
            out.threads = (unsigned)ts.threads;
            out.tile_elems = (unsigned)ts.elems();
            out.num_tiles = sp.params.num_tiles;
            out.tile_index = c.tile_index == kTileDrawn ? DWS_TILE_DRAWN : DWS_TILE_DISPATCH;
            out.nontemporal = c.nt ? 1 : 0;
            out.pause_units = sp.params.backoff == kPause64 ? 64 : 1;
        }
        *plan = out;
        return DWS_OK;
    } catch (...) {
        return DWS_ERR_INVALID_ARG;
    }
}

const char* dws_status_string(dws_status status)
{
    switch (enum_arg(status)) {
    case DWS_OK: return "ok";
    case DWS_ERR_INVALID_ARG: return "invalid argument";
    case DWS_ERR_UNSUPPORTED: return "unsupported size or option combination";
    case DWS_ERR_OVERLAP: return "input and output overlap without being identical";
    case DWS_ERR_MISALIGNED: return "pointer not aligned to the 4-byte element size";
    case DWS_ERR_HIP: return "HIP runtime error";
    case DWS_ERR_OOM: return "out of device memory";
    }
    return "unknown status";
}

int dws_version(void) { return DWS_VERSION; }

int dws_num_tile_shapes(void) { return kNumShapes + 1; }

static int shape_for(int tile_shape, size_t n, int aligned)
{
    if (tile_shape < 0 || tile_shape > kNumShapes) return -1;
    return resolve_shape(tile_shape, n, aligned != 0);
}

unsigned dws_tile_elems(int tile_shape, size_t n, int aligned)
{
    const int s = shape_for(tile_shape, n, aligned);
    if (s < 0) return 0;
    return (unsigned)(aligned ? kShapes[s] : scalar_shape(kShapes[s])).elems();
}

unsigned dws_tile_threads(int tile_shape, size_t n, int aligned)
{
    const int s = shape_for(tile_shape, n, aligned);
    if (s < 0) return 0;
    return (unsigned)kShapes[s].threads;
}

dws_status dws_reserve(size_t n, hipStream_t stream)
{
    try {
        if (n > DWS_MAX_ELEMENTS) return DWS_ERR_UNSUPPORTED;
        Workspace* ws = nullptr;
        dws_status s = get_workspace(stream, &ws);
        if (s != DWS_OK) return s;
        // the most tiles any scan, compaction or generic-operator scan of n
        // elements uses (the smallest tile of each, 4,096 elements for all
        // but the pair types), kDescStride descriptor words each
        const uint64_t m = std::max<uint64_t>(n, 1);
        uint64_t tiles = 0;
        for (int i = 0; i < kNumShapes; ++i) tiles = std::max(tiles, ceil_div(m, (uint64_t)kShapes[i].elems()));
        for (int w = 1; w <= 2; ++w)
            for (int shape = kOpShapeSmall; shape <= kOpShapeUnaligned; ++shape)
                tiles = std::max(tiles, ceil_div(m, op_tile_elems(w, shape)));
        std::lock_guard<std::mutex> lock(ws->mu);
        s = ensure_desc(ws, tiles * kDescStride);
        if (s != DWS_OK) return s;
        const uint64_t stp = stp_scratch_elems(m);
        return stp == 0 ? DWS_OK : ensure_stp(ws, stp);
    } catch (...) {
        return DWS_ERR_OOM;
    }
}

dws_status dws_release_workspaces(void)
{
    try {
        std::lock_guard<std::mutex> lock(g_mu);
        int cur = 0;
        (void)hipGetDevice(&cur);
        dws_status result = DWS_OK;
        for (auto& kv : g_workspaces) {
            Workspace* ws = kv.second.get();
            if (hipSetDevice(ws->device) != hipSuccess) {
                result = DWS_ERR_HIP;
                continue;
            }
            if (hipDeviceSynchronize() != hipSuccess) result = DWS_ERR_HIP;
            if (ws->desc) (void)hipFree(ws->desc);
            if (ws->partials) (void)hipFree(ws->partials);
            if (ws->stp) (void)hipFree(ws->stp);
            if (ws->ctl) (void)hipFree(ws->ctl);
        }
        g_workspaces.clear();
        (void)hipSetDevice(cur);
        return result;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_device_memory_info(int* memory_clock_khz, int* memory_bus_width_bits, int* compute_units)
{
    if (memory_clock_khz == nullptr || memory_bus_width_bits == nullptr || compute_units == nullptr)
        return DWS_ERR_INVALID_ARG;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(memory_clock_khz, hipDeviceAttributeMemoryClockRate, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(memory_bus_width_bits, hipDeviceAttributeMemoryBusWidth, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, dev);
    return e == hipSuccess ? DWS_OK : from_hip(e);
}

dws_status dws_watchdog_trips(unsigned long long* trips)
{
    if (trips == nullptr) return DWS_ERR_INVALID_ARG;
    try {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return from_hip(e);
        e = hipDeviceSynchronize();
        if (e != hipSuccess) return from_hip(e);
        unsigned long long total = 0;
        std::lock_guard<std::mutex> lock(g_mu);
        for (auto& kv : g_workspaces) {
            if (kv.first.first != dev) continue;
            Workspace* ws = kv.second.get();
            unsigned int v = 0;
            e = hipMemcpy(&v, ws->watchdog(), sizeof(v), hipMemcpyDeviceToHost);
            if (e != hipSuccess) return from_hip(e);
            total += v;
            if (v != ws->trips_seen) {
                // a wait that timed out may have left a late workgroup's
                // descriptor under a later launch's epoch: start the look-back
                // state afresh (the count itself is kept). The workspace's
                // stream may be gone by now, so the clearing kernel runs on
                // the null stream of the (synchronised) device.
                std::lock_guard<std::mutex> wlock(ws->mu);
                e = launch_workspace_init(ws->desc, ws->desc_slots, ws->counter(), ws->epoch(), nullptr, nullptr);
                if (e == hipSuccess) e = hipDeviceSynchronize();
                if (e != hipSuccess) return from_hip(e);
                ws->launches = 0;
                ws->trips_seen = v;
            }
        }
        // the fixed array of dws_scan_noalloc, once set up on this device
        unsigned int v = 0;
        e = static_check_trips(dev, &v);
        if (e != hipSuccess) return from_hip(e);
        total += v;
        *trips = total;
        return DWS_OK;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_scan_debug(const void* d_in, void* d_out, size_t n, dws_dtype dtype, int exclusive, int variant,
                          unsigned tile_elems, unsigned delay_every, unsigned delay_phase, unsigned delay_ticks,
                          unsigned long long* h_desc, hipStream_t stream)
{
    try {
        if (variant != DWS_VARIANT_SINGLE_PASS && variant != DWS_VARIANT_CHAINED) return DWS_ERR_INVALID_ARG;
        if (tile_elems == 0 || tile_elems > kDebugMaxTile) return DWS_ERR_INVALID_ARG;
        if (delay_ticks > kMaxDebugDelayTicks) return DWS_ERR_INVALID_ARG;
        if (delay_every != 0 && delay_phase >= delay_every) return DWS_ERR_INVALID_ARG;
        dws_status s = validate(d_in, d_out, n, enum_arg(dtype));
        if (s != DWS_OK || n == 0) return s;
        const uint64_t num_tiles = ceil_div(n, tile_elems);
        if (num_tiles > 0x7fffffffull || num_tiles * 64ull > kMaxGridThreads) return DWS_ERR_UNSUPPORTED;
        Workspace* ws = nullptr;
        s = get_workspace(stream, &ws);
        if (s != DWS_OK) return s;
        std::lock_guard<std::mutex> lock(ws->mu);
        s = ensure_desc(ws, num_tiles * kDescStride);
        if (s != DWS_OK) return s;
        DebugArgs a{};
        s = before_lookback_launch(ws);
        if (s != DWS_OK) return s;
        a.epoch = ws->epoch();
        a.in = d_in;
        a.out = d_out;
        a.n = n;
        a.kind = kind_of(enum_arg(dtype));
        a.exclusive = exclusive != 0;
        a.mode = variant == DWS_VARIANT_CHAINED ? kModeChained : kModeDecoupled;
        a.tile_elems = tile_elems;
        a.delay_every = delay_every;
        a.delay_phase = delay_phase;
        a.delay_ticks = delay_ticks;
        a.desc = ws->desc;
        a.counter = ws->counter();
        a.watchdog = ws->watchdog();
        a.num_tiles = (uint32_t)num_tiles;
        s = from_hip(launch_debug(a, stream));
        if (s != DWS_OK) return s;
        if (h_desc != nullptr) {
            hipError_t e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return from_hip(e);
            if (num_tiles > 1) {
                // every kDescStride-th word of the array: the tiles' descriptors
                e = hipMemcpy2D(h_desc, sizeof(uint64_t), ws->desc, kDescStride * sizeof(uint64_t),
                                sizeof(uint64_t), num_tiles, hipMemcpyDeviceToHost);
                if (e != hipSuccess) return from_hip(e);
            } else {
                h_desc[0] = 0;   // a single tile publishes nothing
            }
        }
        return DWS_OK;
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_scan_profiled(const void* d_in, void* d_out, size_t n, dws_dtype dtype, int exclusive,
                             unsigned long long* d_stamps, size_t stamps_capacity, unsigned* num_tiles,
                             hipStream_t stream)
{
    try {
        if (!valid_dtype(enum_arg(dtype))) return DWS_ERR_INVALID_ARG;
        if (n == 0) {
            if (num_tiles != nullptr) *num_tiles = 0;
            return DWS_OK;
        }
        if (n > DWS_MAX_ELEMENTS) return DWS_ERR_UNSUPPORTED;
        const int shape = auto_shape(n);
        const uint64_t tiles = ceil_div(n, (uint64_t)kShapes[shape].elems());
        if (tiles > 0xffffffffull) return DWS_ERR_UNSUPPORTED;
        if (num_tiles != nullptr) *num_tiles = (unsigned)tiles;
        if (d_stamps == nullptr) return DWS_OK;   // size query
        if (stamps_capacity < tiles * kStampsPerTile) return DWS_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(d_stamps) & 7u) != 0) return DWS_ERR_MISALIGNED;
        dws_status s = validate(d_in, d_out, n, enum_arg(dtype));
        if (s != DWS_OK) return s;
        if (!aligned16(d_in, d_out)) return DWS_ERR_UNSUPPORTED;
        dws_options o{};
        return run_single_pass(d_in, d_out, n, enum_arg(dtype), exclusive != 0, kModeDecoupled, o, stream, d_stamps);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

}  // extern "C"

namespace {

// Compaction and partition by flags (one kernel, see dws_select.hip).
// A predicate of dws_select_if / dws_partition_if: the outcomes of comparing
// an element with the threshold (bit 0 less, 1 equal, 2 greater, 3 unordered)
// that select it, and the comparison's element kind.
struct SelectPredicate {
    uint32_t mask;
    uint32_t threshold;
    int kind;
};

// d_flags is ignored when `pred` is given (the selection comes from the values).
dws_status select_entry(const void* d_in, const void* d_flags, void* d_out, size_t n, int dtype,
                        unsigned long long* d_count, bool partition, hipStream_t stream,
                        const SelectPredicate* pred = nullptr)
{
    if (!valid_dtype(dtype)) return DWS_ERR_INVALID_ARG;
    if (d_count == nullptr) return DWS_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(d_count) & 7u) != 0) return DWS_ERR_MISALIGNED;
    if (n > kSelectMaxElems) return DWS_ERR_UNSUPPORTED;
    if (pred != nullptr) d_flags = d_in;
    if (n > 0) {
        dws_status s = validate(d_in, d_out, n, dtype);
        if (s != DWS_OK) return s;
        s = validate(d_flags, d_flags, n, DWS_INT32);
        if (s != DWS_OK) return s;
        const uintptr_t f = reinterpret_cast<uintptr_t>(d_flags), o = reinterpret_cast<uintptr_t>(d_out);
        const uintptr_t i = reinterpret_cast<uintptr_t>(d_in);
        const uintptr_t c = reinterpret_cast<uintptr_t>(d_count), bytes = (uintptr_t)n * kElemBytes;
        // the flags are read by later tiles while earlier ones write: no overlap with the output
        if (pred == nullptr && f < o + bytes && o < f + bytes) return DWS_ERR_OVERLAP;
        // a partition writes the back of the output before later tiles read their input
        if (partition && i < o + bytes && o < i + bytes) return DWS_ERR_OVERLAP;
        if ((c < o + bytes && o < c + 8) || (c < f + bytes && f < c + 8)) return DWS_ERR_OVERLAP;
        if (c < i + bytes && i < c + 8) return DWS_ERR_OVERLAP;
    }
    SelectArgs a{};
    a.in = d_in;
    a.flags = d_flags;
    a.out = d_out;
    a.n = n;
    a.count = d_count;
    a.partition = partition;
    if (pred != nullptr) {
        a.pred = true;
        a.pred_mask = pred->mask;
        a.threshold = pred->threshold;
        a.kind = pred->kind;
    }
    a.aligned = ((reinterpret_cast<uintptr_t>(d_in) | reinterpret_cast<uintptr_t>(d_out) |
                  reinterpret_cast<uintptr_t>(d_flags)) & 15u) == 0;
    const uint64_t tiles = n == 0 ? 0 : ceil_div(n, select_tile_elems(n, a.aligned));
    a.num_tiles = (uint32_t)tiles;
    if (tiles <= 1) return from_hip(launch_select(a, stream));
    Workspace* ws = nullptr;
    dws_status s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    s = ensure_desc(ws, tiles * kDescStride);
    if (s != DWS_OK) return s;
    s = before_lookback_launch(ws);
    if (s != DWS_OK) return s;
    a.epoch = ws->epoch();
    a.desc = ws->desc;
    a.counter = ws->counter();
    a.watchdog = ws->watchdog();
    return from_hip(launch_select(a, stream));
}

bool overlaps(const void* a, size_t a_bytes, const void* b, size_t b_bytes)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + b_bytes && y < x + a_bytes;
}

// Reduce-by-key and run-length encoding (mode 0 integer values, 1 fp32
// values, 2 run lengths without values).
dws_status rbk_entry(const void* keys, const void* vals, void* ukeys, void* aggs, size_t n, int mode,
                     unsigned long long* num_runs, hipStream_t stream)
{
    if (num_runs == nullptr) return DWS_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(num_runs) & 7u) != 0) return DWS_ERR_MISALIGNED;
    if (n > kSelectMaxElems) return DWS_ERR_UNSUPPORTED;
    if (n > 0) {
        const void* in_arrays[2] = {keys, vals};
        void* out_arrays[2] = {ukeys, aggs};
        const int n_in = mode == 2 ? 1 : 2;
        for (int k = 0; k < n_in; ++k) {
            const dws_status s = validate_sized(in_arrays[k], in_arrays[k], n, kElemBytes);
            if (s != DWS_OK) return s;
        }
        for (int k = 0; k < 2; ++k) {
            const dws_status s = validate_sized(out_arrays[k], out_arrays[k], n, kElemBytes);
            if (s != DWS_OK) return s;
        }
        const size_t bytes = n * kElemBytes;
        // outputs are written while later tiles still read keys around them
        for (int k = 0; k < n_in; ++k)
            for (int m = 0; m < 2; ++m)
                if (overlaps(in_arrays[k], bytes, out_arrays[m], bytes)) return DWS_ERR_OVERLAP;
        if (overlaps(ukeys, bytes, aggs, bytes)) return DWS_ERR_OVERLAP;
        for (int m = 0; m < 2; ++m)
            if (overlaps(num_runs, 8, out_arrays[m], bytes)) return DWS_ERR_OVERLAP;
        for (int k = 0; k < n_in; ++k)
            if (overlaps(num_runs, 8, in_arrays[k], bytes)) return DWS_ERR_OVERLAP;
    }
    RbkArgs a{};
    a.keys = keys;
    a.vals = vals;
    a.ukeys = ukeys;
    a.aggs = aggs;
    a.n = n;
    a.mode = mode;
    a.num_runs = num_runs;
    a.aligned = ((reinterpret_cast<uintptr_t>(keys) | (mode == 2 ? 0u : reinterpret_cast<uintptr_t>(vals))) & 15u) == 0;
    const uint64_t tiles = n == 0 ? 0 : ceil_div(n, rbk_tile_elems(n, a.aligned, mode));
    a.num_tiles = (uint32_t)tiles;
    if (tiles <= 1) return from_hip(launch_rbk(a, stream));
    Workspace* ws = nullptr;
    dws_status s = get_workspace(stream, &ws);
    if (s != DWS_OK) return s;
    std::lock_guard<std::mutex> lock(ws->mu);
    s = ensure_desc(ws, tiles * kDescStride);
    if (s != DWS_OK) return s;
    s = before_lookback_launch(ws);
    if (s != DWS_OK) return s;
    a.epoch = ws->epoch();
    a.desc = ws->desc;
    a.watchdog = ws->watchdog();
    return from_hip(launch_rbk(a, stream));
}

}  // namespace

extern "C" {

dws_status dws_reduce_by_key(const void* d_keys, const void* d_values, void* d_unique_keys, void* d_aggregates,
                             size_t n, dws_dtype value_dtype, unsigned long long* d_num_runs, hipStream_t stream)
{
    try {
        const int vt = enum_arg(value_dtype);
        if (!valid_dtype(vt)) return DWS_ERR_INVALID_ARG;
        return rbk_entry(d_keys, d_values, d_unique_keys, d_aggregates, n, vt == DWS_FLOAT32 ? 1 : 0,
                         d_num_runs, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_run_length_encode(const void* d_keys, void* d_unique_keys, void* d_lengths, size_t n,
                                 unsigned long long* d_num_runs, hipStream_t stream)
{
    try {
        return rbk_entry(d_keys, nullptr, d_unique_keys, d_lengths, n, 2, d_num_runs, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_select_flagged(const void* d_in, const void* d_flags, void* d_out, size_t n, dws_dtype dtype,
                              unsigned long long* d_count, hipStream_t stream)
{
    try {
        return select_entry(d_in, d_flags, d_out, n, enum_arg(dtype), d_count, false, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_partition_flagged(const void* d_in, const void* d_flags, void* d_out, size_t n, dws_dtype dtype,
                                 unsigned long long* d_num_selected, hipStream_t stream)
{
    try {
        return select_entry(d_in, d_flags, d_out, n, enum_arg(dtype), d_num_selected, true, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

}  // extern "C"

namespace {

dws_status select_if_entry(const void* d_in, void* d_out, size_t n, dws_dtype dtype, dws_pred pred,
                           const void* h_threshold, unsigned long long* d_count, bool partition, hipStream_t stream)
{
    const int dt = enum_arg(dtype), pr = enum_arg(pred);
    if (!valid_dtype(dt) || h_threshold == nullptr) return DWS_ERR_INVALID_ARG;
    // outcome bits: 0 less, 1 equal, 2 greater, 3 unordered (a NaN: only
    // "not equal" holds)
    static const uint32_t kMasks[] = {0x2u, 0xDu, 0x1u, 0x3u, 0x4u, 0x6u};
    if (pr < DWS_PRED_EQ || pr > DWS_PRED_GE) return DWS_ERR_INVALID_ARG;
    SelectPredicate p{};
    p.mask = kMasks[pr];
    std::memcpy(&p.threshold, h_threshold, sizeof p.threshold);
    p.kind = dt == DWS_FLOAT32 ? kKindF32 : (dt == DWS_INT32 ? kPredKindI32 : kKindU32);
    return select_entry(d_in, nullptr, d_out, n, dt, d_count, partition, stream, &p);
}

}  // namespace

extern "C" {

dws_status dws_select_if(const void* d_in, void* d_out, size_t n, dws_dtype dtype, dws_pred pred,
                         const void* h_threshold, unsigned long long* d_count, hipStream_t stream)
{
    try {
        return select_if_entry(d_in, d_out, n, dtype, pred, h_threshold, d_count, false, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_partition_if(const void* d_in, void* d_out, size_t n, dws_dtype dtype, dws_pred pred,
                            const void* h_threshold, unsigned long long* d_num_selected, hipStream_t stream)
{
    try {
        return select_if_entry(d_in, d_out, n, dtype, pred, h_threshold, d_num_selected, true, stream);
    } catch (const std::bad_alloc&) {
        return DWS_ERR_OOM;
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

dws_status dws_selftest_wave(const void* d_in, void* d_incl, void* d_shift, size_t n_waves, dws_dtype dtype,
                             hipStream_t stream)
{
    if (!valid_dtype(enum_arg(dtype))) return DWS_ERR_INVALID_ARG;
    if (n_waves == 0) return DWS_OK;
    if (d_in == nullptr || d_incl == nullptr || d_shift == nullptr) return DWS_ERR_INVALID_ARG;
    if (n_waves > 0xffffffffull / 64ull) return DWS_ERR_UNSUPPORTED;
    return from_hip(launch_wave_selftest(d_in, d_incl, d_shift, n_waves, kind_of(enum_arg(dtype)), stream));
}

}  // extern "C"

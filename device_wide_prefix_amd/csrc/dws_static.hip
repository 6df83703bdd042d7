// The scan entry point that allocates nothing (dws_scan_noalloc), for callers
// that cannot allocate device memory: code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc.
//
// It runs exactly the kernels of scan_inclusive / scan_exclusive. What a
// workspace holds for them (control block: tile counter, watchdog, epoch word;
// one descriptor per tile) lives instead in `scratch`, a file-scope device
// array of fixed size. The host code never passes the array's name to a
// kernel: in host code that name is only a stand-in for the symbol. At its
// first multi-tile call on a device, with that device current, the entry point
// asks the runtime for the array's address on that device
// (hipGetSymbolAddress), keeps it per device, and clears the array with a
// kernel on the caller's stream. Every later use goes through that address.
//
// Every call on a device shares its array, which keeps the last call's
// contents. That is how the descriptor epochs work (a descriptor written by an
// earlier launch reads as empty to a later one), so nothing needs clearing
// between calls. The host counts the launches per device and clears the array
// again before the 30-bit epoch could wrap.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "dws_internal.h"
#include "dws_scan.h"

namespace {

using namespace dws;

constexpr uint64_t kCtlWords = kCtlBytes / sizeof(uint64_t);
constexpr uint64_t kDescWords = (uint64_t)DWS_NOALLOC_MAX_TILES * kDescStride;
constexpr uint64_t kScratchWords = kCtlWords + kDescWords;

// Control block (kCtlBytes), then the descriptors of DWS_NOALLOC_MAX_TILES
// tiles, kDescStride words each.
static __device__ __align__(256) uint64_t scratch[kScratchWords];

struct DeviceScratch {
    char* base = nullptr;        // device address of `scratch` on this device
    uint32_t launches = 0;       // look-back launches since the array was cleared
    unsigned int trips_seen = 0; // watchdog count when the state was last cleared after trips
};

std::mutex g_mu;
std::map<int, DeviceScratch> g_dev;

LookbackState state_of(const DeviceScratch& d)
{
    LookbackState s{};
    s.desc = reinterpret_cast<uint64_t*>(d.base + kCtlBytes);
    s.desc_slots = kDescWords;
    s.counter = reinterpret_cast<unsigned long long*>(d.base + kCtlCounterOffset);
    s.watchdog = reinterpret_cast<unsigned int*>(d.base + kCtlWatchdogOffset);
    s.epoch = reinterpret_cast<unsigned int*>(d.base + kCtlEpochOffset);
    return s;
}

bool capturing(hipStream_t stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// The array of the current device, set up on first use: its address, and one
// clearing kernel on `stream` (all descriptors X, counter 0, epoch 1, watchdog
// 0). Call with g_mu held.
dws_status scratch_of_current_device(hipStream_t stream, DeviceScratch** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return status_from_hip(e);
    auto it = g_dev.find(dev);
    if (it != g_dev.end()) {
        *out = &it->second;
        return DWS_OK;
    }
    // the clearing kernel must run before any replay could use the array, so
    // the set-up is not done inside a capture
    if (capturing(stream)) return DWS_ERR_UNSUPPORTED;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return status_from_hip(e);
    if (ptr == nullptr) return DWS_ERR_HIP;
    DeviceScratch d;
    d.base = static_cast<char*>(ptr);
    const LookbackState s = state_of(d);
    e = launch_workspace_init(s.desc, s.desc_slots, s.counter, s.epoch, s.watchdog, stream);
    if (e != hipSuccess) return status_from_hip(e);
    auto ins = g_dev.emplace(dev, d);
    *out = &ins.first->second;
    return DWS_OK;
}

}  // namespace

namespace dws {

hipError_t static_check_trips(int device, unsigned int* trips)
{
    *trips = 0;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_dev.find(device);
    if (it == g_dev.end()) return hipSuccess;
    DeviceScratch& d = it->second;
    const LookbackState st = state_of(d);
    hipError_t e = hipMemcpy(trips, st.watchdog, sizeof(*trips), hipMemcpyDeviceToHost);
    if (e != hipSuccess || *trips == d.trips_seen) return e;
    // a wait that timed out may have left a late workgroup's descriptor under
    // a later launch's epoch: start the look-back state afresh
    e = launch_workspace_init(st.desc, st.desc_slots, st.counter, st.epoch, nullptr, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    d.launches = 0;
    d.trips_seen = *trips;
    return hipSuccess;
}

}  // namespace dws

extern "C" dws_status dws_scan_noalloc(const void* d_in, void* d_out, size_t n, dws_dtype dtype, int exclusive,
                                       hipStream_t stream)
{
    try {
        int dt = 0;
        static_assert(sizeof(dt) == sizeof(dtype), "C enums travel as int");
        __builtin_memcpy(&dt, &dtype, sizeof dt);
        dws_status s = validate_scan_args(d_in, d_out, n, dt);
        if (s != DWS_OK || n == 0) return s;
        SinglePassPlan plan{};
        const dws_options defaults{};
        s = plan_single_pass(d_in, d_out, n, dt, exclusive != 0, kModeDecoupled, defaults, nullptr, &plan);
        if (s != DWS_OK) return s;
        // one tile: no predecessors, and the kernel touches no look-back state
        if (plan.params.num_tiles == 1) return status_from_hip(launch_single_pass_plan(plan, nullptr, stream));
        if (plan.params.num_tiles > DWS_NOALLOC_MAX_TILES) return DWS_ERR_UNSUPPORTED;
        std::lock_guard<std::mutex> lock(g_mu);
        DeviceScratch* d = nullptr;
        s = scratch_of_current_device(stream, &d);
        if (s != DWS_OK) return s;
        const LookbackState st = state_of(*d);
        if (d->launches + 1u >= kEpochMax) {
            const hipError_t e = launch_workspace_init(st.desc, st.desc_slots, st.counter, st.epoch, nullptr, stream);
            if (e != hipSuccess) return status_from_hip(e);
            d->launches = 0;
        }
        ++d->launches;
        return status_from_hip(launch_single_pass_plan(plan, &st, stream));
    } catch (...) {
        return DWS_ERR_HIP;
    }
}

// Host-side interface between the C ABI (dws_abi.cpp) and the kernel
// launchers (dws_kernels_*.hip). Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dws_protocol.h"

namespace dws {

// Workspace control block layout (one 256-byte allocation per workspace):
// the tile counter and the watchdog counter sit on separate cache lines.
constexpr size_t kCtlBytes = 256;
constexpr size_t kCtlCounterOffset = 0;
constexpr size_t kCtlWatchdogOffset = 128;

struct SinglePassArgs {
    const void* in;
    void* out;
    uint64_t n;
    int kind;              // kKindU32 / kKindF32
    bool exclusive;
    bool aligned;          // both pointers 16-byte aligned
    int shape;             // index into kAlignedShapes
    int order;             // kOrderRelaxed / kOrderAcqRel
    int mode;              // kModeDecoupled / kModeChained
    bool nontemporal;
    uint64_t* desc;        // >= num_tiles slots (unused when num_tiles == 1)
    unsigned long long* counter;
    unsigned int* watchdog;
    uint32_t num_tiles;
};

// Whether a single-pass kernel with these compile-time parameters is built.
bool single_pass_available(int shape, bool aligned, int order, int mode, bool nontemporal);
// Elements per tile and threads per workgroup of the kernel the launcher uses.
uint32_t single_pass_tile_elems(int shape, bool aligned);
uint32_t single_pass_threads(int shape, bool aligned);
hipError_t launch_single_pass(const SinglePassArgs& a, hipStream_t stream);

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
uint32_t rts_tile_elems(bool aligned);
hipError_t launch_rts(const RtsArgs& a, hipStream_t stream);

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
};
hipError_t launch_debug(const DebugArgs& a, hipStream_t stream);

// Zero `slots` descriptors and set the counter to kCounterInit and the
// watchdog to 0 (a kernel, not a memset, so that it may sit in a graph).
hipError_t launch_workspace_init(uint64_t* desc, uint64_t slots, unsigned long long* counter,
                                 unsigned int* watchdog, hipStream_t stream);

hipError_t launch_wave_selftest(const void* in, void* incl, void* shift, uint64_t n_waves,
                                int kind, hipStream_t stream);

}  // namespace dws

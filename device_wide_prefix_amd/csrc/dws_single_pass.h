// Kernel arguments and launcher of the single-pass + scan (the only host
// interface the single-pass kernel sources include).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dws_protocol.h"

namespace dws {

struct SinglePassParams {
    const void* in;
    void* out;
    uint64_t n;
    uint64_t* desc;        // >= num_tiles slots (unused when num_tiles == 1)
    unsigned long long* counter;
    unsigned int* watchdog;
    unsigned long long* stamps;   // kStampsPerTile per tile (instrumented kernels only)
    uint32_t num_tiles;
    unsigned int* epoch;          // the workspace's epoch word (unused when num_tiles == 1)
    uint32_t backoff;             // pause level between blocked look-back polls (kPause*)
    const void* seed;             // one element: tile 0's prefix (null: the identity)
};

// Launch built configuration `cfg` (index into kCfgs) for element type T
// (uint32_t or float; instantiated in dws_sp_u32.hip / dws_sp_f32.hip).
template <class T>
hipError_t launch_single_pass_typed(int cfg, bool exclusive, const SinglePassParams& p, hipStream_t stream);

}  // namespace dws

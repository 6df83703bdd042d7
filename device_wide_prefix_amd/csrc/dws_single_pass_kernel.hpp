// Single-pass device-wide + scan with decoupled look-back for gfx950
// (Merrill & Garland, "Single-pass Parallel Prefix Scan with Decoupled
// Look-back", section 4.1 steps and section 4.4 adaptations), and the chained
// scan that waits on the immediate predecessor only (section 3.2, Fig 4).
//
// One workgroup per tile; the kernel is the whole call (no init launch: every
// launch reads a new descriptor epoch from the workspace, and the owner of the
// last tile advances it):
//   1. the tile is the workgroup index (TILE_INDEX == kTileDispatch, the
//      automatic choice), or lane 0 draws it from the workspace counter
//      (dynamic tile index, PMPP 11.3 notes; kTileDrawn);
//   2. every wave loads its segment of the tile with coalesced vector loads,
//      CHUNKS x VEC elements per lane kept in registers (thread coarsening,
//      PMPP 11.2 notes); with NT the loads are non-temporal (the input is read
//      once), the stores never are;
//   3. lane-serial totals -> wave64 DPP scans -> the wave totals go through
//      LDS, giving each wave its prefix inside the tile and the tile aggregate;
//   4. wave 0 publishes {A, aggregate} (tile 0: {P, seed + aggregate}, the
//      seed being the caller's one-element prefix of the whole array, or 0),
//      looks back over 64 predecessor descriptors per step until the nearest
//      P, and publishes {P, prefix + aggregate};
//   5. every element gets prefix + wave prefix + chunk/lane prefix + its
//      serial in-lane prefix, and the tile is stored. The whole tile is in
//      registers before the first store, so d_out == d_in is safe.
#pragma once

#include <utility>

#include "dws_device.hpp"
#include "dws_single_pass.h"

namespace dws {

template <class T, bool EXCL, int BLOCK, int VEC, int CHUNKS, int ORDER, int MODE, bool NT, int TILE_INDEX,
          bool INSTR>
__global__ void __launch_bounds__(BLOCK) k_single_pass(SinglePassParams p)
{
    uint64_t stamp[kStampsPerTile] = {};
    if constexpr (INSTR) stamp[0] = realtime();
    constexpr int W = BLOCK / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    __shared__ uint32_t s_draw, s_epoch;
    __shared__ T s_wave[W];
    __shared__ T s_prefix;

    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const bool multi = p.num_tiles > 1u;
    // the launch's descriptor epoch: read with the draw (drawn index), or in
    // wave 0 after the tile loads (workgroup index); it is only needed to
    // publish, and any time before that is early enough
    uint32_t epoch_v = 0u;

    uint32_t tile = 0u;
    if (multi) {
        if constexpr (TILE_INDEX == kTileDispatch) {
            tile = blockIdx.x;
        } else {
            if (threadIdx.x == 0) {
                // both reads in flight together: one round trip, not two
                const uint32_t e = load_epoch_async(p.epoch);
                s_draw = draw_tile(p.counter, p.num_tiles);
                s_epoch = e;
            }
            __syncthreads();
            tile = uniform(s_draw);
            epoch_v = s_epoch;
            // a counter that was not put back to 0 would hand out indices past
            // the grid; never touch memory with them (counts as a watchdog trip)
            if (tile >= p.num_tiles) {
                if (threadIdx.x == 0) atomicAdd(p.watchdog, 1u);
                return;
            }
        }
    }
    if constexpr (INSTR) stamp[1] = realtime();

    const uint64_t seg_first = (uint64_t)tile * TILE + (uint64_t)wave * SEG;
    const uint32_t seg_valid = valid_bytes(seg_first, SEG, p.n);

    T x[CHUNKS][VEC];
    load_segment<T, VEC, CHUNKS, NT>(make_rsrc(static_cast<const T*>(p.in) + seg_first, seg_valid), lane, x);
    if constexpr (TILE_INDEX == kTileDispatch)
        if (multi && wave == 0) epoch_v = load_epoch_async(p.epoch);
    // a seeded scan: tile 0's prefix is the caller's element, read while the
    // tile's loads are in flight
    uint32_t seed_bits = 0u;
    if (p.seed != nullptr && tile == 0u && wave == 0) seed_bits = *static_cast<const uint32_t*>(p.seed);

    const T seg_total = scan_segment_local<T, EXCL, VEC, CHUNKS>(x);
    pin_in_registers<T, VEC, CHUNKS>(x);

    if (lane == 0) s_wave[wave] = seg_total;
    __syncthreads();
    if constexpr (INSTR) stamp[2] = realtime();
    T wave_pre = T(0), agg = T(0);
#pragma unroll
    for (int w = 0; w < W; ++w) {
        if (w == wave) wave_pre = agg;
        agg = agg + s_wave[w];
    }

    if (wave == 0) {
        T prefix = Elem<T>::from(uniform(seed_bits));
        if (multi) {
            const uint32_t epoch = uniform(epoch_v);
            if (tile == 0u) {
                if (lane == 0)
                    desc_store<ORDER>(desc_at(p.desc, 0u), desc_pack(epoch, kStatusP, Elem<T>::bits(prefix + agg)));
            } else {
                if constexpr (MODE == kModeDecoupled) {
                    if (lane == 0)
                        desc_store<ORDER>(desc_at(p.desc, tile), desc_pack(epoch, kStatusA, Elem<T>::bits(agg)));
                    prefix = lookback_decoupled<T, ORDER, kLookbackSlots, TILE_INDEX == kTileDrawn>(
                        p.desc, tile, epoch, p.watchdog, p.backoff);
                } else {
                    prefix = lookback_chained<T, ORDER>(p.desc, tile, epoch, p.watchdog);
                }
                if (lane == 0) {
                    desc_store<ORDER>(desc_at(p.desc, tile),
                                      desc_pack(epoch, kStatusP, Elem<T>::bits(prefix + agg)));
                    if (tile == p.num_tiles - 1u) advance_epoch(p.epoch, epoch);
                }
            }
        }
        if (lane == 0) s_prefix = prefix;
    }
    __syncthreads();
    if constexpr (INSTR) stamp[3] = realtime();
    const T seed = s_prefix + wave_pre;

    add_seed<T, VEC, CHUNKS>(x, seed);
    store_segment<T, VEC, CHUNKS, false>(make_rsrc(static_cast<T*>(p.out) + seg_first, seg_valid), lane, x);
    if constexpr (INSTR) {
        stamp[4] = realtime();
        if (threadIdx.x == 0) {
#pragma unroll
            for (uint32_t i = 0; i < kStampsPerTile; ++i) p.stamps[(uint64_t)tile * kStampsPerTile + i] = stamp[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Launch of built configuration `cfg` (index into kCfgs) for element type T.
// Each element type is instantiated in its own translation unit.
// ---------------------------------------------------------------------------
template <class T, bool EXCL, int I>
static hipError_t launch_cfg(const SinglePassParams& p, hipStream_t stream)
{
    constexpr KernelCfg c = kCfgs[I];
    constexpr TileShape s = cfg_shape(c);
    const void* fn = reinterpret_cast<const void*>(
        &k_single_pass<T, EXCL, s.threads, s.vec, s.chunks, c.order, c.mode, c.nt, c.tile_index, c.instr>);
    SinglePassParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(fn, dim3(p.num_tiles), dim3(s.threads), args, 0, stream);
}

template <class T, int... I>
static hipError_t dispatch_cfg(int cfg, bool exclusive, const SinglePassParams& p, hipStream_t stream,
                               std::integer_sequence<int, I...>)
{
    hipError_t r = hipErrorInvalidValue;
    (void)((cfg == I ? (r = exclusive ? launch_cfg<T, true, I>(p, stream) : launch_cfg<T, false, I>(p, stream),
                        true)
                     : false) ||
           ...);
    return r;
}

template <class T>
hipError_t launch_single_pass_typed(int cfg, bool exclusive, const SinglePassParams& p, hipStream_t stream)
{
    return dispatch_cfg<T>(cfg, exclusive, p, stream, std::make_integer_sequence<int, kNumCfgs>{});
}

}  // namespace dws

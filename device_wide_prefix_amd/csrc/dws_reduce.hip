// Device-wide + reduction of one array to one element for gfx950: the first
// step of a scan split over several devices, where each device sums its
// contiguous shard, the shard totals are exchanged and scanned, and each
// device then scans its shard seeded with the total of the shards before it
// (the reduce-then-scan decomposition of Merrill & Garland, "Single-pass
// Parallel Prefix Scan with Decoupled Look-back", section 3.2 and Fig 3, taken
// one level up: a device plays the part of a workgroup).
//
// One launch. G workgroups each sum a contiguous run of tiles and publish
// their partial as a descriptor word of the scans' protocol (epoch | status P
// | value, one relaxed 64-bit agent-scope store, so a word left by an earlier
// launch reads as not yet published). The workgroup with the highest index
// then reads the G words, waiting for any not yet published, adds them in
// index order, writes the total and advances the epoch. It is the only
// workgroup that waits, and only on workgroups that never wait, so the wait
// ends whatever order the workgroups run in (the watchdog bounds it all the
// same). Electing the last to finish with a counter instead measured 1.75 to
// 3.5 times slower at 2^25 elements: the 1,024 to 2,048 device-scope atomics
// on one word, issued in one burst as the workgroups finish together,
// serialise at about 11 to 32 ns each. Every addition's operands and order
// depend on n and on whether the input is 16-byte aligned only, so repeated
// calls return the same bits for fp32.
#include "dws_device.hpp"
#include "dws_internal.h"

namespace dws {

struct ReduceParams {
    const void* in;
    uint64_t n;
    uint32_t num_tiles;
    uint32_t tiles_per_group;
    uint32_t groups;
    uint64_t* desc;           // >= groups descriptor slots
    unsigned int* epoch;      // the workspace's epoch word
    unsigned int* watchdog;
    void* total;              // one element
};

template <class T, int BLOCK, int VEC, int CHUNKS, bool NT>
__global__ void __launch_bounds__(BLOCK) k_reduce(ReduceParams p)
{
    constexpr int W = BLOCK / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    constexpr int PER = (int)(kReduceMaxGroups / BLOCK);   // partials per thread of the last group
    static_assert(PER * BLOCK == (int)kReduceMaxGroups, "the last group reads every partial in one round");
    __shared__ T s_wave[W];
    __shared__ uint32_t s_epoch;
    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const uint32_t g = blockIdx.x;
    const uint64_t t0 = (uint64_t)g * p.tiles_per_group;
    const uint64_t t_end = t0 + p.tiles_per_group;
    const uint64_t t1 = t_end < (uint64_t)p.num_tiles ? t_end : (uint64_t)p.num_tiles;
    // the launch's epoch, in flight with the first tile's loads; it only
    // advances once every group has published, so no group reads it late
    uint32_t epoch_v = 0u;
    if (wave == 0) epoch_v = load_epoch_async(p.epoch);

    // each lane sums its elements of one tile, then adds that to its running
    // total: chains of CHUNKS * VEC and of tiles_per_group additions
    T acc = T(0);
    for (uint64_t t = t0; t < t1; ++t) {
        const uint64_t seg_first = t * TILE + (uint64_t)wave * SEG;
        T x[CHUNKS][VEC];
        load_segment<T, VEC, CHUNKS, NT>(
            make_rsrc(static_cast<const T*>(p.in) + seg_first, valid_bytes(seg_first, SEG, p.n)), lane, x);
        T s = T(0);
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e) s = s + x[c][e];
        acc = acc + s;
    }
    const T w = wave_sum(acc);
    if (lane == 0) s_wave[wave] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        T s = T(0);
#pragma unroll
        for (int i = 0; i < W; ++i) s = s + s_wave[i];
        const uint32_t epoch = uniform(epoch_v);
        desc_store<kOrderRelaxed>(desc_at(p.desc, g), desc_pack(epoch, kStatusP, Elem<T>::bits(s)));
        s_epoch = epoch;
    }
    if (g != p.groups - 1u) return;
    __syncthreads();

    // the last group: thread i adds partials i, i + BLOCK, i + 2 BLOCK, ... in
    // that order, then the same wave and workgroup sums as above
    const uint32_t epoch = uniform(s_epoch);
    uint64_t d[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const uint32_t i = threadIdx.x + (uint32_t)(k * BLOCK);
        d[k] = i < p.groups ? desc_load<kOrderRelaxed>(desc_at(p.desc, i)) : desc_pack(epoch, kStatusP, 0u);
    }
    const uint64_t start = realtime();
    for (;;) {
        bool waiting = false;
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (desc_status(d[k], epoch) == kStatusX) waiting = true;
        if (!waiting) break;
        if (realtime() - start > kWatchdogTicks) {
            atomicAdd(p.watchdog, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (desc_status(d[k], epoch) == kStatusX)
                d[k] = desc_load<kOrderRelaxed>(desc_at(p.desc, threadIdx.x + (uint32_t)(k * BLOCK)));
    }
    T v = T(0);
#pragma unroll
    for (int k = 0; k < PER; ++k)
        if (threadIdx.x + (uint32_t)(k * BLOCK) < p.groups) v = v + Elem<T>::from((uint32_t)d[k]);
    const T wv = wave_sum(v);
    if (lane == 0) s_wave[wave] = wv;   // thread 0 read it before the last barrier
    __syncthreads();
    if (threadIdx.x == 0) {
        T s = T(0);
#pragma unroll
        for (int i = 0; i < W; ++i) s = s + s_wave[i];
        *static_cast<T*>(p.total) = s;
        advance_epoch(p.epoch, epoch);
    }
}

template <class T, int BLOCK, int VEC, int CHUNKS, bool NT>
static hipError_t launch_reduce_cfg(const ReduceParams& p, hipStream_t stream)
{
    ReduceParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_reduce<T, BLOCK, VEC, CHUNKS, NT>), dim3(p.groups),
                           dim3(BLOCK), args, 0, stream);
}

template <class T>
static hipError_t launch_reduce_typed(const ReduceArgs& a, const ReduceParams& p, hipStream_t stream)
{
    if (!a.aligned) return launch_reduce_cfg<T, kReduceThreads, 1, kReduceTileElems / kReduceThreads, false>(p, stream);
    if (a.nontemporal)
        return launch_reduce_cfg<T, kReduceThreads, 4, kReduceTileElems / (4 * kReduceThreads), true>(p, stream);
    return launch_reduce_cfg<T, kReduceThreads, 4, kReduceTileElems / (4 * kReduceThreads), false>(p, stream);
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream)
{
    if (a.groups == 0u || a.groups > kReduceMaxGroups) return hipErrorInvalidValue;
    if ((uint64_t)a.groups * a.tiles_per_group < a.num_tiles) return hipErrorInvalidValue;
    ReduceParams p{};
    p.in = a.in;
    p.n = a.n;
    p.num_tiles = a.num_tiles;
    p.tiles_per_group = a.tiles_per_group;
    p.groups = a.groups;
    p.desc = a.desc;
    p.epoch = a.epoch;
    p.watchdog = a.watchdog;
    p.total = a.total;
    return a.kind == kKindF32 ? launch_reduce_typed<float>(a, p, stream)
                              : launch_reduce_typed<uint32_t>(a, p, stream);
}

}  // namespace dws

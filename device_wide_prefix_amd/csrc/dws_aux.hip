// Companion kernels of the scan library for gfx950:
//   - the three-kernel reduce-then-scan comparison variant (Merrill & Garland,
//     section 3.2 and Fig 3; CUDA-Operators-6-Cumsum, section 1.2: G
//     co-resident workgroups, each owning one contiguous chunk);
//   - the protocol-inspection kernel (one wavefront per tile of 1..64
//     elements, optional delays before publishing);
//   - the workspace initialiser and the wavefront-primitive self test.
#include "dws_device.hpp"
#include "dws_internal.h"

namespace dws {

// ---------------------------------------------------------------------------
// Reduce-then-scan: ~3n traffic (n read by the reduce, n read + n written by
// the downsweep). Same tile geometry as the default single-pass shape.
// ---------------------------------------------------------------------------
constexpr int kRtsThreads = 256;

template <class T, int BLOCK, int VEC, int CHUNKS>
__global__ void __launch_bounds__(BLOCK)
    k_rts_reduce(const T* in, uint64_t n, uint32_t num_tiles, uint32_t tiles_per_group, T* partials)
{
    constexpr int W = BLOCK / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    __shared__ T s_wave[W];
    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const uint32_t g = blockIdx.x;
    const uint32_t t0 = g * tiles_per_group;
    const uint32_t t1 = min(t0 + tiles_per_group, num_tiles);

    T acc = T(0);
    for (uint32_t t = t0; t < t1; ++t) {
        const uint64_t seg_first = (uint64_t)t * TILE + (uint64_t)wave * SEG;
        T x[CHUNKS][VEC];
        load_segment<T, VEC, CHUNKS, false>(make_rsrc(in + seg_first, valid_bytes(seg_first, SEG, n)), lane, x);
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc = acc + x[c][e];
    }
    const T w = wave_sum(acc);
    if (lane == 0) s_wave[wave] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        T s = T(0);
#pragma unroll
        for (int i = 0; i < W; ++i) s = s + s_wave[i];
        partials[g] = s;
    }
}

// Exclusive scan of the G <= kRtsMaxGroups partials, in place, by one
// workgroup of 256 threads holding 16 consecutive partials each.
template <class T>
__global__ void __launch_bounds__(256) k_rts_scan_partials(T* partials, uint32_t groups)
{
    constexpr int K = (int)(kRtsMaxGroups / 256u);
    __shared__ T s_wave[4];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const uint32_t base = threadIdx.x * (uint32_t)K;
    T v[K];
    T total = T(0);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        v[k] = (base + k < groups) ? partials[base + k] : T(0);
        total = total + v[k];
    }
    const T incl = wave_inclusive_scan(total);
    const T lane_excl = wave_shift_up1(incl);
    if (lane == 0) s_wave[wave] = wave_read_lane(incl, 63);
    __syncthreads();
    T wave_pre = T(0);
    for (int w = 0; w < wave; ++w) wave_pre = wave_pre + s_wave[w];
    T s = wave_pre + lane_excl;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (base + k < groups) partials[base + k] = s;
        s = s + v[k];
    }
}

template <class T, bool EXCL, int BLOCK, int VEC, int CHUNKS>
__global__ void __launch_bounds__(BLOCK)
    k_rts_downsweep(const T* in, T* out, uint64_t n, uint32_t num_tiles, uint32_t tiles_per_group,
                    const T* prefixes)
{
    constexpr int W = BLOCK / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    // double-buffered: tile i+2 may only overwrite a buffer once every wave has
    // passed the barrier of tile i+1, i.e. finished reading tile i's totals
    __shared__ T s_wave[2][W];
    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const uint32_t g = blockIdx.x;
    const uint32_t t0 = g * tiles_per_group;
    const uint32_t t1 = min(t0 + tiles_per_group, num_tiles);

    T seed = prefixes[g];
    uint32_t it = 0;
    for (uint32_t t = t0; t < t1; ++t, ++it) {
        const uint64_t seg_first = (uint64_t)t * TILE + (uint64_t)wave * SEG;
        const uint32_t valid = valid_bytes(seg_first, SEG, n);
        T x[CHUNKS][VEC];
        load_segment<T, VEC, CHUNKS, false>(make_rsrc(in + seg_first, valid), lane, x);
        const T seg_total = scan_segment_local<T, EXCL, VEC, CHUNKS>(x);
        T* buf = s_wave[it & 1u];
        if (lane == 0) buf[wave] = seg_total;
        __syncthreads();
        T wave_pre = T(0), agg = T(0);
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (w == wave) wave_pre = agg;
            agg = agg + buf[w];
        }
        add_seed<T, VEC, CHUNKS>(x, seed + wave_pre);
        store_segment<T, VEC, CHUNKS, false>(make_rsrc(out + seg_first, valid), lane, x);
        seed = seed + agg;
    }
}

static_assert(kRtsThreads * 16 == (int)kRtsTileElems, "reduce-then-scan tiles are 256 threads x 16 elements");

template <class T, bool EXCL, int VEC, int CHUNKS>
static hipError_t launch_rts_typed(const RtsArgs& a, hipStream_t stream)
{
    const T* in = static_cast<const T*>(a.in);
    T* out = static_cast<T*>(a.out);
    T* part = static_cast<T*>(a.partials);
    uint64_t n = a.n;
    uint32_t nt = a.num_tiles, tpg = a.tiles_per_group, groups = a.groups;
    {
        void* args[] = {&in, &n, &nt, &tpg, &part};
        hipError_t e = hipLaunchKernel(
            reinterpret_cast<const void*>(&k_rts_reduce<T, kRtsThreads, VEC, CHUNKS>), dim3(groups),
            dim3(kRtsThreads), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    {
        void* args[] = {&part, &groups};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&k_rts_scan_partials<T>), dim3(1),
                                       dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    const T* pre = part;
    void* args[] = {&in, &out, &n, &nt, &tpg, &pre};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&k_rts_downsweep<T, EXCL, kRtsThreads, VEC, CHUNKS>), dim3(groups),
        dim3(kRtsThreads), args, 0, stream);
}

hipError_t launch_rts(const RtsArgs& a, hipStream_t stream)
{
    if (a.num_tiles == 0u) return hipSuccess;
    if (a.groups == 0u || a.groups > kRtsMaxGroups) return hipErrorInvalidValue;
    if (a.kind == kKindF32) {
        if (a.aligned)
            return a.exclusive ? launch_rts_typed<float, true, 4, 4>(a, stream)
                               : launch_rts_typed<float, false, 4, 4>(a, stream);
        return a.exclusive ? launch_rts_typed<float, true, 1, 16>(a, stream)
                           : launch_rts_typed<float, false, 1, 16>(a, stream);
    }
    if (a.aligned)
        return a.exclusive ? launch_rts_typed<uint32_t, true, 4, 4>(a, stream)
                           : launch_rts_typed<uint32_t, false, 4, 4>(a, stream);
    return a.exclusive ? launch_rts_typed<uint32_t, true, 1, 16>(a, stream)
                       : launch_rts_typed<uint32_t, false, 1, 16>(a, stream);
}

// ---------------------------------------------------------------------------
// Protocol-inspection kernel: one wavefront per tile, lane l holds element l
// of the tile (tile_elems <= 64; the other lanes hold the identity).
// ---------------------------------------------------------------------------
struct DebugParams {
    const void* in;
    void* out;
    uint64_t n;
    uint64_t* desc;
    unsigned long long* counter;
    unsigned int* watchdog;
    uint32_t num_tiles, tile_elems, delay_every, delay_phase, delay_ticks;
    unsigned int* epoch;
};

template <class T, bool EXCL, int MODE>
__global__ void __launch_bounds__(64) k_debug(DebugParams p)
{
    const int lane = lane_id();
    const bool multi = p.num_tiles > 1u;
    const uint32_t epoch = multi ? load_epoch(p.epoch) : 0u;
    uint32_t tile = 0u;
    if (multi) {
        uint32_t t = 0u;
        if (lane == 0) t = draw_tile(p.counter, p.num_tiles);
        tile = uniform(t);
        if (tile >= p.num_tiles) {   // counter not put back to 0: never index past the grid
            if (lane == 0) atomicAdd(p.watchdog, 1u);
            return;
        }
    }
    const uint64_t i = (uint64_t)tile * p.tile_elems + (uint64_t)lane;
    const bool valid = (uint32_t)lane < p.tile_elems && i < p.n;
    const T x = valid ? static_cast<const T*>(p.in)[i] : T(0);
    const T incl = wave_inclusive_scan(x);
    const T agg = wave_read_lane(incl, 63);

    if (p.delay_every != 0u && tile % p.delay_every == p.delay_phase) {
        const uint64_t t0 = realtime();
        while (realtime() - t0 < (uint64_t)p.delay_ticks) __builtin_amdgcn_s_sleep(8);
    }
    T prefix = T(0);
    if (multi) {
        if (tile == 0u) {
            if (lane == 0) desc_store<kOrderRelaxed>(desc_at(p.desc, 0u), desc_pack(epoch, kStatusP, Elem<T>::bits(agg)));
        } else {
            if constexpr (MODE == kModeDecoupled) {
                if (lane == 0)
                    desc_store<kOrderRelaxed>(desc_at(p.desc, tile), desc_pack(epoch, kStatusA, Elem<T>::bits(agg)));
                prefix = lookback_decoupled<T, kOrderRelaxed, kLookbackSlots>(p.desc, tile, epoch, p.watchdog);
            } else {
                prefix = lookback_chained<T, kOrderRelaxed>(p.desc, tile, epoch, p.watchdog);
            }
            if (lane == 0) {
                desc_store<kOrderRelaxed>(desc_at(p.desc, tile),
                                          desc_pack(epoch, kStatusP, Elem<T>::bits(prefix + agg)));
                if (tile == p.num_tiles - 1u) advance_epoch(p.epoch, epoch);
            }
        }
    }
    const T y = EXCL ? prefix + wave_shift_up1(incl) : prefix + incl;
    if (valid) static_cast<T*>(p.out)[i] = y;
}

template <class T, bool EXCL, int MODE>
static hipError_t launch_debug_typed(const DebugParams& p, hipStream_t stream)
{
    DebugParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_debug<T, EXCL, MODE>), dim3(p.num_tiles), dim3(64),
                           args, 0, stream);
}

hipError_t launch_debug(const DebugArgs& a, hipStream_t stream)
{
    if (a.num_tiles == 0u) return hipSuccess;
    if (a.tile_elems == 0u || a.tile_elems > kDebugMaxTile) return hipErrorInvalidValue;
    const DebugParams p{a.in, a.out, a.n, a.desc, a.counter, a.watchdog, a.num_tiles,
                        a.tile_elems, a.delay_every, a.delay_phase, a.delay_ticks, a.epoch};
    const bool ch = a.mode == kModeChained;
    if (a.kind == kKindF32) {
        if (a.exclusive)
            return ch ? launch_debug_typed<float, true, kModeChained>(p, stream)
                      : launch_debug_typed<float, true, kModeDecoupled>(p, stream);
        return ch ? launch_debug_typed<float, false, kModeChained>(p, stream)
                  : launch_debug_typed<float, false, kModeDecoupled>(p, stream);
    }
    if (a.exclusive)
        return ch ? launch_debug_typed<uint32_t, true, kModeChained>(p, stream)
                  : launch_debug_typed<uint32_t, true, kModeDecoupled>(p, stream);
    return ch ? launch_debug_typed<uint32_t, false, kModeChained>(p, stream)
              : launch_debug_typed<uint32_t, false, kModeDecoupled>(p, stream);
}

// ---------------------------------------------------------------------------
// Workspace initialiser.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    k_workspace_init(uint64_t* desc, uint64_t slots, unsigned long long* counter, unsigned int* epoch,
                     unsigned int* watchdog)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < slots; i += stride) desc[i] = 0ull;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (counter != nullptr) *counter = kCounterInit;
        if (epoch != nullptr) *epoch = 1u;
        if (watchdog != nullptr) *watchdog = 0u;
    }
}

hipError_t launch_workspace_init(uint64_t* desc, uint64_t slots, unsigned long long* counter, unsigned int* epoch,
                                 unsigned int* watchdog, hipStream_t stream)
{
    uint64_t blocks64 = (slots + 255u) / 256u;
    if (blocks64 < 1u) blocks64 = 1u;
    if (blocks64 > 1024u) blocks64 = 1024u;
    void* args[] = {&desc, &slots, &counter, &epoch, &watchdog};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_workspace_init), dim3((uint32_t)blocks64), dim3(256),
                           args, 0, stream);
}

// ---------------------------------------------------------------------------
// Wavefront-primitive self test.
// ---------------------------------------------------------------------------
template <class T>
__global__ void __launch_bounds__(64) k_wave_selftest(const T* in, T* incl, T* shift)
{
    const uint64_t i = (uint64_t)blockIdx.x * 64u + (uint64_t)lane_id();
    const T v = in[i];
    incl[i] = wave_inclusive_scan(v);
    shift[i] = wave_shift_up1(v);
}

hipError_t launch_wave_selftest(const void* in, void* incl, void* shift, uint64_t n_waves, int kind,
                                hipStream_t stream)
{
    if (n_waves == 0u) return hipSuccess;
    void* args[] = {&in, &incl, &shift};
    const void* fn = kind == kKindF32 ? reinterpret_cast<const void*>(&k_wave_selftest<float>)
                                      : reinterpret_cast<const void*>(&k_wave_selftest<uint32_t>);
    return hipLaunchKernel(fn, dim3((uint32_t)n_waves), dim3(64), args, 0, stream);
}

}  // namespace dws

// Scan-then-propagate comparison variant (~4n traffic): the hierarchical scan
// of the PMPP 11.3 notes (section on hierarchical / segmented scan: scan each
// block, scan the block sums, add the scanned sum of the previous blocks), in
// the recursive form of CUDA-Operators-6-Cumsum section 2 (the block sums are
// scanned by the same three steps until they fit one tile). Merrill & Garland
// (section 3.2) count its global traffic as ~4n: the local scan reads and
// writes n, the propagation reads and writes n again.
#include "dws_device.hpp"
#include "dws_internal.h"

namespace dws {

constexpr int kStpThreads = 256;

// Scan every tile on its own (no cross-tile carry), write the local result and
// the tile's total.
template <class T, bool EXCL, int VEC, int CHUNKS>
__global__ void __launch_bounds__(kStpThreads) k_stp_local(const T* in, T* out, uint64_t n, T* tile_sums)
{
    constexpr int W = kStpThreads / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    __shared__ T s_wave[W];
    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const uint64_t seg_first = (uint64_t)blockIdx.x * TILE + (uint64_t)wave * SEG;
    const uint32_t valid = valid_bytes(seg_first, SEG, n);
    T x[CHUNKS][VEC];
    load_segment<T, VEC, CHUNKS, false>(make_rsrc(in + seg_first, valid), lane, x);
    const T seg_total = scan_segment_local<T, EXCL, VEC, CHUNKS>(x);
    if (lane == 0) s_wave[wave] = seg_total;
    __syncthreads();
    T wave_pre = T(0), agg = T(0);
#pragma unroll
    for (int w = 0; w < W; ++w) {
        if (w == wave) wave_pre = agg;
        agg = agg + s_wave[w];
    }
    add_seed<T, VEC, CHUNKS>(x, wave_pre);
    store_segment<T, VEC, CHUNKS, false>(make_rsrc(out + seg_first, valid), lane, x);
    if (tile_sums != nullptr && threadIdx.x == 0) tile_sums[blockIdx.x] = agg;
}

// Add the (exclusive) scanned tile sums to tiles 1 .. num_tiles-1.
template <class T, int VEC, int CHUNKS>
__global__ void __launch_bounds__(kStpThreads) k_stp_add(T* out, uint64_t n, const T* tile_prefix)
{
    constexpr int W = kStpThreads / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const uint32_t tile = blockIdx.x + 1u;   // tile 0 has nothing before it
    const uint64_t seg_first = (uint64_t)tile * TILE + (uint64_t)wave * SEG;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(out + seg_first, valid_bytes(seg_first, SEG, n));
    const T seed = tile_prefix[tile];
    T x[CHUNKS][VEC];
    load_segment<T, VEC, CHUNKS, false>(r, lane, x);
    add_seed<T, VEC, CHUNKS>(x, seed);
    store_segment<T, VEC, CHUNKS, false>(r, lane, x);
}

static_assert(kStpTileElems == 4096u, "scan-then-propagate tiles are 256 threads x 16 elements");

uint64_t stp_scratch_elems(uint64_t n)
{
    uint64_t total = 0;
    uint64_t level = n;
    while (level > kStpTileElems) {
        level = (level + kStpTileElems - 1) / kStpTileElems;
        total += (level + 3u) & ~uint64_t(3);   // keep every level 16-byte aligned
    }
    return total;
}

template <class T, bool EXCL>
static hipError_t stp_level(const T* in, T* out, uint64_t n, T* scratch, hipStream_t stream)
{
    const uint64_t tiles = (n + kStpTileElems - 1) / kStpTileElems;
    T* sums = tiles > 1 ? scratch : nullptr;
    const bool aligned = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15u) == 0;
    {
        void* args[] = {&in, &out, &n, &sums};
        const void* fn = aligned ? reinterpret_cast<const void*>(&k_stp_local<T, EXCL, 4, 4>)
                                 : reinterpret_cast<const void*>(&k_stp_local<T, EXCL, 1, 16>);
        const hipError_t e = hipLaunchKernel(fn, dim3((uint32_t)tiles), dim3(kStpThreads), args, 0, stream);
        if (e != hipSuccess || tiles == 1) return e;
    }
    // scan the tile sums in place (exclusive), one level up
    T* rest = scratch + ((tiles + 3u) & ~uint64_t(3));
    hipError_t e = stp_level<T, true>(sums, sums, tiles, rest, stream);
    if (e != hipSuccess) return e;
    const T* pre = sums;
    void* args[] = {&out, &n, &pre};
    const bool out_aligned = (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
    const void* fn = out_aligned ? reinterpret_cast<const void*>(&k_stp_add<T, 4, 4>)
                                 : reinterpret_cast<const void*>(&k_stp_add<T, 1, 16>);
    return hipLaunchKernel(fn, dim3((uint32_t)(tiles - 1)), dim3(kStpThreads), args, 0, stream);
}

hipError_t launch_stp(const StpArgs& a, hipStream_t stream)
{
    if (a.n == 0) return hipSuccess;
    if (a.n > kStpTileElems && (a.scratch == nullptr || a.scratch_elems < stp_scratch_elems(a.n)))
        return hipErrorInvalidValue;
    if (a.kind == kKindF32) {
        const float* in = static_cast<const float*>(a.in);
        float* out = static_cast<float*>(a.out);
        float* s = static_cast<float*>(a.scratch);
        return a.exclusive ? stp_level<float, true>(in, out, a.n, s, stream)
                           : stp_level<float, false>(in, out, a.n, s, stream);
    }
    const uint32_t* in = static_cast<const uint32_t*>(a.in);
    uint32_t* out = static_cast<uint32_t*>(a.out);
    uint32_t* s = static_cast<uint32_t*>(a.scratch);
    return a.exclusive ? stp_level<uint32_t, true>(in, out, a.n, s, stream)
                       : stp_level<uint32_t, false>(in, out, a.n, s, stream);
}

}  // namespace dws

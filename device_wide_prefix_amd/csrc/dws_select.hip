// Fused stream compaction (select by flags) on the single-pass decoupled
// look-back: Merrill & Garland, section 4.4 (in-place compaction behaviour:
// scatter offsets come from a prefix sum of 0/1 flags; the look-back's
// signalling can guarantee that every predecessor has read its input before a
// tile writes, so the output may overwrite the input) and section A5
// (select-if fused with the scan, no extra pass).
//
// Per tile (one workgroup; the tile index is the workgroup index, or for an
// in-place select from 2^25 elements drawn from the workspace counter; same
// descriptor protocol and workspace as the scan):
//   1. load the flags, then the values of the tile (coalesced, in registers);
//   2. exclusive scan of the 0/1 flags in the tile -> each element's rank
//      among the tile's selected elements, and the tile's selected count;
//   3. publish {A, count}, look back over predecessors' counts -> the number
//      of selected elements before the tile, publish {P, prefix + count};
//   4. every selected element is stored to out[prefix + rank]: the selected
//      elements of a wave's segment are staged in LDS at their rank while
//      wave 0 is in the look-back, then stored with lane-contiguous dword
//      stores through a buffer resource based at the segment's first output
//      and ranged to its count (unselected elements write a spare LDS slot,
//      so the staging needs no branch).
//
// In place (ALIAS: out == in). Writes of tile t land in [prefix_t, prefix_t +
// count_t), which lies below the end of tile t and may reach into the input of
// any earlier tile. They are issued only after tile t knows its prefix, which
// needs an A or P of every earlier tile (a P is published only after its own
// tile's look-back, so by induction every earlier tile has published). What
// makes that safe is the order inside each tile: every wave consumes its value
// registers before the barrier that precedes the tile's A, which makes the
// compiler wait until every value load has returned its data (s_waitcnt
// vmcnt). So when any tile can see this tile's A, its whole input is already
// in registers, and no later store can change what it read. That wait is the
// load-ordering half of a release; the other half (writing back earlier
// stores) has nothing to order, since a tile stores only after its look-back.
// Out of place (ALIAS false) no tile writes another's input, and steps 2 and 3
// wait for the flags only, so the look-back runs while the values are still in
// flight.
//
// Partition (section A5, partition-if) is the same kernel with one more
// store: the rejected elements go to the back of the output in reverse input
// order, element i to out[n - 1 - (number of rejected elements before i)],
// which needs no total count. A wave stages its rejected elements from the
// back of its LDS stage, so they leave as one more contiguous block. Those
// writes land past the input's unread part, so the partition is never in
// place.
#include <type_traits>

#include "dws_device.hpp"
#include "dws_internal.h"

namespace dws {

struct SelectParams {
    const uint32_t* in;
    const uint32_t* flags;
    uint32_t* out;
    uint64_t n;
    uint64_t* desc;
    unsigned long long* counter;
    unsigned int* watchdog;
    unsigned long long* count;
    uint32_t num_tiles;
    unsigned int* epoch;
    uint32_t backoff;        // pause level between blocked look-back polls (kPause*)
    // predicate mode (PRED): element v is selected when bit c of pred_mask is
    // set, c being the outcome of comparing v with threshold in the element
    // type `kind` (kPredKindI32, kKindU32 or kKindF32): 0 less, 1 equal,
    // 2 greater, 3 unordered (a NaN)
    uint32_t pred_mask;
    uint32_t threshold;
    uint32_t kind;
};

// The comparison outcome of v against t as 32-bit patterns of `kind`.
__device__ __forceinline__ uint32_t compare_code(uint32_t v, uint32_t t, uint32_t kind)
{
    if (kind == (uint32_t)kKindF32) {
        const float a = __uint_as_float(v), b = __uint_as_float(t);
        if (a != a || b != b) return 3u;
        return a < b ? 0u : (a == b ? 1u : 2u);
    }
    if (kind == (uint32_t)kPredKindI32) {
        const int32_t a = (int32_t)v, b = (int32_t)t;
        return a < b ? 0u : (a == b ? 1u : 2u);
    }
    return v < t ? 0u : (v == t ? 1u : 2u);
}

template <int BLOCK, int VEC, int CHUNKS, bool PARTITION, int TILE_INDEX, bool NT = false, bool ALIAS = false,
          bool PRED = false>
__global__ void __launch_bounds__(BLOCK) k_select(SelectParams p)
{
    static_assert(!(PARTITION && ALIAS), "a partition is never in place");
    static_assert(VEC * CHUNKS <= 64, "one selection bit per element in a 64-bit mask");
    using Mask = typename std::conditional<(VEC * CHUNKS > 32), uint64_t, uint32_t>::type;
    constexpr int W = BLOCK / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    constexpr uint32_t CH = 64u * VEC;
    __shared__ uint32_t s_draw, s_epoch;
    __shared__ uint32_t s_wave[W];
    __shared__ uint32_t s_prefix;
    // per wave: the segment's selected elements by rank from the front (a
    // partition's rejected elements by rank from the back), then one spare
    // slot per lane that elements past n write to
    __shared__ uint32_t s_stage[W][SEG + 64];

    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const bool multi = p.num_tiles > 1u;
    // the descriptor epoch is read with the draw, or after the tile loads,
    // so that it never costs a round trip of its own (needed only to publish)
    uint32_t epoch_v = 0u;

    uint32_t tile = 0u;
    if (multi) {
        if constexpr (TILE_INDEX == kTileDispatch) {
            tile = blockIdx.x;
        } else {
            if (threadIdx.x == 0) {
                const uint32_t e = load_epoch_async(p.epoch);
                s_draw = draw_tile(p.counter, p.num_tiles);
                s_epoch = e;
            }
            __syncthreads();
            tile = uniform(s_draw);
            epoch_v = s_epoch;
            if (tile >= p.num_tiles) {   // counter not put back to 0: never index past the grid
                if (threadIdx.x == 0) atomicAdd(p.watchdog, 1u);
                return;
            }
        }
    }

    const uint64_t seg_first = (uint64_t)tile * TILE + (uint64_t)wave * SEG;
    const uint32_t seg_valid = valid_bytes(seg_first, SEG, p.n);
    uint32_t x[CHUNKS][VEC], r[CHUNKS][VEC];
    if constexpr (PRED) {
        // the selection comes from the values themselves: no flags to load
        load_segment<uint32_t, VEC, CHUNKS, NT>(make_rsrc(p.in + seg_first, seg_valid), lane, x);
    } else {
        // flags first: the tile's count (its aggregate) needs only the flags,
        // so out of place it is published and the look-back runs while the
        // values are in flight
        load_segment<uint32_t, VEC, CHUNKS, NT>(make_rsrc(p.flags + seg_first, seg_valid), lane, r);
        load_segment<uint32_t, VEC, CHUNKS, NT>(make_rsrc(p.in + seg_first, seg_valid), lane, x);
    }
    if constexpr (TILE_INDEX == kTileDispatch)
        if (multi && wave == 0) epoch_v = load_epoch_async(p.epoch);

    // selection bits, then ranks (exclusive scan of the 0/1 flags) in place
    Mask selected = 0u;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            uint32_t bit;
            if constexpr (PRED) {
                bit = (p.pred_mask >> compare_code(x[c][e], p.threshold, p.kind)) & 1u;
            } else {
                bit = r[c][e] != 0u ? 1u : 0u;
            }
            selected |= (Mask)bit << (c * VEC + e);
            r[c][e] = bit;
        }
    if constexpr (PRED) {
        // values past n load as 0, which a predicate may select: a ragged
        // segment (the array's last, uniform test) clears their bits
        if (seg_valid < SEG * 4u) {
            const uint32_t valid = seg_valid / 4u;
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if ((uint32_t)(c * (int)CH + lane * VEC + e) >= valid) {
                        selected &= ~((Mask)1 << (c * VEC + e));
                        r[c][e] = 0u;
                    }
        }
    }
    const uint32_t seg_count = scan_segment_local<uint32_t, true, VEC, CHUNKS>(r);
    pin_in_registers<uint32_t, VEC, CHUNKS>(r);
    // in place: the values must be in registers before this tile can publish
    // (the use below waits for every value load of the wave; the barrier then
    // covers every wave of the tile)
    if constexpr (ALIAS) pin_in_registers<uint32_t, VEC, CHUNKS>(x);

    if (lane == 0) s_wave[wave] = seg_count;
    __syncthreads();
    uint32_t wave_pre = 0u, count = 0u;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        if (w == wave) wave_pre = count;
        count += s_wave[w];
    }
    // uniform by construction (every lane read the same LDS words); saying so
    // keeps the buffer resources built from them in SGPRs (no per-store loop)
    count = uniform(count);
    wave_pre = uniform(wave_pre);

    if (wave == 0) {
        uint32_t prefix = 0u;
        if (multi) {
            const uint32_t epoch = uniform(epoch_v);
            if (tile == 0u) {
                if (lane == 0) desc_store<kOrderRelaxed>(desc_at(p.desc, 0u), desc_pack(epoch, kStatusP, count));
            } else {
                if (lane == 0) desc_store<kOrderRelaxed>(desc_at(p.desc, tile), desc_pack(epoch, kStatusA, count));
                prefix = lookback_decoupled<uint32_t, kOrderRelaxed, kLookbackSlots>(p.desc, tile, epoch,
                                                                                     p.watchdog, p.backoff);
                if (lane == 0) {
                    desc_store<kOrderRelaxed>(desc_at(p.desc, tile), desc_pack(epoch, kStatusP, prefix + count));
                    if (tile == p.num_tiles - 1u) advance_epoch(p.epoch, epoch);
                }
            }
        }
        if (lane == 0) s_prefix = prefix;
    }
    // While wave 0 waits in the look-back (wave 0 after it), every wave
    // stages its segment: a selected element at its rank in the segment (r
    // holds the exclusive scan of the selection bits), a partition's rejected
    // element j of the segment at SEG - 1 - j. Only the stores are left for
    // after the look-back. Against staging chunk by chunk after it, select
    // measured 2.5% faster out of place and 5.8% in place at 2^30 - 12,345
    // elements, 2 and 4% at 2^25.
    const uint32_t seg_elems = seg_valid / 4u;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const bool sel = (selected >> (c * VEC + e)) & 1u;
            uint32_t slot = sel ? r[c][e] : SEG + (uint32_t)lane;
            if constexpr (PARTITION) {
                const uint32_t idx = (uint32_t)(c * CH) + (uint32_t)(lane * VEC + e);
                if (!sel && idx < seg_elems) slot = SEG - 1u - (idx - r[c][e]);
            }
            s_stage[wave][slot] = x[c][e];
        }
    __syncthreads();
    const uint32_t prefix = uniform(s_prefix);
    // the segment's selected elements fill out[prefix + wave_pre ..): one
    // lane-contiguous store per 64 of them
    const uint32_t seg_n = uniform(seg_count);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.out + ((uint64_t)prefix + wave_pre), seg_n * 4u);
    for (uint32_t g = 0u; g < seg_n; g += 64u) {
        const uint32_t i = g + (uint32_t)lane;
        __builtin_amdgcn_raw_buffer_store_b32(s_stage[wave][i], rs, (int)(i * 4u), 0, 0);
    }
    if constexpr (PARTITION) {
        // the segment's rejected elements, rejected ranks rb .. rb + rej - 1
        // of the array, go to out[n - 1 - rank]: one contiguous block
        // starting at n - rb - rej, in the order they sit in slots
        // SEG - rej .. SEG - 1
        const uint32_t rej = uniform(seg_elems - seg_n);
        const uint64_t rb = seg_first - ((uint64_t)prefix + wave_pre);   // rejected before the segment
        const __amdgpu_buffer_rsrc_t rj = make_rsrc(p.out + (p.n - rb - rej), rej * 4u);
        for (uint32_t g = 0u; g < rej; g += 64u) {
            const uint32_t i = g + (uint32_t)lane;
            __builtin_amdgcn_raw_buffer_store_b32(s_stage[wave][SEG - rej + i], rj, (int)(i * 4u), 0, 0);
        }
    }
    if (tile == p.num_tiles - 1u && threadIdx.x == 0) *p.count = (unsigned long long)prefix + count;
}

__global__ void __launch_bounds__(64) k_store_count(unsigned long long* count, unsigned long long v)
{
    if (threadIdx.x == 0) *count = v;
}

struct SelectShape {
    int threads, vec, chunks;
    constexpr uint32_t elems() const { return (uint32_t)(threads * vec * chunks); }
};
// 32768-element tiles from kSelectLargeMin: with descriptors 64 bytes apart
// and the short pause between polls they measured 2.6 to 5% faster than
// 40960-element tiles (1024 x 4 x 10) at 2^27, 2^28 and 2^30 - 12,345
// elements, and 5 to 7% faster at 2^26 (the larger tile had been 5% faster at
// 2^30 with packed descriptors and a long back-off).
constexpr SelectShape kSelectLarge{1024, 4, 8};   // 32768
constexpr SelectShape kSelectSmall{256, 4, 4};    // 4096
constexpr SelectShape kSelectScalar{256, 1, 16};  // 4096, pointers not 16-byte aligned

static SelectShape select_shape(uint64_t n, bool aligned)
{
    if (!aligned) return kSelectScalar;
    return n >= kSelectLargeMin ? kSelectLarge : kSelectSmall;
}

uint32_t select_tile_elems(uint64_t n, bool aligned) { return select_shape(n, aligned).elems(); }

template <bool PARTITION, int TI, bool NT = false, bool ALIAS = false, bool PRED = false>
static const void* select_kernel(const SelectShape& s)
{
    if (s.vec == 1) return reinterpret_cast<const void*>(
        &k_select<kSelectScalar.threads, kSelectScalar.vec, kSelectScalar.chunks, PARTITION, TI, false, ALIAS, PRED>);
    if (s.threads == kSelectLarge.threads) return reinterpret_cast<const void*>(
        &k_select<kSelectLarge.threads, kSelectLarge.vec, kSelectLarge.chunks, PARTITION, TI, NT, ALIAS, PRED>);
    return reinterpret_cast<const void*>(
        &k_select<kSelectSmall.threads, kSelectSmall.vec, kSelectSmall.chunks, PARTITION, TI, false, ALIAS, PRED>);
}

// The kernel for these arguments; PRED: the selection comes from a
// predicate on the values (dws_select_if, dws_partition_if).
template <bool PRED>
static const void* pick_select_kernel(const SelectArgs& a, const SelectShape& s)
{
    const bool nt = a.n >= kSelectNtMin;
    const bool alias = !a.partition && a.out == a.in;
    if (a.partition)
        return nt ? select_kernel<true, kTileDispatch, true, false, PRED>(s)
                  : select_kernel<true, kTileDispatch, false, false, PRED>(s);
    if (alias)
        return a.n >= kSelectDrawnMin ? select_kernel<false, kTileDrawn, true, true, PRED>(s)
                                      : select_kernel<false, kTileDispatch, false, true, PRED>(s);
    return nt ? select_kernel<false, kTileDispatch, true, false, PRED>(s)
              : select_kernel<false, kTileDispatch, false, false, PRED>(s);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream)
{
    if (a.n == 0) {
        unsigned long long* c = a.count;
        unsigned long long zero = 0ull;
        void* args[] = {&c, &zero};
        return hipLaunchKernel(reinterpret_cast<const void*>(&k_store_count), dim3(1), dim3(64), args, 0, stream);
    }
    const SelectShape s = select_shape(a.n, a.aligned);
    SelectParams p{static_cast<const uint32_t*>(a.in), static_cast<const uint32_t*>(a.flags),
                   static_cast<uint32_t*>(a.out), a.n, a.desc, a.counter, a.watchdog, a.count, a.num_tiles,
                   a.epoch,
                   select_backoff(a.n), a.pred_mask, a.threshold, (uint32_t)a.kind};
    void* args[] = {&p};
    // The tile index is the workgroup index, as for the scan: no atomic on the
    // critical path; the watchdog still bounds every wait. From kSelectNtMin
    // elements (the large shape) the values and flags are loaded
    // non-temporally, each being read once. Against a drawn index with
    // non-temporal loads, alternating whole library builds in one session
    // measured partition 81.7 -> 76.8 us and select 67.6 -> 66.9 us at 2^25,
    // and select 1,797.7 -> 1,789.7 us at 2^30 - 12,345.
    // In place (select only) the kernel waits for its values before it
    // publishes, which is what makes writing over the input safe. There the
    // drawn index stays from kSelectDrawnMin (with non-temporal loads): with
    // the workgroup index the in-place select of the 2^30 - 12,345 flags
    // measured 1.84 to 2.01 ms (mean 1.943) against 1.795 to 1.930 (mean
    // 1.844).
    const void* fn = a.pred ? pick_select_kernel<true>(a, s) : pick_select_kernel<false>(a, s);
    return hipLaunchKernel(fn, dim3(a.num_tiles), dim3(s.threads), args, 0, stream);
}

}  // namespace dws

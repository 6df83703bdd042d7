// Single-pass decoupled look-back scan under a generic associative operator
// (Merrill & Garland, "Single-pass Parallel Prefix Scan with Decoupled
// Look-back", section 4.2: only contiguous inputs or contiguous partial
// reductions are ever combined, so the operator need not be commutative;
// section A4: 32-bit integers and {int32, fp32} pairs).
//
// Same tile structure as the + kernel (one workgroup per tile, coalesced
// buffer loads into registers, wave64 DPP scans, wave totals through LDS, one
// wave runs the look-back), with every combine taking its operands in input
// order: combine(earlier, later). The pieces that differ from the + kernel:
//   - DPP lanes without a source keep the operator's identity (the + kernel
//     lets them read 0);
//   - the look-back reduces each window of predecessors in tile order (the
//     + kernel sums lanes in any order);
//   - an element of two 32-bit words is published as two descriptor words,
//     each carrying the same epoch and status. A reader accepts a descriptor
//     only when both words carry the same tag; each tag is written once per
//     tile and launch, so equal tags mean both words come from the same
//     write (a torn read is polled again).
#pragma once

#include <utility>

#include "dws_device.hpp"
#include "dws_internal.h"

namespace dws {

template <int W>
struct Val {
    uint32_t w[W];
};

__device__ __forceinline__ float u2f(uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------------------
// Operators: kWords 32-bit words per element, identity(), combine(p, q) with
// p the earlier operand.
// ---------------------------------------------------------------------------
struct OpMaxI32 {
    static constexpr int kWords = 1;
    using V = Val<1>;
    static __device__ __forceinline__ V identity() { return {{0x80000000u}}; }
    static __device__ __forceinline__ V combine(V p, V q)
    {
        return {{(uint32_t)max((int32_t)p.w[0], (int32_t)q.w[0])}};
    }
};

struct OpMaxU32 {
    static constexpr int kWords = 1;
    using V = Val<1>;
    static __device__ __forceinline__ V identity() { return {{0u}}; }
    static __device__ __forceinline__ V combine(V p, V q) { return {{max(p.w[0], q.w[0])}}; }
};

struct OpMinI32 {
    static constexpr int kWords = 1;
    using V = Val<1>;
    static __device__ __forceinline__ V identity() { return {{0x7fffffffu}}; }
    static __device__ __forceinline__ V combine(V p, V q)
    {
        return {{(uint32_t)min((int32_t)p.w[0], (int32_t)q.w[0])}};
    }
};

struct OpMinU32 {
    static constexpr int kWords = 1;
    using V = Val<1>;
    static __device__ __forceinline__ V identity() { return {{0xffffffffu}}; }
    static __device__ __forceinline__ V combine(V p, V q) { return {{min(p.w[0], q.w[0])}}; }
};

// {int32, fp32}: componentwise +, the integer part modulo 2^32.
struct OpSumPairIF {
    static constexpr int kWords = 2;
    using V = Val<2>;
    static __device__ __forceinline__ V identity() { return {{0u, 0u}}; }
    static __device__ __forceinline__ V combine(V p, V q)
    {
        return {{p.w[0] + q.w[0], f2u(u2f(p.w[1]) + u2f(q.w[1]))}};
    }
};

struct OpSumPairU32 {
    static constexpr int kWords = 2;
    using V = Val<2>;
    static __device__ __forceinline__ V identity() { return {{0u, 0u}}; }
    static __device__ __forceinline__ V combine(V p, V q) { return {{p.w[0] + q.w[0], p.w[1] + q.w[1]}}; }
};

// (a, b) is the map v -> a v + b modulo 2^32; combine is "p, then q".
struct OpAffineU32 {
    static constexpr int kWords = 2;
    using V = Val<2>;
    static __device__ __forceinline__ V identity() { return {{1u, 0u}}; }
    static __device__ __forceinline__ V combine(V p, V q) { return {{q.w[0] * p.w[0], q.w[0] * p.w[1] + q.w[1]}}; }
};

// (flag, value): a non-zero flag restarts the running value; flags OR up.
struct OpSegSumU32 {
    static constexpr int kWords = 2;
    using V = Val<2>;
    static __device__ __forceinline__ V identity() { return {{0u, 0u}}; }
    static __device__ __forceinline__ V combine(V p, V q)
    {
        return {{p.w[0] | q.w[0], q.w[0] != 0u ? q.w[1] : p.w[1] + q.w[1]}};
    }
};

struct OpSegSumIF {
    static constexpr int kWords = 2;
    using V = Val<2>;
    static __device__ __forceinline__ V identity() { return {{0u, 0u}}; }
    static __device__ __forceinline__ V combine(V p, V q)
    {
        return {{p.w[0] | q.w[0], q.w[0] != 0u ? q.w[1] : f2u(u2f(p.w[1]) + u2f(q.w[1]))}};
    }
};

// ---------------------------------------------------------------------------
// Wavefront primitives under Op.
// ---------------------------------------------------------------------------
enum : int {
    kDppRowShl1 = 0x101,
    kDppRowShl2 = 0x102,
    kDppRowShl4 = 0x104,
    kDppRowShl8 = 0x108,
};

// DPP move of every word; lanes without a source (or in a disabled row) keep
// the identity.
template <class Op, int CTRL, int ROW_MASK>
__device__ __forceinline__ typename Op::V dpp_op(typename Op::V v)
{
    const typename Op::V id = Op::identity();
    typename Op::V r;
#pragma unroll
    for (int k = 0; k < Op::kWords; ++k)
        r.w[k] = (uint32_t)__builtin_amdgcn_update_dpp((int)id.w[k], (int)v.w[k], CTRL, ROW_MASK, 0xf, false);
    return r;
}

// Inclusive scan over the 64 lanes in lane order: Kogge-Stone within each row
// of 16, then row 1 and row 3 take the last lane of the row before them, rows
// 2 and 3 take lane 31. Every step combines (lower lanes, own value).
template <class Op>
__device__ __forceinline__ typename Op::V wave_scan_op(typename Op::V v)
{
    v = Op::combine(dpp_op<Op, kDppRowShr1, 0xf>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowShr2, 0xf>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowShr4, 0xf>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowShr8, 0xf>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowBcast15, 0xa>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowBcast31, 0xc>(v), v);
    return v;
}

// The previous lane's value; lane 0 gets the identity.
template <class Op>
__device__ __forceinline__ typename Op::V wave_shift_up1_op(typename Op::V v)
{
    return dpp_op<Op, kDppWaveShr1, 0xf>(v);
}

template <class Op>
__device__ __forceinline__ typename Op::V wave_read_lane_op(typename Op::V v, int lane)
{
    typename Op::V r;
#pragma unroll
    for (int k = 0; k < Op::kWords; ++k) r.w[k] = (uint32_t)__builtin_amdgcn_readlane((int)v.w[k], lane);
    return r;
}

// Combination of all 64 lanes with lane 63 first and lane 0 last (the order
// of the look-back window, where lane l holds an earlier tile than lane l-1).
// Within each row lane l combines (lane l + s, own value); lane 16 r then
// holds its row, and the rows are combined 3, 2, 1, 0. Uniform result.
template <class Op>
__device__ __forceinline__ typename Op::V wave_reduce_reversed_op(typename Op::V v)
{
    v = Op::combine(dpp_op<Op, kDppRowShl1, 0xf>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowShl2, 0xf>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowShl4, 0xf>(v), v);
    v = Op::combine(dpp_op<Op, kDppRowShl8, 0xf>(v), v);
    const typename Op::V r3 = wave_read_lane_op<Op>(v, 48);
    const typename Op::V r2 = wave_read_lane_op<Op>(v, 32);
    const typename Op::V r1 = wave_read_lane_op<Op>(v, 16);
    const typename Op::V r0 = wave_read_lane_op<Op>(v, 0);
    return Op::combine(Op::combine(Op::combine(r3, r2), r1), r0);
}

// ---------------------------------------------------------------------------
// Tile I/O in 32-bit words: lane l of chunk c moves LOADW consecutive words at
// word offset (64 c + l) LOADW of the wave segment (one dwordx4, dwordx2 or
// dword access per chunk); element e of the lane is words [e W, e W + W).
// ---------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int LOADW, int CHUNKS, bool NT>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, int lane, uint32_t (&raw)[CHUNKS][LOADW])
{
    constexpr int aux = NT ? kBufferNonTemporal : 0;
    const int voff = lane * LOADW * 4;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const int soff = c * 64 * LOADW * 4;
        if constexpr (LOADW == 4) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, aux);
#pragma unroll
            for (int k = 0; k < 4; ++k) raw[c][k] = v[k];
        } else if constexpr (LOADW == 2) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, aux);
            raw[c][0] = v[0];
            raw[c][1] = v[1];
        } else {
            raw[c][0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, aux);
        }
    }
}

template <int LOADW, int CHUNKS>
__device__ __forceinline__ void store_words(__amdgpu_buffer_rsrc_t r, int lane, const uint32_t (&raw)[CHUNKS][LOADW])
{
    const int voff = lane * LOADW * 4;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const int soff = c * 64 * LOADW * 4;
        if constexpr (LOADW == 4) {
            u32x4 v;
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = raw[c][k];
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
        } else if constexpr (LOADW == 2) {
            u32x2 v;
            v[0] = raw[c][0];
            v[1] = raw[c][1];
            __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(raw[c][0], r, voff, soff, 0);
        }
    }
}

// Valid bytes of `len` elements of `esize` bytes from element `first` of n.
__device__ __forceinline__ uint32_t valid_bytes_sized(uint64_t first, uint32_t len, uint64_t n, uint32_t esize)
{
    const uint64_t left = first < n ? n - first : 0u;
    return (uint32_t)((left < len ? left : len) * esize);
}

// Scan of one wave segment in registers, in place, as scan_segment_local of
// the + kernel: in-lane prefix, then (earlier chunks, lower lanes) combined in
// front of it. Returns the segment's combination (uniform).
template <class Op, bool EXCL, int E, int CHUNKS>
__device__ __forceinline__ typename Op::V scan_segment_op(typename Op::V (&x)[CHUNKS][E])
{
    using V = typename Op::V;
    V running = Op::identity();
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        V lane_total = x[c][0];
        if constexpr (EXCL) x[c][0] = Op::identity();
#pragma unroll
        for (int e = 1; e < E; ++e) {
            const V xe = x[c][e];
            if constexpr (EXCL) {
                x[c][e] = lane_total;
                lane_total = Op::combine(lane_total, xe);
            } else {
                lane_total = Op::combine(lane_total, xe);
                x[c][e] = lane_total;
            }
        }
        const V incl = wave_scan_op<Op>(lane_total);
        const V offset = Op::combine(running, wave_shift_up1_op<Op>(incl));
#pragma unroll
        for (int e = 0; e < E; ++e) x[c][e] = Op::combine(offset, x[c][e]);
        running = Op::combine(running, wave_read_lane_op<Op>(incl, 63));
    }
    return running;
}

// ---------------------------------------------------------------------------
// Descriptors of W words per tile (words desc_at(tile) .. + W - 1; W is at
// most 2, within the tile's kDescStride words).
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ void desc_store_val(uint64_t* desc, uint32_t tile, uint32_t epoch, uint32_t status,
                                               const Val<W>& v)
{
#pragma unroll
    for (int k = 0; k < W; ++k)
        desc_store<kOrderRelaxed>(desc_at(desc, tile) + k, desc_pack(epoch, status, v.w[k]));
}

// Look-back slots per lane of the generic-operator kernels: two, 128
// predecessors per poll. On 1 GiB inputs, against one slot: pair operators 0.1
// to 2% faster, max/min within 1%; four slots were no better.
constexpr int kOpLookbackSlots = 2;

// Decoupled look-back under Op (section 4.4, parallelized look-back, K slots
// per lane as in the + kernel): the window's needed descriptors (back to and
// including the nearest P) are combined in tile order, earliest first, and the
// window goes in front of what nearer windows gave. Returns the exclusive
// prefix of `tile` (uniform); a wait beyond kWatchdogTicks counts a trip and
// returns what it has. Back-off as in the + kernel's look-back: the pause of
// level `backoff` (lookback_pause) before every poll after the first re-poll.
template <class Op, int K>
__device__ typename Op::V lookback_op(const uint64_t* desc, uint32_t tile, uint32_t epoch, unsigned int* watchdog,
                                      uint32_t backoff = kPauseShort)
{
    using V = typename Op::V;
    constexpr int W = Op::kWords;
    const int lane = lane_id();
    const uint64_t lane_bit = 1ull << lane;
    V prefix = Op::identity();
    int64_t hi = (int64_t)tile - 1;
    const uint64_t t0 = realtime();
    bool repolled = false;
    V d[K];
    uint32_t st[K];
    // lanes of each slot that the next poll loads: all of a new window; after
    // a blocked poll only the descriptors still awaited (as in the + kernel's
    // look-back; 4 to 6.5% faster for reduce-by-key and 1.5 to 2% for
    // run-length encoding at 2^25 keys, equal for the generic operators)
    uint64_t reload[K];
#pragma unroll
    for (int j = 0; j < K; ++j) reload[j] = ~0ull;
    for (;;) {
        // every slot's loads are issued before any is examined: one round
        // trip per poll whatever K is
        uint64_t wd[K][W];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t idx = hi - (int64_t)(j * 64 + lane);
#pragma unroll
            for (int k = 0; k < W; ++k) wd[j][k] = 0ull;
            if ((reload[j] & lane_bit) && idx >= 0) {
#pragma unroll
                for (int k = 0; k < W; ++k) wd[j][k] = desc_load<kOrderRelaxed>(desc_at(desc, (uint64_t)idx) + k);
            }
        }
        uint64_t has_p[K], has_x[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t idx = hi - (int64_t)(j * 64 + lane);
            if (reload[j] & lane_bit) {
                st[j] = kStatusP;
                d[j] = Op::identity();
                if (idx >= 0) {
                    st[j] = desc_status(wd[j][0], epoch);
#pragma unroll
                    for (int k = 1; k < W; ++k)
                        if ((wd[j][k] >> 32) != (wd[j][0] >> 32)) st[j] = kStatusX;
#pragma unroll
                    for (int k = 0; k < W; ++k) d[j].w[k] = (uint32_t)wd[j][k];
                }
            }
            has_p[j] = __builtin_amdgcn_ballot_w64(st[j] == kStatusP);
            has_x[j] = __builtin_amdgcn_ballot_w64(st[j] == kStatusX);
        }
        int jp = K;
#pragma unroll
        for (int j = K - 1; j >= 0; --j)
            if (has_p[j]) jp = j;
        bool blocked = false;
        uint64_t need_p = 0ull;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (j < jp && has_x[j]) blocked = true;
            if (j == jp) {
                need_p = has_p[j] ^ (has_p[j] - 1ull);   // lanes 0 .. lowest P
                if (has_x[j] & need_p) blocked = true;
            }
        }
        if (!blocked) {
            V win = Op::identity();
#pragma unroll
            for (int j = K - 1; j >= 0; --j) {
                if (j > jp) continue;
                const uint64_t need = (j < jp) ? ~0ull : need_p;
                const V v = (need & lane_bit) ? d[j] : Op::identity();
                win = Op::combine(win, wave_reduce_reversed_op<Op>(v));
            }
            prefix = Op::combine(win, prefix);
            if (jp < K) return prefix;
            hi -= 64 * K;
#pragma unroll
            for (int j = 0; j < K; ++j) reload[j] = ~0ull;
            continue;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) reload[j] = j < jp ? has_x[j] : (j == jp ? has_x[j] & need_p : 0ull);
        if (realtime() - t0 > kWatchdogTicks) {
            if (lane == 0) atomicAdd(watchdog, 1u);
            return prefix;
        }
        lookback_pause(backoff, !repolled);
        repolled = true;
    }
}

// ---------------------------------------------------------------------------
// The kernel. LOADW words per lane per chunk load (4: dwordx4), E = LOADW / W
// elements per lane per chunk.
// ---------------------------------------------------------------------------
template <class Op, bool EXCL, int BLOCK, int LOADW, int CHUNKS, bool NT = false>
__global__ void __launch_bounds__(BLOCK) k_scan_op(OpScanParams p)
{
    using V = typename Op::V;
    constexpr int W = Op::kWords;
    static_assert(LOADW % W == 0, "whole elements per load");
    constexpr int E = LOADW / W;
    constexpr int WAVES = BLOCK / 64;
    constexpr uint32_t SEG = 64u * E * CHUNKS;
    constexpr uint32_t TILE = WAVES * SEG;
    constexpr uint32_t ESIZE = 4u * W;
    __shared__ V s_wave[WAVES];
    __shared__ V s_prefix;

    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const bool multi = p.num_tiles > 1u;
    // the descriptor epoch is read in wave 0 after the tile loads are issued:
    // it is needed only to publish, and never costs a round trip of its own
    uint32_t epoch_v = 0u;
    // the tile index is the workgroup index (each XCD starts its workgroups
    // in index order; the watchdog bounds every wait)
    const uint32_t tile = multi ? (uint32_t)blockIdx.x : 0u;

    const uint64_t seg_first = (uint64_t)tile * TILE + (uint64_t)wave * SEG;
    const uint32_t vb = valid_bytes_sized(seg_first, SEG, p.n, ESIZE);
    uint32_t raw[CHUNKS][LOADW];
    load_words<LOADW, CHUNKS, NT>(make_rsrc(static_cast<const char*>(p.in) + seg_first * ESIZE, vb), lane, raw);
    if (multi && wave == 0) epoch_v = load_epoch_async(p.epoch);
    // a seeded scan: tile 0's prefix is the caller's element, the earlier
    // operand of every combine it enters, read while the tile's loads are in
    // flight
    V seed_v = Op::identity();
    if (p.seed != nullptr && tile == 0u && wave == 0) {
#pragma unroll
        for (int k = 0; k < W; ++k) seed_v.w[k] = static_cast<const uint32_t*>(p.seed)[k];
    }

    V x[CHUNKS][E];
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
            for (int k = 0; k < W; ++k) x[c][e].w[k] = raw[c][e * W + k];

    const V seg_total = scan_segment_op<Op, EXCL, E, CHUNKS>(x);
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
            for (int k = 0; k < W; ++k) asm volatile("" : "+v"(x[c][e].w[k]));

    if (lane == 0) s_wave[wave] = seg_total;
    __syncthreads();
    V wave_pre = Op::identity(), agg = Op::identity();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        if (w == wave) wave_pre = agg;
        agg = Op::combine(agg, s_wave[w]);
    }

    if (wave == 0) {
        V prefix;
#pragma unroll
        for (int k = 0; k < W; ++k) prefix.w[k] = uniform(seed_v.w[k]);
        if (multi) {
            const uint32_t epoch = uniform(epoch_v);
            if (tile == 0u) {
                if (lane == 0) desc_store_val<W>(p.desc, 0u, epoch, kStatusP, Op::combine(prefix, agg));
            } else {
                if (lane == 0) desc_store_val<W>(p.desc, tile, epoch, kStatusA, agg);
                prefix = lookback_op<Op, kOpLookbackSlots>(p.desc, tile, epoch, p.watchdog, p.backoff);
                if (lane == 0) {
                    desc_store_val<W>(p.desc, tile, epoch, kStatusP, Op::combine(prefix, agg));
                    if (tile == p.num_tiles - 1u) advance_epoch(p.epoch, epoch);
                }
            }
        }
        if (lane == 0) s_prefix = prefix;
    }
    __syncthreads();
    const V seed = Op::combine(s_prefix, wave_pre);

#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const V y = Op::combine(seed, x[c][e]);
#pragma unroll
            for (int k = 0; k < W; ++k) raw[c][e * W + k] = y.w[k];
        }
    store_words<LOADW, CHUNKS>(make_rsrc(static_cast<char*>(p.out) + seg_first * ESIZE, vb), lane, raw);
}

// ---------------------------------------------------------------------------
// Reduction under Op to one element (the shard total of a split scan, as
// dws_reduce for +). The grid and the partials follow the + reduction: at
// most kReduceMaxGroups workgroups of BLOCK threads each combine a contiguous
// run of tiles and publish the result as a descriptor of W tagged words; the
// highest-indexed workgroup combines the partials in index order and writes
// the total. Every combine keeps input order: a wave's segment is combined
// chunk by chunk (in-lane, then across lanes by an in-order wave scan), a
// tile's segments wave by wave through LDS, the group's tiles one after the
// other, and the partials in index order (thread q of the last group takes
// partials q PER .. q PER + PER - 1, lanes and waves in order).
// ---------------------------------------------------------------------------
template <class Op, int BLOCK, int LOADW, int CHUNKS, bool NT>
__global__ void __launch_bounds__(BLOCK) k_reduce_op(OpReduceParams p)
{
    using V = typename Op::V;
    constexpr int W = Op::kWords;
    static_assert(LOADW % W == 0, "whole elements per load");
    constexpr int E = LOADW / W;
    constexpr int WAVES = BLOCK / 64;
    constexpr uint32_t SEG = 64u * E * CHUNKS;
    constexpr uint32_t TILE = WAVES * SEG;
    constexpr uint32_t ESIZE = 4u * W;
    constexpr int PER = (int)(kReduceMaxGroups / BLOCK);
    static_assert(PER * BLOCK == (int)kReduceMaxGroups, "the last group reads every partial in one round");
    // double-buffered: tile i + 2 overwrites a buffer only after every wave has
    // passed the barrier of tile i + 1, i.e. has read tile i's totals
    __shared__ V s_wave[2][WAVES];
    __shared__ V s_fin[WAVES];
    __shared__ uint32_t s_epoch;
    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const uint32_t g = blockIdx.x;
    const uint64_t t0 = (uint64_t)g * p.tiles_per_group;
    const uint64_t t_end = t0 + p.tiles_per_group;
    const uint64_t t1 = t_end < (uint64_t)p.num_tiles ? t_end : (uint64_t)p.num_tiles;
    uint32_t epoch_v = 0u;
    if (wave == 0) epoch_v = load_epoch_async(p.epoch);

    V acc = Op::identity();
    uint32_t it = 0;
    for (uint64_t t = t0; t < t1; ++t, ++it) {
        const uint64_t seg_first = t * TILE + (uint64_t)wave * SEG;
        const uint32_t vb = valid_bytes_sized(seg_first, SEG, p.n, ESIZE);
        uint32_t raw[CHUNKS][LOADW];
        load_words<LOADW, CHUNKS, NT>(make_rsrc(static_cast<const char*>(p.in) + seg_first * ESIZE, vb), lane, raw);
        // words past n load as 0, which is not every operator's identity: a
        // ragged segment (the array's last, uniform test) puts the identity
        // in their place
        if (vb < SEG * ESIZE) {
            const uint32_t valid = vb / ESIZE;
            const V id = Op::identity();
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if ((uint32_t)((c * 64 + lane) * E + e) >= valid) {
#pragma unroll
                        for (int k = 0; k < W; ++k) raw[c][e * W + k] = id.w[k];
                    }
        }
        V seg = Op::identity();
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            V lane_total;
#pragma unroll
            for (int k = 0; k < W; ++k) lane_total.w[k] = raw[c][k];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                V xe;
#pragma unroll
                for (int k = 0; k < W; ++k) xe.w[k] = raw[c][e * W + k];
                lane_total = Op::combine(lane_total, xe);
            }
            seg = Op::combine(seg, wave_read_lane_op<Op>(wave_scan_op<Op>(lane_total), 63));
        }
        V* buf = s_wave[it & 1u];
        if (lane == 0) buf[wave] = seg;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) acc = Op::combine(acc, buf[w]);
    }

    if (threadIdx.x == 0) {
        const uint32_t e = uniform(epoch_v);
        desc_store_val<W>(p.desc, g, e, kStatusP, acc);
        s_epoch = e;
    }
    if (g != p.groups - 1u) return;
    __syncthreads();
    const uint32_t epoch = uniform(s_epoch);

    // the last group: thread q combines partials q PER .. q PER + PER - 1
    const uint32_t q0 = threadIdx.x * (uint32_t)PER;
    uint64_t d[PER][W];
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int k = 0; k < W; ++k)
            d[j][k] = q0 + j < p.groups ? desc_load<kOrderRelaxed>(desc_at(p.desc, q0 + j) + k)
                                        : desc_pack(epoch, kStatusP, Op::identity().w[k]);
    const uint64_t start = realtime();
    for (;;) {
        bool waiting = false;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            bool torn = false;
#pragma unroll
            for (int k = 1; k < W; ++k) torn = torn || (d[j][k] >> 32) != (d[j][0] >> 32);
            if (torn || desc_status(d[j][0], epoch) == kStatusX) waiting = true;
        }
        if (!waiting) break;
        if (realtime() - start > kWatchdogTicks) {
            atomicAdd(p.watchdog, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            bool torn = false;
#pragma unroll
            for (int k = 1; k < W; ++k) torn = torn || (d[j][k] >> 32) != (d[j][0] >> 32);
            if (torn || desc_status(d[j][0], epoch) == kStatusX) {
#pragma unroll
                for (int k = 0; k < W; ++k) d[j][k] = desc_load<kOrderRelaxed>(desc_at(p.desc, q0 + j) + k);
            }
        }
    }
    V v = Op::identity();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        V pj;
#pragma unroll
        for (int k = 0; k < W; ++k) pj.w[k] = (uint32_t)d[j][k];
        v = Op::combine(v, pj);
    }
    const V wv = wave_read_lane_op<Op>(wave_scan_op<Op>(v), 63);
    if (lane == 0) s_fin[wave] = wv;
    __syncthreads();
    if (threadIdx.x == 0) {
        V total = Op::identity();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) total = Op::combine(total, s_fin[w]);
#pragma unroll
        for (int k = 0; k < W; ++k) static_cast<uint32_t*>(p.total)[k] = total.w[k];
        advance_epoch(p.epoch, epoch);
    }
}

template <class Op, int BLOCK, int LOADW, int CHUNKS, bool NT = false>
static hipError_t launch_reduce_op_shape(const OpReduceParams& p, hipStream_t stream)
{
    OpReduceParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_reduce_op<Op, BLOCK, LOADW, CHUNKS, NT>),
                           dim3(p.groups), dim3(BLOCK), args, 0, stream);
}

// The reduction's shapes: 16-byte aligned inputs load dwordx4 (8 loads per
// lane, non-temporal as the caller asks), others one element per access
// (16 per lane); kReduceThreads threads either way (op_reduce_tile_elems).
template <class Op>
hipError_t launch_reduce_op_typed(bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream)
{
    constexpr int W = Op::kWords;
    if (!aligned) return launch_reduce_op_shape<Op, kReduceThreads, W, 16>(p, stream);
    return nt ? launch_reduce_op_shape<Op, kReduceThreads, 4, 8, true>(p, stream)
              : launch_reduce_op_shape<Op, kReduceThreads, 4, 8>(p, stream);
}

// ---------------------------------------------------------------------------
// Shapes and launch. Shapes are (threads, words per load, loads per lane);
// the unaligned shape loads one element per access.
// ---------------------------------------------------------------------------
template <class Op, bool EXCL, int BLOCK, int LOADW, int CHUNKS, bool NT = false>
static hipError_t launch_op_shape(const OpScanParams& p, hipStream_t stream)
{
    OpScanParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_scan_op<Op, EXCL, BLOCK, LOADW, CHUNKS, NT>),
                           dim3(p.num_tiles), dim3(BLOCK), args, 0, stream);
}

template <class Op, bool EXCL>
static hipError_t launch_op_excl(int shape, bool nt, const OpScanParams& p, hipStream_t stream)
{
    constexpr int W = Op::kWords;
    switch (shape) {
    case kOpShapeSmall: return launch_op_shape<Op, EXCL, 256, 4, 4>(p, stream);
    case kOpShapeMedium: return launch_op_shape<Op, EXCL, 512, 4, 8>(p, stream);
    case kOpShapeLarge:
        // non-temporal loads are built for the large shape only, which the
        // caller uses them with from kOpNtMin elements
        return nt ? launch_op_shape<Op, EXCL, 1024, 4, 16, true>(p, stream)
                  : launch_op_shape<Op, EXCL, 1024, 4, 16>(p, stream);
    case kOpShapeUnaligned: return launch_op_shape<Op, EXCL, 256, W, 16>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <class Op>
hipError_t launch_op_typed(bool exclusive, int shape, bool nt, const OpScanParams& p, hipStream_t stream)
{
    return exclusive ? launch_op_excl<Op, true>(shape, nt, p, stream)
                     : launch_op_excl<Op, false>(shape, nt, p, stream);
}

}  // namespace dws

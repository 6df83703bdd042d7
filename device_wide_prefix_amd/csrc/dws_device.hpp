// Device primitives of the gfx950 scan kernels: wavefront (wave64) scans on
// DPP, tile loads/stores, the packed tile descriptor and the look-back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dws_protocol.h"

namespace dws {

// ---------------------------------------------------------------------------
// Element traits. Both 32-bit integer types run as uint32_t (wrapping adds are
// the same bits for int32 and uint32), fp32 runs as float.
// ---------------------------------------------------------------------------
template <class T> struct Elem;

template <> struct Elem<uint32_t> {
    static __device__ __forceinline__ uint32_t bits(uint32_t v) { return v; }
    static __device__ __forceinline__ uint32_t from(uint32_t b) { return b; }
    // value a disabled DPP lane contributes: the identity of +
    static constexpr uint32_t kDppOld = 0u;
};

template <> struct Elem<float> {
    static __device__ __forceinline__ uint32_t bits(float v) { return __float_as_uint(v); }
    static __device__ __forceinline__ float from(uint32_t b) { return __uint_as_float(b); }
    // -0.0 is the exact identity of IEEE addition (x + -0.0 == x for all x,
    // +0.0 included); it also lets the compiler fold the DPP move into the add
    static constexpr uint32_t kDppOld = 0x80000000u;
};

// ---------------------------------------------------------------------------
// Wavefront primitives on DPP. A wave64 is four rows of 16 lanes.
// ---------------------------------------------------------------------------
enum : int {
    kDppRowShr1 = 0x111,
    kDppRowShr2 = 0x112,
    kDppRowShr4 = 0x114,
    kDppRowShr8 = 0x118,
    kDppWaveShr1 = 0x138,   // whole-wave shift by one lane
    kDppRowBcast15 = 0x142, // lane 15 of each row -> the next row
    kDppRowBcast31 = 0x143, // lane 31 -> rows 2 and 3
};

template <int CTRL, int ROW_MASK, bool ZERO_OUT_OF_ROW, class T>
__device__ __forceinline__ T dpp_read(T v)
{
    return Elem<T>::from((uint32_t)__builtin_amdgcn_update_dpp(
        (int)Elem<T>::kDppOld, (int)Elem<T>::bits(v), CTRL, ROW_MASK, 0xf, ZERO_OUT_OF_ROW));
}

// Inclusive + scan over the 64 lanes in lane order. Within each row a
// Kogge-Stone doubling (shifts 1, 2, 4, 8; lanes shifted in from outside the
// row read 0), then the row totals are carried forward: row 1 and row 3 add
// the last lane of the row before them, rows 2 and 3 add lane 31.
template <class T>
__device__ __forceinline__ T wave_inclusive_scan(T v)
{
    v = v + dpp_read<kDppRowShr1, 0xf, true>(v);
    v = v + dpp_read<kDppRowShr2, 0xf, true>(v);
    v = v + dpp_read<kDppRowShr4, 0xf, true>(v);
    v = v + dpp_read<kDppRowShr8, 0xf, true>(v);
    v = v + dpp_read<kDppRowBcast15, 0xa, false>(v);
    v = v + dpp_read<kDppRowBcast31, 0xc, false>(v);
    return v;
}

// Value held by the previous lane; lane 0 gets 0 (+0.0 for fp32).
template <class T>
__device__ __forceinline__ T wave_shift_up1(T v)
{
    return Elem<T>::from((uint32_t)__builtin_amdgcn_update_dpp(
        0, (int)Elem<T>::bits(v), kDppWaveShr1, 0xf, 0xf, true));
}

template <class T>
__device__ __forceinline__ T wave_read_lane(T v, int lane)
{
    return Elem<T>::from((uint32_t)__builtin_amdgcn_readlane((int)Elem<T>::bits(v), lane));
}

template <class T>
__device__ __forceinline__ T wave_sum(T v)
{
    return wave_read_lane(wave_inclusive_scan(v), 63);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// ---------------------------------------------------------------------------
// Tile I/O through buffer resources. A tile is W wave segments; a wave segment
// is CHUNKS chunks of 64 * VEC consecutive elements, and lane l holds elements
// [l*VEC, l*VEC+VEC) of every chunk. Each load instruction of a wave therefore
// reads 64*VEC*4 contiguous bytes (1 KiB for dwordx4): fully coalesced, no LDS
// transpose.
//
// Each wave addresses its segment through a buffer resource that starts at the
// segment's first element (a uniform 64-bit base in SGPRs) with num_records =
// the segment's valid bytes. gfx950 range checks raw buffer accesses per dword:
// dwords past num_records load as 0 (the identity, which pads a ragged last
// tile) and are not stored. So full and ragged tiles share one path, and a lane
// needs a single 32-bit offset register.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Third descriptor dword for raw 32-bit buffer access on the gfx9 family.
constexpr int kBufferRsrcFlags = 0x00020000;
// Cache-policy bit of buffer instructions for a non-temporal (streaming) access.
constexpr int kBufferNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t valid_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)valid_bytes,
                                             kBufferRsrcFlags);
}

// Valid bytes of the `len` elements starting at element `first` of an array of
// n elements (first < n is not required: past the end gives 0).
__device__ __forceinline__ uint32_t valid_bytes(uint64_t first, uint32_t len, uint64_t n)
{
    const uint64_t left = first < n ? n - first : 0u;
    return (uint32_t)((left < len ? left : len) * 4u);
}

// Lane l of chunk c reads/writes the VEC elements at byte offset
// 4 * (64 VEC c + VEC l) of the wave segment: the lane part is the only
// per-lane offset; the chunk part is an immediate or scalar offset.
template <class T, int VEC, int CHUNKS, bool NT>
__device__ __forceinline__ void load_segment(__amdgpu_buffer_rsrc_t r, int lane, T (&x)[CHUNKS][VEC])
{
    static_assert(VEC == 1 || VEC == 4, "dword or dwordx4 accesses");
    constexpr int aux = NT ? kBufferNonTemporal : 0;
    const int voff = lane * VEC * 4;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        if constexpr (VEC == 4) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, c * 64 * VEC * 4, aux);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[c][e] = Elem<T>::from(v[e]);
        } else {
            x[c][0] = Elem<T>::from(__builtin_amdgcn_raw_buffer_load_b32(r, voff, c * 64 * VEC * 4, aux));
        }
    }
}

template <class T, int VEC, int CHUNKS, bool NT>
__device__ __forceinline__ void store_segment(__amdgpu_buffer_rsrc_t r, int lane, const T (&y)[CHUNKS][VEC])
{
    constexpr int aux = NT ? kBufferNonTemporal : 0;
    const int voff = lane * VEC * 4;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        if constexpr (VEC == 4) {
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = Elem<T>::bits(y[c][e]);
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, c * 64 * VEC * 4, aux);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(Elem<T>::bits(y[c][0]), r, voff, c * 64 * VEC * 4, aux);
        }
    }
}

// ---------------------------------------------------------------------------
// Scan of one wave segment held in registers, in place (three-phase coarsened
// scan of the PMPP 11.2 notes, with wave scans in place of the block-wide
// phase 2). For each chunk c, each lane
//   1. replaces its VEC elements by their in-lane prefix sums (exclusive or
//      inclusive) and keeps the lane total;
//   2. gets the sum of the lower lanes' totals (wave64 DPP scan) and the sum
//      of the wave's earlier chunks (uniform), and adds both to its elements.
// Afterwards every element holds its prefix inside the wave segment; the
// segment total is returned (uniform). Nothing but the tile stays live for the
// look-back, and the finish is one uniform add per element. Exclusive values
// are formed directly, never as inclusive - x.
// ---------------------------------------------------------------------------
template <class T, bool EXCL, int VEC, int CHUNKS>
__device__ __forceinline__ T scan_segment_local(T (&x)[CHUNKS][VEC])
{
    T running = T(0);   // sum of the wave's chunks before c
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        T lane_total = T(0);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const T xe = x[c][e];
            if constexpr (EXCL) {
                x[c][e] = lane_total;
                lane_total = lane_total + xe;
            } else {
                lane_total = lane_total + xe;
                x[c][e] = lane_total;
            }
        }
        const T incl = wave_inclusive_scan(lane_total);
        const T offset = running + wave_shift_up1(incl);
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[c][e] = offset + x[c][e];
        running = running + wave_read_lane(incl, 63);
    }
    return running;
}

// Keep every element materialised in a VGPR here. Without it the compiler
// sinks the segment-offset adds past the look-back to their single use and
// keeps the offsets alive (spilling them) across it. Emits no instruction.
template <class T, int VEC, int CHUNKS>
__device__ __forceinline__ void pin_in_registers(T (&x)[CHUNKS][VEC])
{
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(x[c][e]));
}

// Add the segment's seed (everything before the wave segment) to every element.
template <class T, int VEC, int CHUNKS>
__device__ __forceinline__ void add_seed(T (&x)[CHUNKS][VEC], T seed)
{
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[c][e] = seed + x[c][e];
}

// ---------------------------------------------------------------------------
// Tile descriptors (Merrill & Garland, sections 4.1 and 4.4): one 64-bit word
// per tile holding the status flag and a single value field, written and read
// as one device-scope atomic, so status and value are always seen together.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t desc_pack(uint32_t epoch, uint32_t status, uint32_t value_bits)
{
    return ((uint64_t)((epoch << kDescStatusBits) | status) << 32) | value_bits;
}

// Status of a descriptor word for the current epoch; words written by an
// earlier call (another epoch) or never written read as X.
__device__ __forceinline__ uint32_t desc_status(uint64_t d, uint32_t epoch)
{
    const uint32_t hi = (uint32_t)(d >> 32);
    return ((hi >> kDescStatusBits) == epoch) ? (hi & kDescStatusMask) : kStatusX;
}

// Address of tile t's descriptor (its first word) in the descriptor array.
__device__ __forceinline__ uint64_t* desc_at(uint64_t* desc, uint64_t t) { return desc + t * kDescStride; }
__device__ __forceinline__ const uint64_t* desc_at(const uint64_t* desc, uint64_t t)
{
    return desc + t * kDescStride;
}

// Pause before re-polling a blocked look-back window. The first re-poll comes
// at once (`first`); after that, level kPauseShort keeps a short pause and
// kPause64 sleeps 64 x 64 clocks: fewer polls while many tiles wait leave the
// memory system to the loads of the tiles being waited on.
__device__ __forceinline__ void lookback_pause(uint32_t level, bool first)
{
    if (first || level == kPauseShort)
        __builtin_amdgcn_s_sleep(1);
    else
        __builtin_amdgcn_s_sleep(64);
}

template <int ORDER>
__device__ __forceinline__ uint64_t desc_load(const uint64_t* p)
{
    if constexpr (ORDER == kOrderAcqRel)
        return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    else
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int ORDER>
__device__ __forceinline__ void desc_store(uint64_t* p, uint64_t w)
{
    if constexpr (ORDER == kOrderAcqRel)
        __hip_atomic_store(p, w, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    else
        __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t realtime() { return __builtin_amdgcn_s_memrealtime(); }

// The launch's descriptor epoch lives in a device word of the workspace, so a
// launch replayed from a captured graph still gets a new one. A workgroup may
// read it any time before it publishes: the word only advances after the last
// tile has published P, and that needs every tile's A or P, so no workgroup
// of the launch can read it late.
__device__ __forceinline__ uint32_t load_epoch(const unsigned int* word)
{
    return uniform(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// The same read, left in a VGPR: take uniform() of it where it is used, so
// the read stays in flight with whatever is issued after it (the tile draw,
// or the tile's own loads) instead of costing a round trip of its own first.
__device__ __forceinline__ uint32_t load_epoch_async(const unsigned int* word)
{
    return __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called once per launch, by the owner of the last tile after its P: the next
// launch on the workspace gets the next epoch (1 again after kEpochMax; the
// host clears the descriptors before that can matter).
__device__ __forceinline__ void advance_epoch(unsigned int* word, uint32_t epoch)
{
    __hip_atomic_store(word, epoch >= kEpochMax ? 1u : epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Draw the next tile index from the workspace counter with one device-scope
// atomic (dynamic tile index assignment, PMPP 11.3 notes; "virtual processors"
// in section 4.4 of the Merrill & Garland notes): the holder of tile t knows
// tiles 0..t-1 were drawn by workgroups that are already running, so waiting
// on them cannot deadlock. The draw of the last tile puts the counter back to
// 0 for the next call on the same workspace (every other draw of the call has
// happened by then). Call from one lane.
__device__ __forceinline__ uint32_t draw_tile(unsigned long long* counter, uint32_t num_draws)
{
    const uint32_t tile =
        (uint32_t)__hip_atomic_fetch_add(counter, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tile == num_draws - 1u)
        __hip_atomic_store(counter, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return tile;
}

// Decoupled look-back by one whole wavefront (section 4.4, parallelized
// look-back), widened to K slots per lane: slot j of lane l inspects the
// descriptor of tile hi - (64 j + l), so one poll covers 64 K predecessors with
// K independent loads per lane in flight at once. The nearest P is the lowest
// lane of the lowest slot that holds one. If any descriptor from tile - 1 back
// to that P (or back through the whole window when there is none) is still X,
// the window is polled again. With RELOAD_ALL false the poll reloads only
// those X descriptors (the others keep what they read: an A stays a valid
// aggregate, a P a valid prefix); that measured 1.2 to 1.7% faster for the
// compaction on the 2^30 - 12,345 flags and the workgroup-index scan of 2^26
// elements, and 0.9% slower for the drawn-index scan of 2^28, which reloads
// the whole window. Otherwise those descriptors' values are summed
// into the running exclusive prefix (aggregates of the A tiles plus the
// inclusive prefix of the nearest P); with a P the look-back ends, without one
// the window slides back by 64 K. Indices below 0 read as P with value 0, so
// the walk ends at tile 0 at the latest. Returns the exclusive prefix of
// `tile` (uniform). A wait longer than kWatchdogTicks counts one trip in
// *watchdog and returns the incomplete prefix instead of hanging. Call with the
// whole wave active.
//
// The width: a tile publishes P only after its own look-back, so if one poll
// of latency L covers W = 64 K predecessors, P can advance by at most W tiles
// per L; W must keep W / L above the rate at which tiles arrive.
//
// Back-off: a blocked window is polled again at once, then after the pause
// of level `backoff` (lookback_pause) before every further poll.
template <class T, int ORDER, int K, bool RELOAD_ALL = false>
__device__ T lookback_decoupled(const uint64_t* desc, uint32_t tile, uint32_t epoch,
                               unsigned int* watchdog, uint32_t backoff = 0u)
{
    const int lane = lane_id();
    const uint64_t lane_bit = 1ull << lane;
    T prefix = T(0);
    int64_t hi = (int64_t)tile - 1;
    const uint64_t t0 = realtime();
    bool repolled = false;
    uint64_t d[K];
    // lanes of each slot that the next poll loads: all of a new window; after
    // a blocked poll only the descriptors still awaited (the rest keep what
    // they read: an A stays a valid aggregate, a P a valid prefix)
    uint64_t reload[K];
#pragma unroll
    for (int j = 0; j < K; ++j) reload[j] = ~0ull;
    for (;;) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int64_t idx = hi - (int64_t)(j * 64 + lane);
            if (reload[j] & lane_bit)
                d[j] = (idx >= 0) ? desc_load<ORDER>(desc_at(desc, (uint64_t)idx)) : desc_pack(epoch, kStatusP, 0u);
        }
        uint64_t has_p[K], has_x[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const uint32_t st = desc_status(d[j], epoch);
            has_p[j] = __builtin_amdgcn_ballot_w64(st == kStatusP);
            has_x[j] = __builtin_amdgcn_ballot_w64(st == kStatusX);
        }
        // slot of the nearest P (K if none) and the lanes needed in it
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
            T v = T(0);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const uint64_t need = (j < jp) ? ~0ull : ((j == jp) ? need_p : 0ull);
                if (need & lane_bit) v = v + Elem<T>::from((uint32_t)d[j]);
            }
            prefix = prefix + wave_sum(v);
            if (jp < K) return prefix;
            hi -= 64 * K;
#pragma unroll
            for (int j = 0; j < K; ++j) reload[j] = ~0ull;
            continue;
        }
        if constexpr (!RELOAD_ALL) {
#pragma unroll
            for (int j = 0; j < K; ++j) reload[j] = j < jp ? has_x[j] : (j == jp ? has_x[j] & need_p : 0ull);
        }
        if (realtime() - t0 > kWatchdogTicks) {
            if (lane == 0) atomicAdd(watchdog, 1u);
            return prefix;
        }
        lookback_pause(backoff, !repolled);
        repolled = true;
    }
}

// Chained scan (section 3.2, Fig 4): wait for the immediate predecessor's
// inclusive prefix only. Lane 0 polls; the result is broadcast to the wave.
template <class T, int ORDER>
__device__ T lookback_chained(const uint64_t* desc, uint32_t tile, uint32_t epoch,
                             unsigned int* watchdog)
{
    uint32_t bits = 0u;
    if (lane_id() == 0) {
        const uint64_t t0 = realtime();
        for (;;) {
            const uint64_t d = desc_load<ORDER>(desc_at(desc, tile - 1u));
            if (desc_status(d, epoch) == kStatusP) {
                bits = (uint32_t)d;
                break;
            }
            if (realtime() - t0 > kWatchdogTicks) {
                atomicAdd(watchdog, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    return Elem<T>::from((uint32_t)__builtin_amdgcn_readfirstlane((int)bits));
}

}  // namespace dws

// Reduce-by-key and run-length encoding fused with the single-pass decoupled
// look-back (Merrill & Garland, section 4.4 compaction behaviour; section A5,
// reduce-by-key and run-length-encode).
//
// Per element i: head(i) = (i == 0 or key[i] != key[i-1]). A run ends where
// the next one starts, so the head at p stores its key to unique_keys[run]
// and also finishes the run before it in aggregates[run - 1]; only the array's
// last run has no head after it and is stored from its segment's aggregate.
// The look-back carries the pair (heads, value since the last head) under
// "count the heads, restart the value sum after the last head" (a segmented
// sum, not commutative); the last tile stores the number of runs. Values are
// 32-bit integers (sums wrap modulo 2^32) or fp32 (k_run_ends), or the
// constant 1 (k_rle: the sum is the run length).
//
// The neighbour key[i-1] comes from the same lane, the adjacent lane (DPP
// wave shift), the previous chunk (readlane) or, at a wave segment's start,
// one extra 4-byte load. The heads of one chunk of a wave (64 x VEC elements)
// hold consecutive runs, so their outputs are two contiguous ranges: each
// head writes into a per-wave LDS stage at its rank among the chunk's heads,
// and the wave then stores the ranges with lane-contiguous dword stores, one
// instruction per 64 heads and array. Storing from the elements' own lanes
// instead (lanes 16 bytes apart, one instruction per element and array,
// mostly dropped) measured 1.35 to 1.55x slower with all keys distinct at
// 2^25 and 3 to 7% slower at mean run 16.
#include "dws_op_kernel.hpp"

namespace dws {

// (heads so far, running value since the last head); q restarts the value
// when it holds a head.
template <bool FLOAT>
struct OpRunSum {
    static constexpr int kWords = 2;
    using V = Val<2>;
    static __device__ __forceinline__ V identity() { return {{0u, 0u}}; }
    static __device__ __forceinline__ V combine(V p, V q)
    {
        uint32_t sum;
        if constexpr (FLOAT) sum = f2u(u2f(p.w[1]) + u2f(q.w[1]));
        else sum = p.w[1] + q.w[1];
        return {{p.w[0] + q.w[0], q.w[0] != 0u ? q.w[1] : sum}};
    }
};

struct RbkParams {
    const uint32_t* keys;
    const uint32_t* vals;     // unused for run-length encoding
    uint32_t* ukeys;
    uint32_t* aggs;           // sums, or run lengths
    uint64_t n;
    uint64_t* desc;
    unsigned int* watchdog;
    unsigned long long* num_runs;
    uint32_t num_tiles;
    unsigned int* epoch;
    uint32_t backoff;         // pause level between blocked look-back polls (kPause*)
};

// Look-back slots per lane for the run kernels, with every slot's loads issued
// before any is examined (one round trip per poll): two, 128 predecessors per
// poll, for run-length encoding and integer sums. Against one slot, alternating
// builds at 2^25 keys (three runs each): run-length encoding 1.5% faster at mean
// run 16 and 0.9% with all keys distinct, integer sums 0.8 to 1% faster. The
// fp32 sums kernel measured 1.4% slower with two slots with all keys distinct
// (equal at mean run 16) and keeps one. Four slots spill registers.
constexpr int kRunLookbackSlots = 2;
constexpr int kRunF32LookbackSlots = 1;

// A wave segment of the large shapes (2,048 elements or more) with at most
// this many heads stages all of them in LDS right after publishing its
// aggregate, while wave 0 waits in the look-back (wave 0 itself after it), so
// that only the stores are left once the prefix is known. Segments with more
// heads, and the small shapes, stage chunk by chunk after the look-back. With
// 1,024 (8 KiB per wave) it measured 11% faster at mean run 16 for run-length
// encoding (2^22, 2^25 and 2^28 keys) and equal with all keys distinct or at
// mean run 3 (which take the chunk path); 512 measured the same at mean run
// 16.
constexpr uint32_t kRunPreHeads = 1024u;

// Inclusive fp32 + scan over the 64 lanes in lane order, restarted at the
// lanes set in `starts`: lane l sums lanes s..l, where s is the highest lane
// <= l in starts (lane 0 when there is none). It is the plain scan's row-shift
// and row-broadcast doubling with each step taken only when its source lane
// is not before s; a step not taken adds -0.0, the exact identity.
__device__ __forceinline__ float wave_segmented_scan_f32(float v, uint64_t starts, int lane)
{
    const uint64_t upto = starts & (lane == 63 ? ~0ull : ((2ull << lane) - 1ull));
    const int dist = upto != 0ull ? lane - (63 - __builtin_clzll(upto)) : lane;
    const int pos = lane & 15;
    float t;
    t = dpp_read<kDppRowShr1, 0xf, true>(v);
    v = v + (dist >= 1 ? t : -0.0f);
    t = dpp_read<kDppRowShr2, 0xf, true>(v);
    v = v + (dist >= 2 ? t : -0.0f);
    t = dpp_read<kDppRowShr4, 0xf, true>(v);
    v = v + (dist >= 4 ? t : -0.0f);
    t = dpp_read<kDppRowShr8, 0xf, true>(v);
    v = v + (dist >= 8 ? t : -0.0f);
    t = dpp_read<kDppRowBcast15, 0xa, false>(v);   // rows 1 and 3 take lane 15 of the row before
    v = v + (dist > pos ? t : -0.0f);
    t = dpp_read<kDppRowBcast31, 0xc, false>(v);   // rows 2 and 3 take lane 31
    v = v + (dist >= lane - 31 ? t : -0.0f);
    return v;
}

// Inside a wave segment no (heads, value) pairs are scanned. Heads are
// counted with ballots before the look-back; after it, chunk by chunk, each
// head stages its key and a value in LDS at its rank among the chunk's heads
// (mbcnt over the ballots), and one lane per head stores the key and the run
// it finishes:
//   integer sums: S(i), the segment's values before i (wrapping +), is formed
//     before the look-back; the run finished by the head at p sums to
//     S(p) - S(previous head), exact modulo 2^32, where the previous head is
//     the next lower lane's staged one, or the previous chunk's last, or, for
//     the segment's first head, at S = minus the value carried in;
//   fp32 sums: differences of long fp32 prefix sums would lose short runs'
//     precision, so each element instead holds its run's fp32 sum since the
//     last head: summed in the lane, then across the lanes by a segmented
//     wave scan restarted at lanes that hold a head, with the sum carried in
//     from earlier chunks. A head stages the sum of the element before it;
//     the segment's first head adds the value carried in.
// The segment's aggregate for the look-back is (heads, value from its last
// head on). Against the former kernel (per-lane run starts formed before the
// look-back with a ds_bpermute per chunk) this measured 2 to 3% faster at
// mean run 16 (2^25 and 2^28 keys) and equal with all keys distinct. The
// heads are found again after the look-back, and the last head's S by a
// search from the segment's end, rather than keeping ballot masks in scalar
// registers. At most 128 VGPRs (four waves per SIMD): two 512-thread
// workgroups share a CU, so one's loads overlap the other's look-back and
// stores. The tile index is the workgroup index (measured faster than a drawn
// index at 2^25 and 2^28 elements in every mode): it relies on the GPU
// starting each XCD's workgroups in index order, and the watchdog bounds
// every wait.
template <int BLOCK, int VEC, int CHUNKS, int MODE, bool NT = false>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) k_run_ends(RbkParams p)
{
    static_assert(MODE == 0 || MODE == 1, "integer or fp32 sums");
    using Op = OpRunSum<MODE == 1>;
    using V = Val<2>;
    constexpr int W = BLOCK / 64;
    constexpr uint32_t CH = 64u * VEC;
    constexpr uint32_t SEG = CH * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    __shared__ V s_wave[W];
    __shared__ V s_prefix;
    // per wave: keys, then values, of the segment's heads (or of one
    // chunk's) by rank, then one spare slot per lane that the other elements
    // write to
    constexpr uint32_t PRE = SEG < 2048u ? 0u : (SEG < kRunPreHeads ? SEG : kRunPreHeads);
    constexpr uint32_t SLOTS = PRE > CH ? PRE : CH;
    __shared__ uint32_t s_stage[W][2][SLOTS + 64];

    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const bool multi = p.num_tiles > 1u;
    const uint32_t tile = multi ? (uint32_t)blockIdx.x : 0u;
    const uint64_t seg_first = (uint64_t)tile * TILE + (uint64_t)wave * SEG;
    const uint32_t vb = valid_bytes(seg_first, SEG, p.n);
    const uint32_t seg_elems = vb / 4u;
    uint32_t k[CHUNKS][VEC];
    load_segment<uint32_t, VEC, CHUNKS, NT>(make_rsrc(p.keys + seg_first, vb), lane, k);
    uint32_t v[CHUNKS][VEC];
    load_segment<uint32_t, VEC, CHUNKS, NT>(make_rsrc(p.vals + seg_first, vb), lane, v);
    const uint32_t epoch_v = (multi && wave == 0) ? load_epoch_async(p.epoch) : 0u;
    const bool has_prev = seg_first > 0u && seg_first < p.n;
    const uint32_t prev_key = __builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(p.keys + (has_prev ? seg_first - 1u : 0u), has_prev ? 4u : 0u), 0, 0, 0);
    const bool holds_last = seg_elems > 0u && seg_first + seg_elems == p.n;
    uint32_t left0 = seg_first == 0u ? ~(uint32_t)__builtin_amdgcn_readlane((int)k[0][0], 0) : prev_key;
    if (seg_elems < SEG) {
        const uint32_t last_key = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.keys + (p.n - 1u), 4u), 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if ((uint32_t)(c * CH) + (uint32_t)(lane * VEC + e) >= seg_elems) k[c][e] = last_key;
        if (seg_elems == 0u) left0 = last_key;
    }

    uint32_t fprev[CHUNKS];
    uint32_t h_seg = 0u, s_seg = 0u;
    float f_carry = -0.0f;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const uint32_t from_left = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k[c][VEC - 1], kDppWaveShr1, 0xf,
                                                                         0xf, true);
        const uint32_t edge = c > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)k[c - 1][VEC - 1], 63) : left0;
        fprev[c] = lane > 0 ? from_left : edge;
        bool head[VEC];
        uint64_t any = 0ull;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            head[e] = k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c]);
            const uint64_t m = __builtin_amdgcn_ballot_w64(head[e]);
            any |= m;
            h_seg += (uint32_t)__builtin_popcountll(m);
        }
        if constexpr (MODE == 0) {
            uint32_t sx[VEC];
            uint32_t acc = 0u;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                sx[e] = acc;
                acc += v[c][e];
            }
            const uint32_t incl = wave_inclusive_scan(acc);
            const uint32_t base = s_seg + (incl - acc);
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[c][e] = sx[e] + base;
            s_seg += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        } else {
            float g[VEC];
            bool seen[VEC];
            float acc = -0.0f;
            bool any_head = false;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float x = u2f(v[c][e]);
                acc = head[e] ? x : acc + x;
                g[e] = acc;
                any_head = any_head || head[e];
                seen[e] = any_head;
            }
            const float lane_total = (lane == 0 && !any_head) ? f_carry + acc : acc;
            const float incl = wave_segmented_scan_f32(lane_total, any, lane);
            const float from_lower = wave_shift_up1(incl);
            const float into = lane == 0 ? f_carry : from_lower;
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[c][e] = f2u(seen[e] ? g[e] : into + g[e]);
            f_carry = u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(incl), 63));
        }
        asm volatile("" : "+v"(fprev[c]));
#pragma unroll
        for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(v[c][e]));
    }
    h_seg = uniform(h_seg);
    V seg_total;
    if constexpr (MODE == 1) {
        seg_total = {{h_seg, f2u(f_carry)}};
    } else {
        // S at the segment's last head, from the last chunk that has one
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(k[c][e]));
        uint32_t b_last = 0u;
        bool found = h_seg == 0u;
#pragma unroll
        for (int c = CHUNKS - 1; c >= 0; --c) {
            if (!found) {
                uint64_t m[VEC];
                uint64_t any = 0ull;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    m[e] = __builtin_amdgcn_ballot_w64(k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c]));
                    any |= m[e];
                }
                if (any != 0ull) {
                    const int top = 63 - __builtin_clzll(any);
                    bool got = false;
#pragma unroll
                    for (int e = VEC - 1; e >= 0; --e) {
                        if (!got && ((m[e] >> top) & 1ull)) {
                            b_last = (uint32_t)__builtin_amdgcn_readlane((int)v[c][e], top);
                            got = true;
                        }
                    }
                    found = true;
                }
            }
        }
        seg_total = {{h_seg, h_seg > 0u ? s_seg - uniform(b_last) : s_seg}};
    }

    if (lane == 0) s_wave[wave] = seg_total;
    __syncthreads();
    V wave_pre = Op::identity(), agg = Op::identity();
#pragma unroll
    for (int w = 0; w < W; ++w) {
        if (w == wave) wave_pre = agg;
        agg = Op::combine(agg, s_wave[w]);
    }
    if (wave == 0) {
        V prefix = Op::identity();
        if (multi) {
            const uint32_t epoch = uniform(epoch_v);
            if (tile == 0u) {
                if (lane == 0) desc_store_val<2>(p.desc, 0u, epoch, kStatusP, agg);
            } else {
                if (lane == 0) desc_store_val<2>(p.desc, tile, epoch, kStatusA, agg);
                constexpr int K = MODE == 1 ? kRunF32LookbackSlots : kRunLookbackSlots;
                prefix = lookback_op<Op, K>(p.desc, tile, epoch, p.watchdog, p.backoff);
                if (lane == 0) {
                    desc_store_val<2>(p.desc, tile, epoch, kStatusP, Op::combine(prefix, agg));
                    if (tile == p.num_tiles - 1u) advance_epoch(p.epoch, epoch);
                }
            }
        }
        if (lane == 0) s_prefix = prefix;
    }
    // a segment with few heads stages all of them now (key and value at the
    // head's rank in the segment)
    const bool pre = PRE > 0u && (SEG <= PRE || h_seg <= PRE);
    if (pre) {
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(k[c][e]));
        uint32_t base = 0u;   // heads of the segment before chunk c (uniform)
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            bool hd[VEC];
            uint64_t m[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                hd[e] = k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c]);
                m[e] = __builtin_amdgcn_ballot_w64(hd[e]);
            }
            uint32_t r = base;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[e], r));
            uint32_t g_first = 0u;
            if constexpr (MODE == 1) {
                const uint32_t g_left = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[c][VEC - 1], kDppWaveShr1,
                                                                              0xf, 0xf, true);
                const uint32_t g_edge =
                    c > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)v[c > 0 ? c - 1 : 0][VEC - 1], 63) : 0x80000000u;
                g_first = lane > 0 ? g_left : g_edge;
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t slot = hd[e] ? r : SLOTS + (uint32_t)lane;
                s_stage[wave][0][slot] = k[c][e];
                if constexpr (MODE == 0) s_stage[wave][1][slot] = v[c][e];
                else s_stage[wave][1][slot] = e > 0 ? v[c][e - 1] : g_first;
                r += hd[e] ? 1u : 0u;
            }
            base = uniform((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
        }
    }
    __syncthreads();
    const V tile_prefix = s_prefix;
    const V seed = Op::combine(tile_prefix, wave_pre);
    const uint32_t seed_heads = uniform(seed.w[0]);
    const uint32_t seed_value = uniform(seed.w[1]);
    const uint32_t heads_before = uniform(tile_prefix.w[0]);
    const uint32_t tile_heads = uniform(agg.w[0]);

    if (pre) {
        // head i of the segment is run seed_heads + i and finishes run
        // seed_heads + i - 1 (the array's first head finishes none)
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.ukeys + seed_heads, h_seg * 4u);
        const bool first_of_array = seed_heads == 0u;
        const uint32_t abase = uniform(first_of_array ? 0u : seed_heads - 1u);
        const uint32_t arange = uniform(first_of_array ? (h_seg > 0u ? h_seg * 4u - 4u : 0u) : h_seg * 4u);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.aggs + abase, arange);
        uint32_t before = 0u - seed_value;   // integer sums: S at the head before this group's first
        for (uint32_t g = 0u; g < h_seg; g += 64u) {
            const uint32_t i = g + (uint32_t)lane;
            const uint32_t key = s_stage[wave][0][i];
            const uint32_t val = s_stage[wave][1][i];
            uint32_t fin;
            if constexpr (MODE == 0) {
                const uint32_t left = wave_shift_up1(val);
                fin = val - (lane == 0 ? before : left);
                before = (uint32_t)__builtin_amdgcn_readlane((int)val, 63);
            } else {
                // the segment's first head finishes a run that started before
                // the segment: it adds the value carried in
                fin = i == 0u ? f2u(u2f(seed_value) + u2f(val)) : val;
            }
            __builtin_amdgcn_raw_buffer_store_b32(key, rk, (int)(i * 4u), 0, 0);
            if (!first_of_array || i > 0u)
                __builtin_amdgcn_raw_buffer_store_b32(fin, ra, (int)((first_of_array ? i - 1u : i) * 4u), 0, 0);
        }
    } else {
        // the chunk path
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(k[c][e]));
        uint32_t run0 = seed_heads;
        uint32_t before = 0u - seed_value;   // integer sums: S at the head before the chunk's first head
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            bool hd[VEC];
            uint64_t m[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                hd[e] = k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c]);
                m[e] = __builtin_amdgcn_ballot_w64(hd[e]);
            }
            // rank among the chunk's heads (as in k_rle: every element writes,
            // the others to their lane's spare slot)
            uint32_t r = 0u;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[e], r));
            uint32_t g_first = 0u;
            if constexpr (MODE == 1) {
                const uint32_t g_left = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[c][VEC - 1], kDppWaveShr1, 0xf,
                                                                              0xf, true);
                const uint32_t g_edge =
                    c > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)v[c > 0 ? c - 1 : 0][VEC - 1], 63) : 0x80000000u;
                g_first = lane > 0 ? g_left : g_edge;
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t slot = hd[e] ? r : CH + (uint32_t)lane;
                s_stage[wave][0][slot] = k[c][e];
                if constexpr (MODE == 0) s_stage[wave][1][slot] = v[c][e];
                else s_stage[wave][1][slot] = e > 0 ? v[c][e - 1] : g_first;
                r += hd[e] ? 1u : 0u;
            }
            const uint32_t cnt = uniform((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
            __builtin_amdgcn_wave_barrier();
            if (cnt > 0u) {
                const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.ukeys + run0, cnt * 4u);
                const bool first_of_array = run0 == 0u;
                const bool first_of_seg = run0 == seed_heads;
                const uint32_t abase = uniform(first_of_array ? 0u : run0 - 1u);
                const uint32_t arange = uniform(first_of_array ? cnt * 4u - 4u : cnt * 4u);
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.aggs + abase, arange);
#pragma unroll
                for (int q = 0; q < VEC; ++q) {
                    if (cnt > (uint32_t)(64 * q)) {
                        const uint32_t i = (uint32_t)(64 * q + lane);
                        const uint32_t key = s_stage[wave][0][i];
                        const uint32_t val = s_stage[wave][1][i];
                        uint32_t fin;
                        if constexpr (MODE == 0) {
                            const uint32_t left = wave_shift_up1(val);
                            fin = val - (lane == 0 ? before : left);
                            const uint32_t in_group = cnt - (uint32_t)(64 * q);
                            before = (uint32_t)__builtin_amdgcn_readlane((int)val,
                                                                         in_group >= 64u ? 63 : (int)in_group - 1);
                        } else {
                            // the segment's first head finishes a run that started
                            // before the segment: it adds the value carried in
                            fin = (first_of_seg && i == 0u) ? f2u(u2f(seed_value) + u2f(val)) : val;
                        }
                        __builtin_amdgcn_raw_buffer_store_b32(key, rk, (int)(i * 4u), 0, 0);
                        if (!first_of_array || i > 0u)
                            __builtin_amdgcn_raw_buffer_store_b32(fin, ra, (int)((first_of_array ? i - 1u : i) * 4u), 0,
                                                                  0);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            run0 += cnt;
        }
    }
    if (holds_last && lane == 0) {
        const uint32_t base_run = heads_before > 0u ? heads_before - 1u : 0u;
        const __amdgpu_buffer_rsrc_t raggs = make_rsrc(p.aggs + base_run, (tile_heads + 1u) * 4u);
        const uint32_t last_off = (seed_heads + h_seg - 1u - base_run) * 4u;
        __builtin_amdgcn_raw_buffer_store_b32(Op::combine(seed, seg_total).w[1], raggs, (int)last_off, 0, 0);
    }
    if (tile == p.num_tiles - 1u && threadIdx.x == 0) *p.num_runs = (unsigned long long)heads_before + tile_heads;
}

// Run-length encoding (the value of every element is 1, so a run's value is
// its length). The run a head finishes has the length pos(head) - pos(head
// before), and no per-element prefix is needed:
//   first pass (before the look-back): the segment's head count and its last
//     head, whose distance to the segment's end is the value carried on;
//   second pass (after it), chunk by chunk: each head's rank among the
//     chunk's heads (mbcnt over the ballots), its key and its position staged
//     in LDS at that rank, then one lane per head reads them back and stores
//     its key and the length of the run it finishes (its position minus the
//     next lower lane's, or minus the previous chunk's last head).
// The first head of a segment finishes a run that started seed value
// elements before the segment (the value carried in). Against the former
// shared kernel with the constant 1 as the value (per-element positions, run
// starts and ranks formed before the look-back, a ds_bpermute per chunk: 1,653
// VALU instructions per wave) this has 761, and measured 10 to 16% faster at
// mean run 16 (2^25 and 2^28 keys) and 1 to 2% with all keys distinct. The
// heads are found again after the look-back instead of keeping 64 ballot
// masks per wave in scalar registers.
template <int BLOCK, int VEC, int CHUNKS, bool NT = false>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) k_rle(RbkParams p)
{
    using Op = OpRunSum<false>;
    using V = Val<2>;
    constexpr int W = BLOCK / 64;
    constexpr uint32_t CH = 64u * VEC;
    constexpr uint32_t SEG = CH * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    __shared__ V s_wave[W];
    __shared__ V s_prefix;
    // per wave: keys, then positions, of the segment's heads (or of one
    // chunk's) by rank, then one spare slot per lane that the other elements
    // write to
    constexpr uint32_t PRE = SEG < 2048u ? 0u : (SEG < kRunPreHeads ? SEG : kRunPreHeads);
    constexpr uint32_t SLOTS = PRE > CH ? PRE : CH;
    __shared__ uint32_t s_stage[W][2][SLOTS + 64];

    const int lane = lane_id();
    const int wave = (int)uniform(threadIdx.x >> 6);
    const bool multi = p.num_tiles > 1u;
    const uint32_t tile = multi ? (uint32_t)blockIdx.x : 0u;
    const uint64_t seg_first = (uint64_t)tile * TILE + (uint64_t)wave * SEG;
    const uint32_t vb = valid_bytes(seg_first, SEG, p.n);
    const uint32_t seg_elems = vb / 4u;
    uint32_t k[CHUNKS][VEC];
    load_segment<uint32_t, VEC, CHUNKS, NT>(make_rsrc(p.keys + seg_first, vb), lane, k);
    const uint32_t epoch_v = (multi && wave == 0) ? load_epoch_async(p.epoch) : 0u;
    const bool has_prev = seg_first > 0u && seg_first < p.n;
    const uint32_t prev_key = __builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(p.keys + (has_prev ? seg_first - 1u : 0u), has_prev ? 4u : 0u), 0, 0, 0);
    const bool holds_last = seg_elems > 0u && seg_first + seg_elems == p.n;
    // the key compared with the segment's first element: the array's first
    // element is always a head
    uint32_t left0 = seg_first == 0u ? ~(uint32_t)__builtin_amdgcn_readlane((int)k[0][0], 0) : prev_key;
    if (seg_elems < SEG) {
        // elements past n take the key at n - 1, so they are never heads
        const uint32_t last_key = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.keys + (p.n - 1u), 4u), 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if ((uint32_t)(c * CH) + (uint32_t)(lane * VEC + e) >= seg_elems) k[c][e] = last_key;
        if (seg_elems == 0u) left0 = last_key;
    }

    // first pass: the key before each lane's first element of every chunk
    // (kept for the second pass) and the segment's head count
    uint32_t fprev[CHUNKS];
    uint32_t h_seg = 0u;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const uint32_t from_left = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k[c][VEC - 1], kDppWaveShr1, 0xf,
                                                                         0xf, true);
        const uint32_t edge = c > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)k[c - 1][VEC - 1], 63) : left0;
        fprev[c] = lane > 0 ? from_left : edge;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            h_seg += (uint32_t)__builtin_popcountll(
                __builtin_amdgcn_ballot_w64(k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c])));
        asm volatile("" : "+v"(fprev[c]));
    }
    h_seg = uniform(h_seg);
    // the segment's last head: in the last chunk that has one, searched from
    // the end (at mean runs above a few elements, the last chunk). Its
    // compares are made again (the opaque copies below) rather than keeping
    // the first pass's masks in scalar registers.
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(k[c][e]));
    uint32_t last_pos = 0u;
    bool found = h_seg == 0u;
#pragma unroll
    for (int c = CHUNKS - 1; c >= 0; --c) {
        if (!found) {
            uint64_t m[VEC];
            uint64_t any = 0ull;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                m[e] = __builtin_amdgcn_ballot_w64(k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c]));
                any |= m[e];
            }
            if (any != 0ull) {
                const int top = 63 - __builtin_clzll(any);
                uint32_t em = 0u;
                bool got = false;
#pragma unroll
                for (int e = VEC - 1; e > 0; --e) {
                    if (!got && ((m[e] >> top) & 1ull)) {
                        em = (uint32_t)e;
                        got = true;
                    }
                }
                last_pos = (uint32_t)(c * CH) + (uint32_t)top * VEC + em;
                found = true;
            }
        }
    }
    const V seg_total = {{h_seg, h_seg > 0u ? seg_elems - uniform(last_pos) : seg_elems}};

    if (lane == 0) s_wave[wave] = seg_total;
    __syncthreads();
    V wave_pre = Op::identity(), agg = Op::identity();
#pragma unroll
    for (int w = 0; w < W; ++w) {
        if (w == wave) wave_pre = agg;
        agg = Op::combine(agg, s_wave[w]);
    }
    if (wave == 0) {
        V prefix = Op::identity();
        if (multi) {
            const uint32_t epoch = uniform(epoch_v);
            if (tile == 0u) {
                if (lane == 0) desc_store_val<2>(p.desc, 0u, epoch, kStatusP, agg);
            } else {
                if (lane == 0) desc_store_val<2>(p.desc, tile, epoch, kStatusA, agg);
                prefix = lookback_op<Op, kRunLookbackSlots>(p.desc, tile, epoch, p.watchdog, p.backoff);
                if (lane == 0) {
                    desc_store_val<2>(p.desc, tile, epoch, kStatusP, Op::combine(prefix, agg));
                    if (tile == p.num_tiles - 1u) advance_epoch(p.epoch, epoch);
                }
            }
        }
        if (lane == 0) s_prefix = prefix;
    }
    // a segment with few heads stages all of them now (key and position at
    // the head's rank in the segment)
    const bool pre = PRE > 0u && (SEG <= PRE || h_seg <= PRE);
    uint32_t pos_lane = (uint32_t)lane * VEC;
    asm volatile("" : "+v"(pos_lane));   // formed here, not held through the look-back
    if (pre) {
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(k[c][e]));
        uint32_t base = 0u;   // heads of the segment before chunk c (uniform)
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            bool hd[VEC];
            uint64_t m[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                hd[e] = k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c]);
                m[e] = __builtin_amdgcn_ballot_w64(hd[e]);
            }
            uint32_t r = base;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[e], r));
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t slot = hd[e] ? r : SLOTS + (uint32_t)lane;
                s_stage[wave][0][slot] = k[c][e];
                s_stage[wave][1][slot] = (uint32_t)(c * CH + e) + pos_lane;
                r += hd[e] ? 1u : 0u;
            }
            base = uniform((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
        }
    }
    __syncthreads();
    const V tile_prefix = s_prefix;
    const V seed = Op::combine(tile_prefix, wave_pre);
    const uint32_t seed_heads = uniform(seed.w[0]);
    const uint32_t seed_value = uniform(seed.w[1]);
    const uint32_t heads_before = uniform(tile_prefix.w[0]);
    const uint32_t tile_heads = uniform(agg.w[0]);

    if (pre) {
        // head i of the segment is run seed_heads + i: its key goes to
        // unique_keys[seed_heads + i], and it finishes run seed_heads + i - 1
        // (the array's first head finishes none, so its lane stores no length)
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.ukeys + seed_heads, h_seg * 4u);
        const bool first_of_array = seed_heads == 0u;
        const uint32_t abase = uniform(first_of_array ? 0u : seed_heads - 1u);
        const uint32_t arange = uniform(first_of_array ? (h_seg > 0u ? h_seg * 4u - 4u : 0u) : h_seg * 4u);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.aggs + abase, arange);
        uint32_t before = 0u - seed_value;   // position of the head before this group's first
        for (uint32_t g = 0u; g < h_seg; g += 64u) {
            const uint32_t i = g + (uint32_t)lane;
            const uint32_t key = s_stage[wave][0][i];
            const uint32_t pos = s_stage[wave][1][i];
            const uint32_t left = wave_shift_up1(pos);
            const uint32_t len = pos - (lane == 0 ? before : left);
            __builtin_amdgcn_raw_buffer_store_b32(key, rk, (int)(i * 4u), 0, 0);
            if (!first_of_array || i > 0u)
                __builtin_amdgcn_raw_buffer_store_b32(len, ra, (int)((first_of_array ? i - 1u : i) * 4u), 0, 0);
            before = (uint32_t)__builtin_amdgcn_readlane((int)pos, 63);
        }
    } else {
        // the chunk path
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(k[c][e]));
        uint32_t run0 = seed_heads;          // run of the chunk's first head (uniform)
        uint32_t before = 0u - seed_value;   // position of the head before the chunk's first head
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            bool hd[VEC];
            uint64_t m[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                hd[e] = k[c][e] != (e > 0 ? k[c][e - 1] : fprev[c]);
                m[e] = __builtin_amdgcn_ballot_w64(hd[e]);
            }
            // rank among the chunk's heads: heads in lower lanes, then the lane's
            // own; every element writes, the others to their lane's spare slot
            // (one write per element without a branch measured 2 to 3% faster at
            // mean run 16 than writing the heads alone under an execution mask)
            uint32_t r = 0u;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[e], r));
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const uint32_t slot = hd[e] ? r : CH + (uint32_t)lane;
                s_stage[wave][0][slot] = k[c][e];
                s_stage[wave][1][slot] = pos_lane + (uint32_t)e;
                r += hd[e] ? 1u : 0u;
            }
            // the chunk's head count: lane 63's rank after its own heads
            const uint32_t cnt = uniform((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
            // the wave's LDS accesses run in order: the reads below see every
            // lane's writes above (and the next chunk's writes follow the reads)
            __builtin_amdgcn_wave_barrier();
            if (cnt > 0u) {
                // head q of the chunk is run run0 + q: its key goes to
                // unique_keys[run0 + q], and it finishes run run0 + q - 1 (the
                // array's first head finishes none, so its lane stores no length)
                const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.ukeys + run0, cnt * 4u);
                const bool first_of_array = run0 == 0u;
                const uint32_t abase = uniform(first_of_array ? 0u : run0 - 1u);
                const uint32_t arange = uniform(first_of_array ? cnt * 4u - 4u : cnt * 4u);
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.aggs + abase, arange);
#pragma unroll
                for (int q = 0; q < VEC; ++q) {
                    if (cnt > (uint32_t)(64 * q)) {
                        const uint32_t i = (uint32_t)(64 * q + lane);
                        const uint32_t key = s_stage[wave][0][i];
                        const uint32_t pos = s_stage[wave][1][i] + (uint32_t)(c * CH);
                        const uint32_t left = wave_shift_up1(pos);
                        const uint32_t len = pos - (lane == 0 ? before : left);
                        __builtin_amdgcn_raw_buffer_store_b32(key, rk, (int)(i * 4u), 0, 0);
                        if (!first_of_array || i > 0u)
                            __builtin_amdgcn_raw_buffer_store_b32(len, ra, (int)((first_of_array ? i - 1u : i) * 4u), 0,
                                                                  0);
                        // the last head of this group of 64 is the next group's
                        // (or the next chunk's) head before
                        const uint32_t in_group = cnt - (uint32_t)(64 * q);
                        before = (uint32_t)__builtin_amdgcn_readlane((int)pos,
                                                                     in_group >= 64u ? 63 : (int)in_group - 1);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            run0 += cnt;
        }
    }
    if (holds_last && lane == 0) {
        // the array's last run has no head after it: its length is the value
        // carried to the end of the array
        const uint32_t base_run = heads_before > 0u ? heads_before - 1u : 0u;
        const __amdgpu_buffer_rsrc_t raggs = make_rsrc(p.aggs + base_run, (tile_heads + 1u) * 4u);
        const uint32_t last_off = (seed_heads + h_seg - 1u - base_run) * 4u;
        __builtin_amdgcn_raw_buffer_store_b32(Op::combine(seed, seg_total).w[1], raggs, (int)last_off, 0, 0);
    }
    if (tile == p.num_tiles - 1u && threadIdx.x == 0) *p.num_runs = (unsigned long long)heads_before + tile_heads;
}

__global__ void __launch_bounds__(64) k_store_runs(unsigned long long* count)
{
    if (threadIdx.x == 0) *count = 0ull;
}

template <int BLOCK, int VEC, int CHUNKS, int MODE, bool NT = false>
static hipError_t launch_rbk_mode(const RbkParams& p, hipStream_t stream)
{
    RbkParams arg = p;
    void* args[] = {&arg};
    const void* fn;
    if constexpr (MODE == 2) fn = reinterpret_cast<const void*>(&k_rle<BLOCK, VEC, CHUNKS, NT>);
    else fn = reinterpret_cast<const void*>(&k_run_ends<BLOCK, VEC, CHUNKS, MODE, NT>);
    return hipLaunchKernel(fn, dim3(p.num_tiles), dim3(BLOCK), args, 0, stream);
}

template <int BLOCK, int VEC, int CHUNKS>
static hipError_t launch_rbk_shape(int mode, const RbkParams& p, hipStream_t stream)
{
    switch (mode) {
    case 0: return launch_rbk_mode<BLOCK, VEC, CHUNKS, 0>(p, stream);
    case 1: return launch_rbk_mode<BLOCK, VEC, CHUNKS, 1>(p, stream);
    case 2: return launch_rbk_mode<BLOCK, VEC, CHUNKS, 2>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

uint32_t rbk_tile_elems(uint64_t n, bool aligned, int mode)
{
    if (!aligned) return 256u * 16u;
    if (n < kRbkLargeMin) return 256u * 4u * 4u;
    return mode == 2 ? 512u * 4u * 16u : 512u * 4u * 8u;
}

hipError_t launch_rbk(const RbkArgs& a, hipStream_t stream)
{
    if (a.n == 0) {
        unsigned long long* c = a.num_runs;
        void* args[] = {&c};
        return hipLaunchKernel(reinterpret_cast<const void*>(&k_store_runs), dim3(1), dim3(64), args, 0, stream);
    }
    RbkParams p{static_cast<const uint32_t*>(a.keys), static_cast<const uint32_t*>(a.vals),
                static_cast<uint32_t*>(a.ukeys),      static_cast<uint32_t*>(a.aggs),
                a.n,                                  a.desc,
                a.watchdog,                           a.num_runs,
                a.num_tiles,                          a.epoch,
                rbk_backoff(a.n)};
    if (!a.aligned) return launch_rbk_shape<256, 1, 16>(a.mode, p, stream);
    if (a.n >= kRbkLargeMin) {
        // sums: 16,384-element tiles (512 x 4 x 8); run lengths hold no values,
        // so 32,768 (512 x 4 x 16) fit the same registers (measured 5 to 11%
        // faster at 2^25 and 2^28). For k_rle at 2^25 keys and mean run 16,
        // 512 x 4 x 16 was 6% faster than 1024 x 4 x 16 and 3% faster than
        // 256 x 4 x 16; with all keys distinct 1024 x 4 x 16 was 4% faster.
        // from kRbkNtMin keys the keys and values are loaded non-temporally
        // (each is read once): 1.6 to 3.4% faster with all keys distinct and
        // up to 1.3% at mean run 16, at 2^25, 2^26 and 2^28 keys
        if (a.n >= kRbkNtMin) {
            switch (a.mode) {
            case 0: return launch_rbk_mode<512, 4, 8, 0, true>(p, stream);
            case 1: return launch_rbk_mode<512, 4, 8, 1, true>(p, stream);
            case 2: return launch_rbk_mode<512, 4, 16, 2, true>(p, stream);
            default: return hipErrorInvalidValue;
            }
        }
        switch (a.mode) {
        case 0: return launch_rbk_mode<512, 4, 8, 0>(p, stream);
        case 1: return launch_rbk_mode<512, 4, 8, 1>(p, stream);
        case 2: return launch_rbk_mode<512, 4, 16, 2>(p, stream);
        default: return hipErrorInvalidValue;
        }
    }
    return launch_rbk_shape<256, 4, 4>(a.mode, p, stream);
}

}  // namespace dws

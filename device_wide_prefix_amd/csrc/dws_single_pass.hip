// Single-pass device-wide + scan with decoupled look-back for gfx950
// (Merrill & Garland, "Single-pass Parallel Prefix Scan with Decoupled
// Look-back", section 4.1 steps and section 4.4 adaptations), and the chained
// scan that waits on the immediate predecessor only (section 3.2, Fig 4).
//
// One workgroup per tile; the kernel is the whole call (no init launch):
//   1. lane 0 draws (tile, epoch) from the workspace counter (dynamic tile
//      index, PMPP 11.3 notes);
//   2. every wave loads its segment of the tile with coalesced vector loads,
//      CHUNKS x VEC elements per lane kept in registers (thread coarsening,
//      PMPP 11.2 notes);
//   3. lane-serial totals -> wave64 DPP scans -> the wave totals go through
//      LDS, giving each wave its prefix inside the tile and the tile aggregate;
//   4. wave 0 publishes {A, aggregate} (tile 0: {P, aggregate}), looks back
//      over 64 predecessor descriptors per step until the nearest P, and
//      publishes {P, prefix + aggregate};
//   5. every element gets prefix + wave prefix + chunk/lane prefix + its
//      serial in-lane prefix, and the tile is stored. The whole tile is in
//      registers before the first store, so d_out == d_in is safe.
#include <utility>

#include "dws_device.hpp"
#include "dws_internal.h"

namespace dws {

struct SinglePassParams {
    const void* in;
    void* out;
    uint64_t n;
    uint64_t* desc;
    unsigned long long* counter;
    unsigned int* watchdog;
    uint32_t num_tiles;
};

template <class T, bool EXCL, int BLOCK, int VEC, int CHUNKS, int ORDER, int MODE, bool NT>
__global__ void __launch_bounds__(BLOCK) k_single_pass(SinglePassParams p)
{
    constexpr int W = BLOCK / 64;
    constexpr uint32_t SEG = 64u * VEC * CHUNKS;
    constexpr uint32_t TILE = W * SEG;
    __shared__ uint32_t s_draw[2];
    __shared__ T s_wave[W];
    __shared__ T s_prefix;

    const int lane = lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const bool multi = p.num_tiles > 1u;

    uint32_t tile = 0u, epoch = 0u;
    if (multi) {
        if (threadIdx.x == 0) {
            uint32_t t, e;
            draw_tile(p.counter, p.num_tiles, t, e);
            s_draw[0] = t;
            s_draw[1] = e;
        }
        __syncthreads();
        tile = uniform(s_draw[0]);
        epoch = uniform(s_draw[1]);
        // a counter that was not re-armed would hand out indices past the
        // grid; never touch memory with them (counts as a watchdog trip)
        if (tile >= p.num_tiles) {
            if (threadIdx.x == 0) atomicAdd(p.watchdog, 1u);
            return;
        }
    }

    const uint64_t tile_base = (uint64_t)tile * TILE;
    const uint64_t seg_base = tile_base + (uint64_t)wave * SEG;
    const bool full = tile_base + TILE <= p.n;

    T x[CHUNKS][VEC];
    load_segment<T, VEC, CHUNKS, NT>(static_cast<const T*>(p.in), seg_base, p.n, full, lane, x);

    T lane_excl[CHUNKS], chunk_pre[CHUNKS];
    const T seg_total = scan_segment<T, VEC, CHUNKS>(x, lane_excl, chunk_pre);

    if (lane == 0) s_wave[wave] = seg_total;
    __syncthreads();
    T wave_pre = T(0), agg = T(0);
#pragma unroll
    for (int w = 0; w < W; ++w) {
        if (w == wave) wave_pre = agg;
        agg = agg + s_wave[w];
    }

    if (wave == 0) {
        T prefix = T(0);
        if (multi) {
            if (tile == 0u) {
                if (lane == 0) desc_store<ORDER>(p.desc, desc_pack(epoch, kStatusP, Elem<T>::bits(agg)));
            } else {
                if constexpr (MODE == kModeDecoupled) {
                    if (lane == 0)
                        desc_store<ORDER>(p.desc + tile, desc_pack(epoch, kStatusA, Elem<T>::bits(agg)));
                    prefix = lookback_decoupled<T, ORDER>(p.desc, tile, epoch, p.watchdog);
                } else {
                    prefix = lookback_chained<T, ORDER>(p.desc, tile, epoch, p.watchdog);
                }
                if (lane == 0)
                    desc_store<ORDER>(p.desc + tile,
                                      desc_pack(epoch, kStatusP, Elem<T>::bits(prefix + agg)));
            }
        }
        if (lane == 0) s_prefix = prefix;
    }
    __syncthreads();
    const T seed = s_prefix + wave_pre;

    T y[CHUNKS][VEC];
    finish_segment<T, EXCL, VEC, CHUNKS>(x, lane_excl, chunk_pre, seed, y);
    store_segment<T, VEC, CHUNKS, NT>(static_cast<T*>(p.out), seg_base, p.n, full, lane, y);
}

// ---------------------------------------------------------------------------
// Built kernel configurations.
// ---------------------------------------------------------------------------
struct KernelCfg {
    int threads, vec, chunks, order, mode;
    bool nt;
};

constexpr KernelCfg kCfgs[] = {
    // decoupled look-back, relaxed descriptor atomics: every aligned shape
    {kAlignedShapes[0].threads, 4, kAlignedShapes[0].chunks, kOrderRelaxed, kModeDecoupled, false},
    {kAlignedShapes[1].threads, 4, kAlignedShapes[1].chunks, kOrderRelaxed, kModeDecoupled, false},
    {kAlignedShapes[2].threads, 4, kAlignedShapes[2].chunks, kOrderRelaxed, kModeDecoupled, false},
    {kAlignedShapes[3].threads, 4, kAlignedShapes[3].chunks, kOrderRelaxed, kModeDecoupled, false},
    {kAlignedShapes[4].threads, 4, kAlignedShapes[4].chunks, kOrderRelaxed, kModeDecoupled, false},
    {kAlignedShapes[5].threads, 4, kAlignedShapes[5].chunks, kOrderRelaxed, kModeDecoupled, false},
    // default shape: unaligned (scalar loads), release/acquire, non-temporal
    {256, 1, 16, kOrderRelaxed, kModeDecoupled, false},
    {256, 4, 4, kOrderAcqRel, kModeDecoupled, false},
    {256, 1, 16, kOrderAcqRel, kModeDecoupled, false},
    {256, 4, 4, kOrderRelaxed, kModeDecoupled, true},
    // chained scan
    {256, 4, 4, kOrderRelaxed, kModeChained, false},
    {256, 4, 4, kOrderAcqRel, kModeChained, false},
    {256, 1, 16, kOrderRelaxed, kModeChained, false},
    {256, 1, 16, kOrderAcqRel, kModeChained, false},
};
constexpr size_t kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

static_assert(kAlignedShapes[0].threads == 256 && kAlignedShapes[0].vec == 4 &&
                  kAlignedShapes[0].chunks == 4,
              "the unaligned and comparison kernels assume the default shape 256 x 4 x 4");

static TileShape shape_of(int shape, bool aligned)
{
    const TileShape s = kAlignedShapes[shape];
    // unaligned pointers always take the default shape with scalar loads
    return aligned ? s : unaligned_shape(kAlignedShapes[0]);
}

static int find_cfg(int shape, bool aligned, int order, int mode, bool nt)
{
    if (shape < 0 || shape >= kNumShapes) return -1;
    const TileShape s = shape_of(shape, aligned);
    for (size_t i = 0; i < kNumCfgs; ++i) {
        const KernelCfg& c = kCfgs[i];
        if (c.threads == s.threads && c.vec == s.vec && c.chunks == s.chunks && c.order == order &&
            c.mode == mode && c.nt == nt)
            return (int)i;
    }
    return -1;
}

bool single_pass_available(int shape, bool aligned, int order, int mode, bool nontemporal)
{
    return find_cfg(shape, aligned, order, mode, nontemporal) >= 0;
}

uint32_t single_pass_tile_elems(int shape, bool aligned)
{
    if (shape < 0 || shape >= kNumShapes) return 0;
    return (uint32_t)shape_of(shape, aligned).elems();
}

uint32_t single_pass_threads(int shape, bool aligned)
{
    if (shape < 0 || shape >= kNumShapes) return 0;
    return (uint32_t)shape_of(shape, aligned).threads;
}

template <class T, bool EXCL, size_t I>
static hipError_t launch_typed(const SinglePassParams& p, hipStream_t stream)
{
    constexpr KernelCfg c = kCfgs[I];
    const void* fn = reinterpret_cast<const void*>(
        &k_single_pass<T, EXCL, c.threads, c.vec, c.chunks, c.order, c.mode, c.nt>);
    SinglePassParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(fn, dim3(p.num_tiles), dim3(c.threads), args, 0, stream);
}

template <size_t I>
static hipError_t launch_cfg(const SinglePassArgs& a, hipStream_t stream)
{
    const SinglePassParams p{a.in, a.out, a.n, a.desc, a.counter, a.watchdog, a.num_tiles};
    if (a.kind == kKindF32)
        return a.exclusive ? launch_typed<float, true, I>(p, stream) : launch_typed<float, false, I>(p, stream);
    return a.exclusive ? launch_typed<uint32_t, true, I>(p, stream) : launch_typed<uint32_t, false, I>(p, stream);
}

template <size_t... I>
static hipError_t dispatch(int idx, const SinglePassArgs& a, hipStream_t stream, std::index_sequence<I...>)
{
    hipError_t r = hipErrorInvalidValue;
    (void)((idx == (int)I ? (r = launch_cfg<I>(a, stream), true) : false) || ...);
    return r;
}

hipError_t launch_single_pass(const SinglePassArgs& a, hipStream_t stream)
{
    const int idx = find_cfg(a.shape, a.aligned, a.order, a.mode, a.nontemporal);
    if (idx < 0) return hipErrorInvalidValue;
    if (a.num_tiles == 0u) return hipSuccess;
    return dispatch(idx, a, stream, std::make_index_sequence<kNumCfgs>{});
}

}  // namespace dws

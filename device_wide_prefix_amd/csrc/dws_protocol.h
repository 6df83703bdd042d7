// Constants shared by the host launcher and the kernels: descriptor word
// layout, epochs, memory orders, look-back modes and tile shapes.
#pragma once

#include <stdint.h>

namespace dws {

// Descriptor word: [63:34] epoch, [33:32] status, [31:0] value bits.
// Status codes follow the three states of the decoupled look-back
// (Merrill & Garland, section 4.1): X no information, A aggregate available,
// P inclusive prefix available. A word whose epoch is not the current call's
// reads as X, so a zeroed array (epoch 0, never used) is all-X. The host gives
// every launch on a workspace the next epoch, which replaces the separate
// descriptor-initialisation step of section 4.1 (step 1).
constexpr uint32_t kStatusX = 0u;
constexpr uint32_t kStatusA = 1u;
constexpr uint32_t kStatusP = 2u;
constexpr uint32_t kDescStatusBits = 2u;
constexpr uint32_t kDescStatusMask = 3u;
constexpr uint32_t kEpochMax = (1u << 30) - 1u;  // epochs run 1 .. kEpochMax

// Descriptor spacing: the descriptor of tile t (the first of its words, for
// the two-word descriptors of the pair operators) is word t * kDescStride of
// the descriptor array, so consecutive tiles' descriptors sit 64 bytes apart.
// Packed 8 bytes apart, the few cache lines of the most recent tiles' words
// take every look-back poll and every publication on the GPU at once; spread
// out, the same traffic goes to many lines. Measured on MI355X (+ scan, fp32,
// exclusive in place, one look-back slot): 342 us at 2^28 against 359-362 us
// packed (the best packed schedule), 5-10% faster at 2^20 to 2^23, 2-3% at
// 2^24, 4-6% at 2^25 to 2^27 and 3% at 2^30. 128- and 256-byte spacing measured
// the same as 64; 4 KiB apart (a poll then touches 64 distinct pages) was
// slower.
constexpr uint32_t kDescStride = 8;

// Tile counter word: draws made in the current call (the last draw of a call
// puts it back to 0).
constexpr uint64_t kCounterInit = 0ull;

// Look-back safety limit: 2 s of the 100 MHz real-time counter.
constexpr uint64_t kWatchdogTicks = 200000000ull;

constexpr int kOrderRelaxed = 0;
constexpr int kOrderAcqRel = 1;

constexpr int kModeDecoupled = 0;
constexpr int kModeChained = 1;

// Where a workgroup's tile index comes from. kTileDrawn: one atomic add on
// the workspace counter per workgroup, in the order workgroups start running
// (PMPP 11.3 notes, dynamic block index). kTileDispatch: the workgroup index
// itself, relying on the dispatcher starting workgroups in index order within
// each XCD, so every tile a workgroup waits on has been started before it. No
// atomic, but the guarantee is the hardware's, not the protocol's; a wait that
// outlives the watchdog still ends.
constexpr int kTileDrawn = 0;
constexpr int kTileDispatch = 1;

// Element kinds the kernels are built for (int32 runs as u32).
constexpr int kKindU32 = 0;
constexpr int kKindF32 = 1;

// Tile shapes of the single-pass kernel: threads per workgroup, elements per
// load (4 = one dwordx4 per lane, 1 = scalar loads for pointers that are not
// 16-byte aligned) and loads per lane.
struct TileShape {
    int threads;
    int vec;
    int chunks;
    constexpr int elems() const { return threads * vec * chunks; }
};

// Explicit shapes (option tile_shape = index + 1; tile_shape 0 is automatic).
// Large tiles matter on this GPU: every tile costs one draw on the single
// tile counter and a look-back wait for its slowest predecessor, during which
// the workgroup holds its registers without loading. 32K-65K-element tiles
// keep enough bytes in flight to run at memory speed.
constexpr TileShape kShapes[] = {
    {256, 4, 4},     // 0:  4096 elements (16 KiB)
    {256, 4, 8},     // 1:  8192
    {512, 4, 8},     // 2:  16384
    {1024, 4, 4},    // 3:  16384
    {1024, 4, 8},    // 4:  32768
    {1024, 4, 16},   // 5:  65536 (256 KiB)
};
constexpr int kNumShapes = (int)(sizeof(kShapes) / sizeof(kShapes[0]));

// Automatic shape, from a sweep of every shape with both tile index sources
// at n = 2^16 .. 2^28 on MI355X (fp32, exclusive, in place, caches flushed):
// the best tile grows with n as long as every CU still gets tiles.
constexpr uint64_t kAutoHugeMin = (uint64_t)1 << 24;    // 65536-element tiles
constexpr uint64_t kAutoLargeMin = (uint64_t)1 << 23;   // 32768
constexpr uint64_t kAutoMediumMin = (uint64_t)1 << 20;  // 16384 (512 threads)
// Back-off levels of a look-back that is still blocked after its first,
// immediate re-poll (lookback_pause): a short pause (s_sleep 1), or 64 units
// of 64 clocks before every further poll. (Sleeps of 127 and 190 units paid
// only while descriptors were packed 8 bytes apart.)
constexpr uint32_t kPauseShort = 0u;
constexpr uint32_t kPause64 = 1u;
// A + scan with a drawn tile index backs off from here: 64 units, the best of
// 16 / 32 / 64 / 127 at 2^27 to 2^30 with spread descriptors (127 equal). The
// workgroup-index scan keeps the short pause at every size: 1.3 to 3.4% faster
// than 64 units at 2^24 to 2^26 elements, 2% at 2^28 (6,540 against 6,413 GB/s,
// three alternating runs each) and 0.7% at 2^30 - 12,345.
constexpr uint64_t kScanBackoffMin = (uint64_t)1 << 27;

constexpr uint32_t scan_backoff(uint64_t n, int tile_index)
{
    return tile_index == kTileDrawn && n >= kScanBackoffMin ? kPause64 : kPauseShort;
}
// From here the automatic choice loads the input with non-temporal loads (each
// element is read once), in place or not; stores stay ordinary. Measured on
// MI355X: with the 65,536-element drawn kernel, alternating builds on two
// GPUs, 3.4 to 3.9% faster at 2^28 elements, 3.0 to 3.2% at 2^29, 3.3% at 2^30;
// with descriptors 64 bytes apart and the workgroup index (cold caches, three
// rounds of 30 to 40 calls), 2.5 to 3.5% faster at 2^23 (32,768-element
// tiles), 2% at 2^24, 4.5% at 2^25, 2.7% at 2^26 in place and 4.9% out of
// place, and equal at 2^20 to 2^22. Non-temporal stores, alone or with the
// loads, were slower at every size measured. The generic operators, select,
// partition and the run kernels measured faster from 2^25 elements and load
// non-temporally from there (with their large-tile kernels).
constexpr uint64_t kNtLoadMin = (uint64_t)1 << 23;

constexpr int auto_shape(uint64_t n)
{
    return n >= kAutoHugeMin ? 5 : (n >= kAutoLargeMin ? 4 : (n >= kAutoMediumMin ? 2 : 0));
}

// Automatic tile index of the relaxed single pass: the workgroup index, at
// every size. It needs no atomic on the critical path. With non-temporal loads
// in both kernels it measured 4.4% faster than a drawn index at 2^28 elements
// in place (6,540 against 6,265 GB/s, three alternating runs each) and 6.9% at
// 2^30 - 12,345 (6,506 against 6,087), 1.5 to 3% at 2^25 and 2^26. Earlier
// comparisons that favoured the drawn index from 2^27 set a drawn kernel with
// non-temporal loads against a workgroup-index kernel without them. The
// workgroup index relies on the GPU starting each XCD's workgroups in index
// order (the lowest unfinished tile is then always running); the watchdog
// bounds every wait. The drawn index stays selectable (DWS_TILE_DRAWN), and
// the chained and release/acquire kernels always draw.
constexpr int auto_tile_index(uint64_t) { return kTileDispatch; }

// Scalar-load version of a shape: one element per load, at most 16 loads per
// lane (each load is one wave scan; more would spill registers).
constexpr TileShape scalar_shape(const TileShape& s)
{
    return TileShape{s.threads, 1, s.vec * s.chunks < 16 ? s.vec * s.chunks : 16};
}

// Look-back width: descriptors per lane per poll (64 * K per poll). With
// spread descriptors one slot is enough: P advances by up to 64 tiles per poll
// latency, and each poll costs half the lines of two slots. Measured at 2^25 to
// 2^30 elements: K = 1 equal to or up to 2% faster than K = 2, 1-5% faster than
// K = 4. (With packed descriptors K = 4 had been the best.)
constexpr int kLookbackSlots = 1;

// Built single-pass kernel configurations. Shape index into kShapes; vec 1
// means the scalar-load version of that shape.
struct KernelCfg {
    int shape, vec, order, mode;
    bool nt;
    int tile_index = kTileDrawn;
    bool instr = false;   // records per-tile phase time stamps (measurement build)
};

#define DWS_AUTO_SHAPES(VEC, ORDER, MODE, NT) \
    {0, VEC, ORDER, MODE, NT}, {2, VEC, ORDER, MODE, NT}, {4, VEC, ORDER, MODE, NT}, {5, VEC, ORDER, MODE, NT}
#define DWS_DISPATCH(SHAPE, VEC) {SHAPE, VEC, kOrderRelaxed, kModeDecoupled, false, kTileDispatch}

constexpr KernelCfg kCfgs[] = {
    // decoupled look-back, relaxed descriptor atomics: every shape, and the
    // scalar-load versions of the automatic shapes
    {1, 4, kOrderRelaxed, kModeDecoupled, false},
    {3, 4, kOrderRelaxed, kModeDecoupled, false},
    DWS_AUTO_SHAPES(4, kOrderRelaxed, kModeDecoupled, false),
    DWS_AUTO_SHAPES(1, kOrderRelaxed, kModeDecoupled, false),
    // release/acquire descriptors
    DWS_AUTO_SHAPES(4, kOrderAcqRel, kModeDecoupled, false),
    DWS_AUTO_SHAPES(1, kOrderAcqRel, kModeDecoupled, false),
    // non-temporal loads (aligned pointers only)
    DWS_AUTO_SHAPES(4, kOrderRelaxed, kModeDecoupled, true),
    // chained scan
    DWS_AUTO_SHAPES(4, kOrderRelaxed, kModeChained, false),
    DWS_AUTO_SHAPES(1, kOrderRelaxed, kModeChained, false),
    DWS_AUTO_SHAPES(4, kOrderAcqRel, kModeChained, false),
    DWS_AUTO_SHAPES(1, kOrderAcqRel, kModeChained, false),
    // tile index = workgroup index: every shape aligned, automatic shapes
    // with scalar loads
    DWS_DISPATCH(0, 4), DWS_DISPATCH(1, 4), DWS_DISPATCH(2, 4), DWS_DISPATCH(3, 4), DWS_DISPATCH(4, 4),
    DWS_DISPATCH(5, 4), DWS_DISPATCH(0, 1), DWS_DISPATCH(2, 1), DWS_DISPATCH(4, 1), DWS_DISPATCH(5, 1),
    // the same with non-temporal loads: the automatic choice from kNtLoadMin
    // (32,768- and 65,536-element tiles)
    {4, 4, kOrderRelaxed, kModeDecoupled, true, kTileDispatch},
    {5, 4, kOrderRelaxed, kModeDecoupled, true, kTileDispatch},
    // instrumented (time stamps): the automatic configurations
    {0, 4, kOrderRelaxed, kModeDecoupled, false, kTileDispatch, true},
    {2, 4, kOrderRelaxed, kModeDecoupled, false, kTileDispatch, true},
    {4, 4, kOrderRelaxed, kModeDecoupled, false, kTileDispatch, true},
    {5, 4, kOrderRelaxed, kModeDecoupled, false, kTileDispatch, true},
    {4, 4, kOrderRelaxed, kModeDecoupled, true, kTileDispatch, true},
    {5, 4, kOrderRelaxed, kModeDecoupled, true, kTileDispatch, true},
};
#undef DWS_AUTO_SHAPES
#undef DWS_DISPATCH
constexpr int kNumCfgs = (int)(sizeof(kCfgs) / sizeof(kCfgs[0]));

constexpr TileShape cfg_shape(const KernelCfg& c)
{
    return c.vec == 4 ? kShapes[c.shape] : scalar_shape(kShapes[c.shape]);
}

// Reduce-then-scan: at most this many chunks (one partial each).
constexpr uint32_t kRtsMaxGroups = 4096u;

// Protocol-inspection kernel: one wavefront per tile of 1..64 elements.
constexpr uint32_t kDebugMaxTile = 64u;

// Instrumented scan: 64-bit time stamps per tile (start, tile index known, aggregate
// published, prefix known, stores issued).
constexpr uint32_t kStampsPerTile = 5u;

}  // namespace dws

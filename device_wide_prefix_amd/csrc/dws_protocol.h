// Constants shared by the host launcher and the kernels: descriptor word
// layout, epochs, memory orders, look-back modes and tile shapes.
#pragma once

#include <stdint.h>

namespace dws {

// Descriptor word: [63:34] epoch, [33:32] status, [31:0] value bits.
// Status codes follow the three states of the decoupled look-back
// (Merrill & Garland, section 4.1): X no information, A aggregate available,
// P inclusive prefix available. A word whose epoch is not the current call's
// reads as X, so a zeroed array (epoch 0, never used) is all-X.
constexpr uint32_t kStatusX = 0u;
constexpr uint32_t kStatusA = 1u;
constexpr uint32_t kStatusP = 2u;
constexpr uint32_t kDescStatusBits = 2u;
constexpr uint32_t kDescStatusMask = 3u;
constexpr uint32_t kEpochMax = (1u << 30) - 1u;  // epochs run 1 .. kEpochMax

// Tile counter word: [63:32] epoch, [31:0] draws made in the current call.
constexpr uint64_t kCounterInit = (uint64_t)1 << 32;  // epoch 1, no draws

// Look-back safety limit: 2 s of the 100 MHz real-time counter.
constexpr uint64_t kWatchdogTicks = 200000000ull;

constexpr int kOrderRelaxed = 0;
constexpr int kOrderAcqRel = 1;

constexpr int kModeDecoupled = 0;
constexpr int kModeChained = 1;

// Element kinds the kernels are built for (int32 runs as u32).
constexpr int kKindU32 = 0;
constexpr int kKindF32 = 1;

// Tile shapes of the single-pass kernel: threads per workgroup, elements per
// load (4 = one dwordx4 per lane) and loads per lane.
struct TileShape {
    int threads;
    int vec;
    int chunks;
    constexpr int elems() const { return threads * vec * chunks; }
};

// index 0 is the default; the unaligned path uses VEC 1 with the same tile size
constexpr TileShape kAlignedShapes[] = {
    {256, 4, 4},    // 4096 elements (16 KiB)
    {256, 4, 8},    // 8192
    {512, 4, 4},    // 8192
    {512, 4, 8},    // 16384
    {1024, 4, 4},   // 16384
    {128, 4, 8},    // 4096
};
constexpr int kNumShapes = (int)(sizeof(kAlignedShapes) / sizeof(kAlignedShapes[0]));

constexpr TileShape unaligned_shape(const TileShape& s) { return TileShape{s.threads, 1, s.vec * s.chunks}; }

// Reduce-then-scan: at most this many chunks (one partial each).
constexpr uint32_t kRtsMaxGroups = 4096u;

// Protocol-inspection kernel: one wavefront per tile of 1..64 elements.
constexpr uint32_t kDebugMaxTile = 64u;

}  // namespace dws

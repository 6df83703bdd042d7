// Host side of the single-pass scan: shape policy and configuration lookup.
#include "dws_internal.h"

namespace dws {

static bool scalar_version_built(int shape)
{
    for (int i = 0; i < kNumCfgs; ++i)
        if (kCfgs[i].shape == shape && kCfgs[i].vec == 1) return true;
    return false;
}

int resolve_shape(int option_shape, uint64_t n, bool aligned)
{
    int s = option_shape == 0 ? auto_shape(n) : option_shape - 1;
    if (s < 0 || s >= kNumShapes) return -1;
    if (!aligned && !scalar_version_built(s)) s = auto_shape(n);
    return s;
}

int find_single_pass_cfg(int shape, bool aligned, int order, int mode, bool nontemporal, int tile_index,
                         bool instr)
{
    const int vec = aligned ? 4 : 1;
    for (int i = 0; i < kNumCfgs; ++i) {
        const KernelCfg& c = kCfgs[i];
        if (c.shape == shape && c.vec == vec && c.order == order && c.mode == mode && c.nt == nontemporal &&
            c.tile_index == tile_index && c.instr == instr)
            return i;
    }
    return -1;
}

}  // namespace dws

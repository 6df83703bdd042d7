// Single-pass scan kernels instantiated for 32-bit integers (int32 and
// uint32 share them: wrapping addition gives the same bits).
#include "dws_single_pass_kernel.hpp"

namespace dws {
template hipError_t launch_single_pass_typed<uint32_t>(int, bool, const SinglePassParams&, hipStream_t);
}  // namespace dws

// Single-pass scan kernels instantiated for fp32.
#include "dws_single_pass_kernel.hpp"

namespace dws {
template hipError_t launch_single_pass_typed<float>(int, bool, const SinglePassParams&, hipStream_t);
}  // namespace dws

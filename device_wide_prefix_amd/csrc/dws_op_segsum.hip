// Segmented + on (flag, value) pairs, a non-commutative operator, on the
// generic-operator single-pass scan.
#include "dws_op_kernel.hpp"

namespace dws {

hipError_t launch_op_segsum(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                            hipStream_t stream)
{
    switch (kind) {
    case kOpSegSumIF: return launch_op_typed<OpSegSumIF>(exclusive, shape, nt, p, stream);
    case kOpSegSumU32: return launch_op_typed<OpSegSumU32>(exclusive, shape, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce_op_segsum(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream)
{
    switch (kind) {
    case kOpSegSumIF: return launch_reduce_op_typed<OpSegSumIF>(aligned, nt, p, stream);
    case kOpSegSumU32: return launch_reduce_op_typed<OpSegSumU32>(aligned, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dws

// Componentwise + of {int32, fp32} and uint32 pairs, on the generic-operator
// single-pass scan.
#include "dws_op_kernel.hpp"

namespace dws {

hipError_t launch_op_pairsum(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                             hipStream_t stream)
{
    switch (kind) {
    case kOpSumPairIF: return launch_op_typed<OpSumPairIF>(exclusive, shape, nt, p, stream);
    case kOpSumPairU32: return launch_op_typed<OpSumPairU32>(exclusive, shape, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce_op_pairsum(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream)
{
    switch (kind) {
    case kOpSumPairIF: return launch_reduce_op_typed<OpSumPairIF>(aligned, nt, p, stream);
    case kOpSumPairU32: return launch_reduce_op_typed<OpSumPairU32>(aligned, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dws

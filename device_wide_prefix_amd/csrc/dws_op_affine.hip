// Composition of affine maps modulo 2^32 (first-order linear recurrences), a
// non-commutative operator, on the generic-operator single-pass scan.
#include "dws_op_kernel.hpp"

namespace dws {

hipError_t launch_op_affine(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                            hipStream_t stream)
{
    if (kind != kOpAffineU32) return hipErrorInvalidValue;
    return launch_op_typed<OpAffineU32>(exclusive, shape, nt, p, stream);
}

hipError_t launch_reduce_op_affine(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream)
{
    switch (kind) {
    case kOpAffineU32: return launch_reduce_op_typed<OpAffineU32>(aligned, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dws

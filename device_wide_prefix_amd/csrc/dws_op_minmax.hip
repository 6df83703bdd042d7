// Running max and min of 32-bit integers (signed and unsigned), on the
// generic-operator single-pass scan.
#include "dws_op_kernel.hpp"

namespace dws {

hipError_t launch_op_minmax(int kind, bool exclusive, int shape, bool nt, const OpScanParams& p,
                            hipStream_t stream)
{
    switch (kind) {
    case kOpMaxI32: return launch_op_typed<OpMaxI32>(exclusive, shape, nt, p, stream);
    case kOpMaxU32: return launch_op_typed<OpMaxU32>(exclusive, shape, nt, p, stream);
    case kOpMinI32: return launch_op_typed<OpMinI32>(exclusive, shape, nt, p, stream);
    case kOpMinU32: return launch_op_typed<OpMinU32>(exclusive, shape, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce_op_minmax(int kind, bool aligned, bool nt, const OpReduceParams& p, hipStream_t stream)
{
    switch (kind) {
    case kOpMaxI32: return launch_reduce_op_typed<OpMaxI32>(aligned, nt, p, stream);
    case kOpMaxU32: return launch_reduce_op_typed<OpMaxU32>(aligned, nt, p, stream);
    case kOpMinI32: return launch_reduce_op_typed<OpMinI32>(aligned, nt, p, stream);
    case kOpMinU32: return launch_reduce_op_typed<OpMinU32>(aligned, nt, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dws

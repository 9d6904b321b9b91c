// Forward-kernel instantiations, f16 element type, fused bias / activation /
// residual epilogue.
#include "eql_fwd_inst.h"

namespace eql {

hipError_t launch_fwd_fused_f16(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
  return FwdInst<_Float16, 1>::run(T, NB, a, grid, s);
}

}  // namespace eql

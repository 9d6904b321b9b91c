// Forward-kernel instantiations, f32 element type, fused bias / activation /
// residual epilogue.
#include "eql_fwd_inst.h"

namespace eql {

hipError_t launch_fwd_fused_f32(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
  return FwdInst<float, 1>::run(T, NB, a, grid, s);
}

}  // namespace eql

// Fused weight-gradient kernel instantiations: T in {1, 2, 4}, fp16 and fp32.
#include "eql_bwdw4.h"
#include "eql_launch.h"

namespace eql {

template <typename Elt>
static hipError_t bwdw4_one(int T, const Bwdw4Args& a, unsigned grid, hipStream_t s) {
  switch (T) {
    case 1: return launch_kernel((const void*)&eql_bwdw4_kernel<1, Elt>, grid, a, s);
    case 2: return launch_kernel((const void*)&eql_bwdw4_kernel<2, Elt>, grid, a, s);
    case 4: return launch_kernel((const void*)&eql_bwdw4_kernel<4, Elt>, grid, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwdw4(bool f16, int T, const Bwdw4Args& a, unsigned grid, hipStream_t s) {
  return f16 ? bwdw4_one<_Float16>(T, a, grid, s) : bwdw4_one<float>(T, a, grid, s);
}

}  // namespace eql

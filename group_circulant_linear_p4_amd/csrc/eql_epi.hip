// Fused-epilogue backward instantiations, both element types, T = 1..16.
#include "eql_epi.h"
#include "eql_launch.h"

namespace eql {

template <int T, typename Elt>
static hipError_t epi_one(const EpiBwdArgs& a, unsigned grid, hipStream_t s) {
  return launch_kernel((const void*)&eql_epi_bwd_kernel<T, Elt>, grid, a, s);
}

hipError_t launch_epi_bwd(int T, bool f16, const EpiBwdArgs& a, unsigned grid, hipStream_t s) {
  if (f16) {
#define EQL_CASE(t) return epi_one<t, _Float16>(a, grid, s);
    EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
  } else {
#define EQL_CASE(t) return epi_one<t, float>(a, grid, s);
    EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
  }
}

hipError_t launch_epi_bias(bool f16, const EpiBwdArgs& a, unsigned grid, hipStream_t s) {
  return f16 ? launch_kernel((const void*)&eql_epi_bias_kernel<_Float16>, grid, a, s)
             : launch_kernel((const void*)&eql_epi_bias_kernel<float>, grid, a, s);
}

}  // namespace eql

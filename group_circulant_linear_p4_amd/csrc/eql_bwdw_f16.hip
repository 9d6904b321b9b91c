// Weight-gradient transform and reduce instantiations for the f16 element type, T = 1..16.
#include "eql_launch.h"

namespace eql {

template <int T>
static hipError_t spec_one(const SpecArgs& a, unsigned grid, hipStream_t s) {
  return launch_kernel((const void*)&eql_spec_kernel<T, _Float16>, grid, a, s);
}

template <int T>
static hipError_t reduce_one(int waves, const BwdwReduceArgs& a, unsigned grid, hipStream_t s) {
  return waves == 16  ? launch_kernel((const void*)&eql_bwdw_reduce<T, _Float16, 16>, grid, a, s)
         : waves == 4 ? launch_kernel((const void*)&eql_bwdw_reduce<T, _Float16, 4>, grid, a, s)
                      : launch_kernel((const void*)&eql_bwdw_reduce<T, _Float16, 1>, grid, a, s);
}

hipError_t launch_spec_f16(int T, const SpecArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return spec_one<t>(a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

hipError_t launch_bwdw_reduce_f16(int T, int waves, const BwdwReduceArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return reduce_one<t>(waves, a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

}  // namespace eql

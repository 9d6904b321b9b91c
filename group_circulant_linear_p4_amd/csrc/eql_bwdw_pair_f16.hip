// Weight-gradient GEMM instantiations (complex pairs), f16 element type, T = 1..16.
#include "eql_launch.h"

namespace eql {

template <int T>
static hipError_t gemm_one(int DB, int CB, const BwdwArgs& a, unsigned grid, hipStream_t s) {
  if constexpr (n_pairs(T) == 0) {
    return hipErrorInvalidValue;
  } else {
    if (DB == 4 && CB == 2) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, true, 4, 2>, grid, a, s);
    if (DB == 4 && CB == 1) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, true, 4, 1>, grid, a, s);
    if (DB == 1 && CB == 2) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, true, 1, 2>, grid, a, s);
    if (DB == 1 && CB == 1) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, true, 1, 1>, grid, a, s);
    return hipErrorInvalidValue;
  }
}

hipError_t launch_bwdw_pair_f16(int T, int DB, int CB, const BwdwArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return gemm_one<t>(DB, CB, a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

}  // namespace eql

// Weight-gradient GEMM instantiations (real frequencies), f16 element type, T = 1..16.
#include "eql_launch.h"

namespace eql {

template <int T>
static hipError_t gemm_one(int DB, int CB, int WCN, const BwdwArgs& a, unsigned grid, hipStream_t s) {
  if (DB == 4 && CB == 4 && WCN == 2) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, false, 4, 4, 2>, grid, a, s);
  if (DB == 4 && CB == 1 && WCN == 2) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, false, 4, 1, 2>, grid, a, s);
  if (DB == 1 && CB == 4 && WCN == 2) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, false, 1, 4, 2>, grid, a, s);
  if (DB == 1 && CB == 1 && WCN == 2) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, false, 1, 1, 2>, grid, a, s);
  if (DB == 4 && CB == 2 && WCN == 4) return launch_kernel((const void*)&eql_bwdw_gemm<T, _Float16, false, 4, 2, 4>, grid, a, s, 512);
  return hipErrorInvalidValue;
}

hipError_t launch_bwdw_real_f16(int T, int DB, int CB, int WCN, const BwdwArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return gemm_one<t>(DB, CB, WCN, a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

}  // namespace eql

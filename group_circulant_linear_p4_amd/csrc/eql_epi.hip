// Fused-epilogue backward instantiations: both element types, every chunk width
// (and, for the bias reduction, every T).
#include "eql_epi.h"
#include "eql_launch.h"

namespace eql {

template <typename Elt, int W>
static hipError_t epi_one(const EpiBwdArgs& a, unsigned grid, hipStream_t s) {
  return launch_kernel((const void*)&eql_epi_bwd_kernel<Elt, W>, grid, a, s);
}

hipError_t launch_epi_bwd(bool f16, int W, const EpiBwdArgs& a, unsigned grid, hipStream_t s) {
  switch (W) {
    case 16: return f16 ? epi_one<_Float16, 16>(a, grid, s) : epi_one<float, 16>(a, grid, s);
    case 8: return f16 ? epi_one<_Float16, 8>(a, grid, s) : epi_one<float, 8>(a, grid, s);
    case 4: return f16 ? epi_one<_Float16, 4>(a, grid, s) : epi_one<float, 4>(a, grid, s);
    case 2: return f16 ? epi_one<_Float16, 2>(a, grid, s) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int T>
static hipError_t bias_one(bool f16, const EpiBwdArgs& a, unsigned grid, hipStream_t s) {
  return f16 ? launch_kernel((const void*)&eql_epi_bias_kernel<T, _Float16>, grid, a, s)
             : launch_kernel((const void*)&eql_epi_bias_kernel<T, float>, grid, a, s);
}

hipError_t launch_epi_bias(bool f16, const EpiBwdArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return bias_one<t>(f16, a, grid, s);
  EQL_FOR_EACH_T(a.T, EQL_CASE)
#undef EQL_CASE
}

}  // namespace eql

// Forward-kernel instantiations for the f32 element type, T = 1..16.
#include "eql_launch.h"

namespace eql {

// Aligned rows: the full-width and the one-column-block tile.  Unaligned rows
// (narrow loads): the one-column-block tile only.
template <int T>
static hipError_t fwd_one(int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
  constexpr int NBM = fwd_nb_max(T), JC = fwd_jc(T);
  if (!a.aligned16) {
    if (NB != 1) return hipErrorInvalidValue;
    return launch_kernel((const void*)&eql_fwd_kernel<T, float, 1, JC, false>, grid, a, s);
  }
  if (NB == NBM) return launch_kernel((const void*)&eql_fwd_kernel<T, float, NBM, JC, true>, grid, a, s);
  if constexpr (NBM != 1) {
    if (NB == 1) return launch_kernel((const void*)&eql_fwd_kernel<T, float, 1, JC, true>, grid, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return fwd_one<t>(NB, a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

}  // namespace eql

// Forward-kernel instantiations for the f32 element type, T = 1..16.
#include "eql_launch.h"

namespace eql {

// Load modes (see eql_fwd.h): full and checked aligned loads with the full-width
// and the one-column-block tile; narrow loads with the one-column-block tile only.
template <int T, int NB, int MODE>
static hipError_t fwd_launch(const FwdArgs& a, unsigned grid, hipStream_t s) {
  return launch_kernel((const void*)&eql_fwd_kernel<T, float, NB, fwd_jc(T), MODE>, grid, a, s);
}

template <int T>
static hipError_t fwd_one(int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
  constexpr int NBM = fwd_nb_max(T);
  if (a.loadMode == kLoadNarrow) return NB == 1 ? fwd_launch<T, 1, kLoadNarrow>(a, grid, s) : hipErrorInvalidValue;
  if (NB == NBM) {
    return a.loadMode == kLoadFull ? fwd_launch<T, NBM, kLoadFull>(a, grid, s)
                                   : fwd_launch<T, NBM, kLoadAligned>(a, grid, s);
  }
  if constexpr (NBM != 1) {
    if (NB == 1) {
      return a.loadMode == kLoadFull ? fwd_launch<T, 1, kLoadFull>(a, grid, s)
                                     : fwd_launch<T, 1, kLoadAligned>(a, grid, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return fwd_one<t>(NB, a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

}  // namespace eql

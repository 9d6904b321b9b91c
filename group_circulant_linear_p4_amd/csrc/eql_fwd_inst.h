// Forward-kernel instantiations for one element type and epilogue: T = 1..16, the
// full-width tile (fwd_nb_max(T) column blocks), the two-block tile where the full
// width is four blocks, the one-block tile, and the three load modes (see
// eql_fwd.h); T <= 4 with 16-byte rows takes eql_fwd4_kernel.  Each of eql_fwd_{f16,f32}.hip (plain epilogue) and
// eql_fwd_fused_{f16,f32}.hip (bias / activation / residual) instantiates one.
#pragma once

#include "eql_launch.h"

namespace eql {

template <typename Elt, int EPI>
struct FwdInst {
  // T <= 4 with 16-byte rows: the fast kernel; otherwise the generic one.
  template <int T, int NB, int MODE>
  static hipError_t launch(const FwdArgs& a, unsigned grid, hipStream_t s) {
    if constexpr (T <= 4 && MODE != kLoadNarrow) {
      return launch_kernel((const void*)&eql_fwd4_kernel<T, Elt, NB, MODE, EPI>, grid, a, s,
                           64u * (unsigned)fwd4_waves(T, NB));
    } else {
      return launch_kernel((const void*)&eql_fwd_kernel<T, Elt, NB, fwd_jc(T), MODE, EPI>, grid, a, s);
    }
  }

  // Narrow loads with the one-column-block tile only.
  template <int T>
  static hipError_t one(int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
    constexpr int NBM = fwd_nb_max(T);
    if (a.loadMode == kLoadNarrow) return NB == 1 ? launch<T, 1, kLoadNarrow>(a, grid, s) : hipErrorInvalidValue;
    if (NB == NBM) {
      return a.loadMode == kLoadFull ? launch<T, NBM, kLoadFull>(a, grid, s)
                                     : launch<T, NBM, kLoadAligned>(a, grid, s);
    }
    if constexpr (NBM == 4) {
      if (NB == 2) {
        return a.loadMode == kLoadFull ? launch<T, 2, kLoadFull>(a, grid, s)
                                       : launch<T, 2, kLoadAligned>(a, grid, s);
      }
    }
    if constexpr (NBM != 1) {
      if (NB == 1) {
        return a.loadMode == kLoadFull ? launch<T, 1, kLoadFull>(a, grid, s)
                                       : launch<T, 1, kLoadAligned>(a, grid, s);
      }
    }
    return hipErrorInvalidValue;
  }

  static hipError_t run(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return one<t>(NB, a, grid, s);
    EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
  }
};

}  // namespace eql

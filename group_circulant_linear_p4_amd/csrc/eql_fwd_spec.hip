// Forward-kernel instantiations with the spectrum side output (eql_fwd4_kernel,
// SPEC = 1): p4, f16 element type, plain (EPI = 0) or fused (EPI = 1) epilogue, every
// tile width and 16-byte load mode of the fast path.
#include "eql_launch.h"

namespace eql {

namespace {

template <int NB, int EPI>
hipError_t launch_spec_nb(const FwdArgs& a, unsigned grid, hipStream_t s) {
  const unsigned block = 64u * (unsigned)fwd4_waves(4, NB);
  if (a.loadMode == kLoadFull)
    return launch_kernel((const void*)&eql_fwd4_kernel<4, _Float16, NB, kLoadFull, EPI, 1>, grid, a, s, block);
  if (a.loadMode == kLoadAligned)
    return launch_kernel((const void*)&eql_fwd4_kernel<4, _Float16, NB, kLoadAligned, EPI, 1>, grid, a, s, block);
  return hipErrorInvalidValue;
}

template <int EPI>
hipError_t launch_spec_epi(int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
  switch (NB) {
    case 4: return launch_spec_nb<4, EPI>(a, grid, s);
    case 2: return launch_spec_nb<2, EPI>(a, grid, s);
    case 1: return launch_spec_nb<1, EPI>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_spec_f16(int NB, bool epi, const FwdArgs& a, unsigned grid, hipStream_t s) {
  return epi ? launch_spec_epi<1>(NB, a, grid, s) : launch_spec_epi<0>(NB, a, grid, s);
}

}  // namespace eql

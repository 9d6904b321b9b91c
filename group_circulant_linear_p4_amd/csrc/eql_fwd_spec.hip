// Forward-kernel instantiations with the spectrum side output (eql_fwd4_kernel,
// SPEC = 1): p4, f16 element type, plain epilogue, every tile width and 16-byte load
// mode of the fast path.
#include "eql_launch.h"

namespace eql {

namespace {

template <int NB>
hipError_t launch_spec_nb(const FwdArgs& a, unsigned grid, hipStream_t s) {
  const unsigned block = 64u * (unsigned)fwd4_waves(4, NB);
  if (a.loadMode == kLoadFull)
    return launch_kernel((const void*)&eql_fwd4_kernel<4, _Float16, NB, kLoadFull, 0, 1>, grid, a, s, block);
  if (a.loadMode == kLoadAligned)
    return launch_kernel((const void*)&eql_fwd4_kernel<4, _Float16, NB, kLoadAligned, 0, 1>, grid, a, s, block);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_spec_f16(int NB, const FwdArgs& a, unsigned grid, hipStream_t s) {
  switch (NB) {
    case 4: return launch_spec_nb<4>(a, grid, s);
    case 2: return launch_spec_nb<2>(a, grid, s);
    case 1: return launch_spec_nb<1>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eql

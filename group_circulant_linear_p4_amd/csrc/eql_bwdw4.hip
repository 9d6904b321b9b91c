// Fused weight-gradient kernel instantiations: T in {1, 2, 4}, column tiles of 64, 96
// and 128 channels, fp16 and fp32.
#include "eql_bwdw4.h"
#include "eql_launch.h"

namespace eql {

template <typename Elt>
static hipError_t bwdw4_one(int T, int NB, const Bwdw4Args& a, unsigned grid, hipStream_t s) {
  // Tile widths whose spectrum stage splits evenly over the four waves (T NB % 4 == 0).
  const int key = T * 8 + NB;
  switch (key) {
    case 1 * 8 + 4: return launch_kernel((const void*)&eql_bwdw4_kernel<1, Elt, 4>, grid, a, s);
    case 2 * 8 + 2: return launch_kernel((const void*)&eql_bwdw4_kernel<2, Elt, 2>, grid, a, s);
    case 2 * 8 + 4: return launch_kernel((const void*)&eql_bwdw4_kernel<2, Elt, 4>, grid, a, s);
    case 4 * 8 + 2: return launch_kernel((const void*)&eql_bwdw4_kernel<4, Elt, 2>, grid, a, s);
    case 4 * 8 + 3: return launch_kernel((const void*)&eql_bwdw4_kernel<4, Elt, 3>, grid, a, s);
    case 4 * 8 + 4: return launch_kernel((const void*)&eql_bwdw4_kernel<4, Elt, 4>, grid, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwdw4(bool f16, int T, int NB, const Bwdw4Args& a, unsigned grid, hipStream_t s) {
  return f16 ? bwdw4_one<_Float16>(T, NB, a, grid, s) : bwdw4_one<float>(T, NB, a, grid, s);
}

}  // namespace eql

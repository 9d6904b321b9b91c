// Weight-packing kernel instantiations, T = 1..16, fp16 and fp32.
#include "eql_launch.h"

namespace eql {

template <int T, typename Elt>
static hipError_t pack_one(const PackArgs& a, unsigned grid, hipStream_t s) {
  return launch_kernel((const void*)&eql_pack_kernel<T, Elt>, grid, a, s);
}

hipError_t launch_pack_f16(int T, const PackArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return pack_one<t, _Float16>(a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

hipError_t launch_pack_f32(int T, const PackArgs& a, unsigned grid, hipStream_t s) {
#define EQL_CASE(t) return pack_one<t, float>(a, grid, s);
  EQL_FOR_EACH_T(T, EQL_CASE)
#undef EQL_CASE
}

}  // namespace eql

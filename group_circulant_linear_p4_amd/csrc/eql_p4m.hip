// p4m weight expansion and weight-gradient fold: fp16 and fp32.
#include "eql_launch.h"
#include "eql_p4m.h"

namespace eql {

hipError_t launch_p4m_expand(bool f16, const P4mArgs& a, unsigned grid, hipStream_t s) {
  return f16 ? launch_kernel((const void*)&eql_p4m_expand_kernel<_Float16>, grid, a, s)
             : launch_kernel((const void*)&eql_p4m_expand_kernel<float>, grid, a, s);
}

hipError_t launch_p4m_fold(bool f16, const P4mArgs& a, unsigned grid, hipStream_t s) {
  return f16 ? launch_kernel((const void*)&eql_p4m_fold_kernel<_Float16>, grid, a, s)
             : launch_kernel((const void*)&eql_p4m_fold_kernel<float>, grid, a, s);
}

}  // namespace eql

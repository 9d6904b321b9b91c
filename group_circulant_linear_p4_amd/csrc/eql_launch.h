// Internal launch interface between the C ABI (eql_api.hip) and the kernel
// instantiations (one translation unit per kernel family and element type).
#pragma once

#include <hip/hip_runtime.h>

#include "eql_bwdw.h"
#include "eql_bwdw4.h"
#include "eql_epi.h"
#include "eql_fwd.h"
#include "eql_p4m.h"
#include "eql_pack.h"

namespace eql {

// Tile policy, shared by the host (grid sizes, workspace) and the instantiations.
// NB = 32-column blocks per wave: T*NB*16 fp32 accumulators per lane stay <= 256.
__host__ __device__ constexpr int fwd_nb_max(int T) { return T <= 4 ? 4 : (T <= 8 ? 2 : 1); }
// Channel groups per K chunk (two per k-step).
__host__ __device__ constexpr int fwd_jc(int) { return 2; }

// The packed weight's input axis is padded to a multiple of this many 16-byte
// groups, so that every K stage of the forward kernel reads whole groups.
constexpr int kPackGroupAlign = 4;
static_assert(kPackGroupAlign % fwd_jc(1) == 0 && kPackGroupAlign % fwd_jc(16) == 0, "stage size");

// elt: 2 = fp16, 4 = fp32.  Each returns the launch status.
hipError_t launch_fwd_f16(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_fwd_f32(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_fwd_fused_f16(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_fwd_fused_f32(int T, int NB, const FwdArgs& a, unsigned grid, hipStream_t s);
// The forward kernel that also stores the transformed input of the column-0 tiles
// as weight-gradient operand units (p4 fp16, 16-byte rows; FwdArgs::spec), with the
// plain or (epi) the fused epilogue.
hipError_t launch_fwd_spec_f16(int NB, bool epi, const FwdArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_spec_f16(int T, const SpecArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_spec_f32(int T, const SpecArgs& a, unsigned grid, hipStream_t s);
// Weight-gradient GEMMs: the real planes' (DB, CB in {4, 1}) and the complex pairs'
// (DB in {4, 1}, CB in {2, 1}; T >= 3), workgroup tile 64 DB x 64 CB.
hipError_t launch_bwdw_real_f16(int T, int DB, int CB, int WCN, const BwdwArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_bwdw_real_f32(int T, int DB, int CB, int WCN, const BwdwArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_bwdw_pair_f16(int T, int DB, int CB, int WCN, const BwdwArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_bwdw_pair_f32(int T, int DB, int CB, int WCN, const BwdwArgs& a, unsigned grid, hipStream_t s);
// Weight gradient with dy's transform fused into the GEMM (T in {1, 2, 4}).
hipError_t launch_bwdw4(bool f16, int T, int NB, const Bwdw4Args& a, unsigned grid, hipStream_t s);
// p4m: the tied C_4 weight from w, and the p4m weight gradient from the C_4 one.
hipError_t launch_p4m_expand(bool f16, const P4mArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_p4m_fold(bool f16, const P4mArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_bwdw_reduce_f16(int T, int waves, const BwdwReduceArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_bwdw_reduce_f32(int T, int waves, const BwdwReduceArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_pack_f16(int T, const PackArgs& a, unsigned grid, hipStream_t s);
// Fused-epilogue backward: dpre and the bias partials, then the bias sum.
hipError_t launch_epi_bwd(bool f16, int W, const EpiBwdArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_epi_bias(bool f16, const EpiBwdArgs& a, unsigned grid, hipStream_t s);
hipError_t launch_pack_f32(int T, const PackArgs& a, unsigned grid, hipStream_t s);

template <typename A>
inline hipError_t launch_kernel(const void* fn, unsigned grid, const A& args, hipStream_t s, unsigned block = 256) {
  void* kargs[] = {const_cast<A*>(&args)};
  return hipLaunchKernel(fn, dim3(grid), dim3(block), kargs, 0, s);
}

// Expands F(T) for T = 1..16 inside a switch on `t`.
#define EQL_FOR_EACH_T(t, F) \
  switch (t) {               \
    case 1: F(1)             \
    case 2: F(2)             \
    case 3: F(3)             \
    case 4: F(4)             \
    case 5: F(5)             \
    case 6: F(6)             \
    case 7: F(7)             \
    case 8: F(8)             \
    case 9: F(9)             \
    case 10: F(10)           \
    case 11: F(11)           \
    case 12: F(12)           \
    case 13: F(13)           \
    case 14: F(14)           \
    case 15: F(15)           \
    case 16: F(16)           \
    default: return hipErrorInvalidValue; \
  }

}  // namespace eql

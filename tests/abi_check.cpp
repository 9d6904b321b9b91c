// Host-side checks of the C ABI in include/eqlinear.h, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (the library's argument validation,
// size queries and launch planning; device code is not instrumented).  Every call
// here either fails validation or has N = 0, so nothing is launched and no device
// memory is touched; the pointers are never dereferenced.  Exit status 0 when every
// check holds; a sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "eqlinear.h"

namespace {

int g_checks = 0, g_failures = 0;

void check(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    std::fprintf(stderr, "abi_check: FAILED at line %d: %s\n", line, what);
  }
}
#define CHECK(cond) check((cond), #cond, __LINE__)

// Fake, never-dereferenced addresses: 16-byte aligned, and one that is not.
void* const A = reinterpret_cast<void*>(uintptr_t{0x10000});
void* const B = reinterpret_cast<void*>(uintptr_t{0x20000});
void* const C = reinterpret_cast<void*>(uintptr_t{0x30000});
void* const D = reinterpret_cast<void*>(uintptr_t{0x40000});
void* const MIS = reinterpret_cast<void*>(uintptr_t{0x10008});
// Misaligned for an fp32 element (bias and dbias need element alignment only).
void* const MIS2 = reinterpret_cast<void*>(uintptr_t{0x10002});

constexpr int F16 = EQL_F16, F32 = EQL_F32;

void sizes() {
  CHECK(eqlinear_abi_version() == 205);
  for (int s = -3; s < 12; ++s) CHECK(eqlinear_status_string(s) != nullptr && std::strlen(eqlinear_status_string(s)) > 0);
  // Packed weight: out channels padded to 32, input 16-byte groups padded per stage.
  CHECK(eqlinear_packed_weight_bytes(3, 5, 4, F16) == 32u * 4 * 16 * 4);
  CHECK(eqlinear_packed_weight_bytes(1024, 1024, 4, F16) == 1024u * 128 * 16 * 4);
  CHECK(eqlinear_packed_weight_bytes(0, 5, 4, F16) == 0);
  CHECK(eqlinear_packed_weight_bytes(5, 5, 17, F16) == 0);
  CHECK(eqlinear_packed_weight_bytes(5, 5, 4, 7) == 0);
  // Edges of the size rules: rows of 2^23 bytes pass, one element more fails.
  CHECK(eqlinear_packed_weight_bytes(1, (int64_t{1} << 23) / (16 * 2), 16, F16) > 0);
  CHECK(eqlinear_packed_weight_bytes(1, (int64_t{1} << 23) / (16 * 2) + 1, 16, F16) == 0);
  CHECK(eqlinear_packed_weight_bytes(INT64_MAX, 4, 4, F16) == 0);
  CHECK(eqlinear_packed_weight_bytes(4, INT64_MAX, 4, F32) == 0);
  // Workspaces at the largest N and the widest rows the ABI accepts (the planning
  // arithmetic must not overflow).
  const int64_t nmax = (int64_t{1} << 31) - (int64_t{1} << 20);
  for (int dt : {F16, F32}) {
    for (int T : {1, 2, 3, 4, 5, 8, 16}) {
      CHECK(eqlinear_bwd_w_workspace_bytes(nmax, 64, 64, T, dt) > 0);
      CHECK(eqlinear_bwd_w_workspace_bytes(nmax + 1, 64, 64, T, dt) == 0);
      CHECK(eqlinear_bwd_w_workspace_bytes(1000, (int64_t{1} << 23) / (T * 4), 3, T, dt) > 0);
      CHECK(eqlinear_bwd_w_workspace_bytes(1000, 3, (int64_t{1} << 23) / (T * 4), T, dt) > 0);
      CHECK(eqlinear_fused_epilogue_bwd_workspace_bytes(nmax, (int64_t{1} << 23) / (T * 4), T, dt) > 0);
      CHECK(eqlinear_fused_epilogue_bwd_workspace_bytes(nmax, 1, T, dt) > 0);
      CHECK(eqlinear_fused_epilogue_bwd_workspace_bytes(0, 5, T, dt) == 0);
      CHECK(eqlinear_bwd_w_workspace_bytes(0, 5, 5, T, dt) == 0);
    }
  }
  CHECK(eqlinear_bwd_w_workspace_bytes(-1, 5, 5, 4, F16) == 0);
  CHECK(eqlinear_bwd_w_workspace_bytes(10, 5, 5, 4, 9) == 0);
  CHECK(eqlinear_fused_epilogue_bwd_workspace_bytes(10, INT64_MAX, 4, F16) == 0);
}

void validation() {
  // Forward and input gradient.
  for (auto fn : {eqlinear_fwd, eqlinear_bwd_x}) {
    CHECK(fn(A, B, C, 8, 4, 4, 4, 5, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, C, 8, 4, 4, 0, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, C, 8, 4, 4, 17, F16, nullptr) == EQL_EUNSUPPORTED);
    CHECK(fn(A, B, C, -1, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, C, INT64_MIN, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, C, INT64_MAX, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, C, 8, 0, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, C, 8, INT64_MAX, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, C, 8, 4, INT64_MIN, 4, F32, nullptr) == EQL_EINVAL);
    CHECK(fn(nullptr, B, C, 8, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, nullptr, C, 8, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, nullptr, 8, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(MIS, B, C, 8, 4, 4, 4, F16, nullptr) == EQL_EALIGN);
    CHECK(fn(A, MIS, C, 8, 4, 4, 4, F16, nullptr) == EQL_EALIGN);
    CHECK(fn(A, B, MIS, 8, 4, 4, 4, F16, nullptr) == EQL_EALIGN);
    CHECK(fn(nullptr, nullptr, nullptr, 0, 4, 4, 4, F16, nullptr) == EQL_OK);
  }
  // Fused forward.
  CHECK(eqlinear_fwd_fused(A, B, nullptr, nullptr, C, nullptr, 8, 4, 4, 4, F16, 2, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_fused(A, B, MIS2, nullptr, C, nullptr, 8, 4, 4, 4, F32, EQL_ACT_GELU, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused(A, B, nullptr, MIS, C, nullptr, 8, 4, 4, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused(A, B, nullptr, nullptr, C, MIS, 8, 4, 4, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused(A, B, nullptr, nullptr, nullptr, nullptr, 8, 4, 4, 4, F16, 0, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_fused(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 4, 4, F16, 0, nullptr) ==
        EQL_OK);
  // Packing.
  CHECK(eqlinear_pack_weight(A, B, 4, 4, 4, F16, 2, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight(nullptr, B, 4, 4, 4, F16, 0, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight(A, nullptr, 4, 4, 4, F16, 1, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight(MIS, B, 4, 4, 4, F16, 0, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_pack_weight(A, B, 4, 4, 20, F16, 0, nullptr) == EQL_EUNSUPPORTED);
  CHECK(eqlinear_pack_weight(A, B, 0, 4, 4, F16, 0, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight(A, B, INT64_MAX, INT64_MAX, 4, F16, 0, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight_both(A, B, nullptr, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight_both(nullptr, B, C, 4, 4, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight_both(A, B, MIS, 4, 4, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_pack_weight_both(A, B, C, 4, 4, 20, F16, nullptr) == EQL_EUNSUPPORTED);
  CHECK(eqlinear_pack_weight_both(A, B, C, 0, 4, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_pack_weight_both(A, B, C, INT64_MAX, INT64_MAX, 4, F16, nullptr) == EQL_EINVAL);
  // Weight gradient.
  const size_t ws = eqlinear_bwd_w_workspace_bytes(300, 5, 7, 4, F16);
  CHECK(ws > 0);
  CHECK(eqlinear_bwd_w(A, B, C, D, ws - 1, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w(A, B, C, nullptr, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w(nullptr, B, C, D, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w(A, B, nullptr, D, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w(A, B, C, MIS, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_bwd_w(A, MIS, C, D, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_bwd_w(A, B, C, D, ws, 300, 5, 7, 0, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w(A, B, C, D, ws, 300, 5, 7, 4, 3, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w(A, B, C, D, SIZE_MAX, INT64_MAX, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  // Training-step entry points (share the weight-gradient workspace).  (300, 8, 8, 4)
  // takes the fused weight-gradient path, (300, 5, 7, 4) the separate one.
  const size_t wf = eqlinear_bwd_w_workspace_bytes(300, 8, 8, 4, F16);
  CHECK(wf > 0);
  CHECK(eqlinear_fwd_train(A, B, C, D, ws - 1, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_train(A, B, C, nullptr, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_train(A, B, C, MIS, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_train(MIS, B, C, D, wf, 300, 8, 8, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_train(nullptr, B, C, D, wf, 300, 8, 8, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_train(A, B, C, D, ws, 300, 5, 7, 0, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_train(A, B, C, D, ws, 300, 5, 7, 20, F16, nullptr) == EQL_EUNSUPPORTED);
  CHECK(eqlinear_fwd_train(A, B, C, D, SIZE_MAX, INT64_MAX, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_train(nullptr, nullptr, nullptr, nullptr, 0, 0, 5, 7, 4, F16, nullptr) == EQL_OK);
  CHECK(eqlinear_fwd_fused_train(A, B, nullptr, nullptr, C, nullptr, D, ws - 1, 300, 5, 7, 4, F16, 0, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_fused_train(A, B, nullptr, nullptr, C, nullptr, nullptr, ws, 300, 5, 7, 4, F16, 0, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_fused_train(A, B, nullptr, nullptr, C, nullptr, MIS, ws, 300, 5, 7, 4, F16, 0, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused_train(A, B, nullptr, nullptr, C, nullptr, D, ws, 300, 5, 7, 4, F16, 7, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fwd_fused_train(A, B, MIS2, nullptr, C, nullptr, D, eqlinear_bwd_w_workspace_bytes(300, 5, 7, 4, F32),
                                 300, 5, 7, 4, F32, 1, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused_train(A, B, nullptr, MIS, C, nullptr, D, ws, 300, 5, 7, 4, F16, 1, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused_train(A, B, nullptr, nullptr, C, MIS, D, ws, 300, 5, 7, 4, F16, 1, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused_train(MIS, B, nullptr, nullptr, C, nullptr, D, wf, 300, 8, 8, 4, F16, 1, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fwd_fused_train(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 5, 7, 4, F16, 1,
                                 nullptr) == EQL_OK);
  CHECK(eqlinear_bwd_x_train(A, B, C, D, ws - 1, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_x_train(A, B, C, nullptr, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_x_train(A, B, C, MIS, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_bwd_x_train(MIS, B, C, D, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_bwd_x_train(MIS, B, C, D, wf, 300, 8, 8, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_bwd_x_train(nullptr, nullptr, nullptr, nullptr, 0, 0, 5, 7, 4, F16, nullptr) == EQL_OK);
  CHECK(eqlinear_bwd_w_train(B, C, D, ws - 1, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w_train(B, nullptr, D, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w_train(B, C, nullptr, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_bwd_w_train(B, C, MIS, ws, 300, 5, 7, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_bwd_w_train(nullptr, C, D, wf, 300, 8, 8, 4, F16, nullptr) == EQL_EINVAL);  // fused: dy read
  CHECK(eqlinear_bwd_w_train(MIS, C, D, wf, 300, 8, 8, 4, F16, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_bwd_w_train(B, C, D, ws, 300, 5, 7, 4, 3, nullptr) == EQL_EINVAL);
  // Epilogue backward, with and without a workspace.
  const size_t es = eqlinear_fused_epilogue_bwd_workspace_bytes(300, 5, 4, F16);
  CHECK(es == 19u * 20 * 4);
  CHECK(eqlinear_fused_epilogue_bwd(A, B, C, D, A, es, 300, 5, 4, F16, 3, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fused_epilogue_bwd(A, nullptr, C, D, A, es, 300, 5, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fused_epilogue_bwd(A, B, C, D, A, es - 1, 300, 5, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fused_epilogue_bwd(A, B, C, D, nullptr, es, 300, 5, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fused_epilogue_bwd(MIS, B, C, D, A, es, 300, 5, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fused_epilogue_bwd(A, B, C, MIS2, A, es, 300, 5, 4, F32, EQL_ACT_NONE, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fused_epilogue_bwd(A, B, C, D, A, es, 300, 5, 17, F16, EQL_ACT_GELU, nullptr) ==
        EQL_EUNSUPPORTED);
  CHECK(eqlinear_fused_epilogue_bwd_noalloc(A, B, C, D, 300, 5, 4, F16, 3, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fused_epilogue_bwd_noalloc(A, nullptr, C, D, 300, 5, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EINVAL);
  CHECK(eqlinear_fused_epilogue_bwd_noalloc(MIS, B, C, D, 300, 5, 4, F16, EQL_ACT_GELU, nullptr) == EQL_EALIGN);
  CHECK(eqlinear_fused_epilogue_bwd_noalloc(A, B, C, D, int64_t{1} << 21, 1024, 4, F16, EQL_ACT_NONE, nullptr) ==
        EQL_ESCRATCH);
  CHECK(eqlinear_fused_epilogue_bwd_noalloc(A, B, C, D, INT64_MAX, 1024, 4, F16, EQL_ACT_NONE, nullptr) ==
        EQL_EINVAL);
  // p4m weight expansion and gradient fold (the C_4 view's size rules).
  for (auto fn : {eqlinear_p4m_expand_weight, eqlinear_p4m_fold_weight_grad}) {
    CHECK(fn(A, B, 4, 4, 7, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, 0, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, 4, INT64_MIN, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, INT64_MAX, 4, F32, nullptr) == EQL_EINVAL);
    CHECK(fn(A, B, 4, (int64_t{1} << 20) + 1, F32, nullptr) == EQL_EINVAL);
    CHECK(fn(nullptr, B, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(A, nullptr, 4, 4, F16, nullptr) == EQL_EINVAL);
    CHECK(fn(MIS, B, 4, 4, F16, nullptr) == EQL_EALIGN);
  }
}

}  // namespace

int main() {
  sizes();
  validation();
  std::printf("abi_check: %d checks, %d failed\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}

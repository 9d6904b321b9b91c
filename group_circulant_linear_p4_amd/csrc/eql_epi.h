// Backward of the fused forward epilogue, y = act(pre) + residual with
// pre = x W^T + bias (the transformer MLP-block epilogue of "Nivel de Rede" in
// "Resumo Tecnico: Flash EQ-Linear"):
//   dpre[n][d*T+g] = dy[n][d*T+g] * act'(pre[n][d*T+g])    (act' = 1 without activation)
//   dbias[d]       = sum over n and g of dpre[n][d*T+g]
// The input and weight gradients of the layer then follow from the input-gradient and
// weight-gradient kernels applied to dpre; the residual's gradient is dy itself.
#pragma once

#include "eql_device.h"
#include "eql_fwd.h"

namespace eql {

struct EpiBwdArgs {
  const void* dy;    // [N][Dp*T]
  const void* pre;   // [N][Dp*T] (read only with an activation)
  void* dpre;        // [N][Dp*T] (may be dy)
  float* part;       // [rowBlocks][Dp] fp32 bias partials, or null (no bias gradient)
  void* dbias;       // [Dp]
  int N, Dp, act, chBlocks, rowBlocks;
};

constexpr int kEpiRows = 256;  // rows per workgroup
constexpr int kEpiCh = 64;     // output channels per workgroup

// GELU'(v) = Phi(v) + v phi(v), phi the standard normal density, in fp32 (erf as in
// the forward; exp(-v^2/2) through the hardware exp2).
__device__ __forceinline__ float gelu_grad(float v) {
  const float cdf = 0.5f * (1.0f + erf_as(v * 0.7071067811865475f));
  const float pdf = 0.3989422804014327f * __builtin_amdgcn_exp2f((-0.7213475204444817f * v) * v);
  return __builtin_fmaf(v, pdf, cdf);
}

// Workgroup (channel block, row block): 64 channels x 4 row lanes; lane (c, l) takes
// channel c's T group elements in rows l, l+4, ... of the block.  The four lanes'
// bias sums are added in a fixed order.
template <int T, typename Elt>
__global__ void __launch_bounds__(256) eql_epi_bwd_kernel(const EpiBwdArgs a) {
  __shared__ float red[4][kEpiCh];
  const int ch = threadIdx.x % kEpiCh, rl = threadIdx.x / kEpiCh;
  const int cb = blockIdx.x % a.chBlocks, rb = blockIdx.x / a.chBlocks;
  const int d = cb * kEpiCh + ch;
  const int r0 = rb * kEpiRows, r1 = min(a.N, r0 + kEpiRows);
  const size_t rowElems = (size_t)a.Dp * T;
  float s = 0.0f;
  if (d < a.Dp) {
    for (int r = r0 + rl; r < r1; r += 4) {
      const size_t at = (size_t)r * rowElems + (size_t)d * T;
      float g[T], o[T];
      load_group<T, Elt>(static_cast<const Elt*>(a.dy) + at, g);
      if (a.act == 1) {
        float p[T];
        load_group<T, Elt>(static_cast<const Elt*>(a.pre) + at, p);
#pragma unroll
        for (int e = 0; e < T; ++e) o[e] = g[e] * gelu_grad(p[e]);
      } else {
#pragma unroll
        for (int e = 0; e < T; ++e) o[e] = g[e];
      }
      store_group<T, Elt>(static_cast<Elt*>(a.dpre) + at, o);
#pragma unroll
      for (int e = 0; e < T; ++e) s += o[e];
    }
  }
  if (a.part) {
    red[rl][ch] = s;
    __syncthreads();
    if (rl == 0 && d < a.Dp) a.part[(size_t)rb * a.Dp + d] = ((red[0][ch] + red[1][ch]) + red[2][ch]) + red[3][ch];
  }
}

// dbias[d]: the row blocks' partials added in order, rounded once.
template <typename Elt>
__global__ void __launch_bounds__(256) eql_epi_bias_kernel(const EpiBwdArgs a) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= a.Dp) return;
  float s = 0.0f;
  for (int rb = 0; rb < a.rowBlocks; ++rb) s += a.part[(size_t)rb * a.Dp + d];
  static_cast<Elt*>(a.dbias)[d] = (Elt)s;
}

}  // namespace eql

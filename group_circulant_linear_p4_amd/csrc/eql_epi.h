// Backward of the fused forward epilogue, y = act(pre) + residual with
// pre = x W^T + bias (the transformer MLP-block epilogue of "Nivel de Rede" in
// "Resumo Tecnico: Flash EQ-Linear"):
//   dpre[n][d*T+g] = dy[n][d*T+g] * act'(pre[n][d*T+g])    (act' = 1 without activation)
//   dbias[d]       = sum over n and g of dpre[n][d*T+g]
// The input and weight gradients of the layer then follow from the input-gradient and
// weight-gradient kernels applied to dpre; the residual's gradient is dy itself.
//
// The first part is elementwise, so the kernel streams each row as a flat array in
// chunks of W bytes (the widest power of two, up to 16, dividing the row), with no
// regard to group boundaries.  The bias sum is kept per element position: each
// workgroup writes the column sums of its row block, and the bias kernel adds, for
// channel d, the T positions d*T .. d*T+T-1 of every row block in a fixed order.
#pragma once

#include "eql_device.h"
#include "eql_fwd.h"

namespace eql {

struct EpiBwdArgs {
  const void* dy;    // [N][Dp*T]
  const void* pre;   // [N][Dp*T] (read only with an activation)
  void* dpre;        // [N][Dp*T] (may be dy)
  float* part;       // [rowBlocks][Dp*T] fp32 column sums, or null (no bias gradient)
  void* dbias;       // [Dp]
  int N, Dp, T, act;
  int rowElems;      // Dp*T
  int rowsPerBlock;  // rows of one workgroup (a multiple of 4)
  int chunkBlocks;   // workgroups across a row (64 chunks each)
  int rowBlocks;
};

// GELU'(v) = Phi(v) + v phi(v), phi the standard normal density, in fp32.  exp(-v^2/2)
// serves both phi and the erf of Phi (erf(v/sqrt 2) needs exp(-(v/sqrt 2)^2)).
__device__ __forceinline__ float gelu_grad(float v) {
  const float e = __builtin_amdgcn_exp2f((-0.7213475204444817f * v) * v);  // exp(-v^2/2)
  const float cdf = __builtin_fmaf(0.5f, erf_as_e(v * 0.7071067811865475f, e), 0.5f);
  return __builtin_fmaf(v, 0.3989422804014327f * e, cdf);
}

// W bytes at p as 32-bit words (W = 2: the low half of one word).
template <int W>
__device__ __forceinline__ void load_chunk(const char* p, uint32_t (&w)[W >= 4 ? W / 4 : 1]) {
  if constexpr (W == 16) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    w[0] = q[0]; w[1] = q[1]; w[2] = q[2]; w[3] = q[3];
  } else if constexpr (W == 8) {
    const u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    w[0] = q[0]; w[1] = q[1];
  } else if constexpr (W == 4) {
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else {
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
  }
}

template <int W>
__device__ __forceinline__ void store_chunk(char* p, const uint32_t (&w)[W >= 4 ? W / 4 : 1]) {
  if constexpr (W == 16) {
    __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(p));
  } else if constexpr (W == 8) {
    __builtin_nontemporal_store((u32x2){w[0], w[1]}, reinterpret_cast<u32x2*>(p));
  } else if constexpr (W == 4) {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
  } else {
    __builtin_nontemporal_store((uint16_t)w[0], reinterpret_cast<uint16_t*>(p));
  }
}

template <typename Elt, int W>
__device__ __forceinline__ float chunk_elt(const uint32_t (&w)[W >= 4 ? W / 4 : 1], int e) {
  if constexpr (sizeof(Elt) == 4) return __builtin_bit_cast(float, w[e]);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e / 2] >> ((e & 1) * 16)));
}

// V values rounded to Elt into the chunk's words (fp16 pairs in one packed
// round-to-nearest-even conversion).
template <typename Elt, int W>
__device__ __forceinline__ void pack_chunk(const float (&d)[W / sizeof(Elt)], uint32_t (&w)[W >= 4 ? W / 4 : 1]) {
  constexpr int V = W / (int)sizeof(Elt);
  if constexpr (sizeof(Elt) == 4) {
#pragma unroll
    for (int v = 0; v < V; ++v) w[v] = __builtin_bit_cast(uint32_t, d[v]);
  } else if constexpr (V == 1) {
    w[0] = __builtin_bit_cast(uint16_t, (_Float16)d[0]);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      const h2 pr = {(_Float16)d[2 * i], (_Float16)d[2 * i + 1]};
      w[i] = __builtin_bit_cast(uint32_t, pr);
    }
  }
}

// Workgroup (chunk block cb, row block rb): lane c of each wave takes chunk
// cb*64 + c of the rows; wave l takes rows l, l+4, ... of the block, four at a
// time so that eight loads are in flight per lane.  The four waves' column sums
// are added in a fixed order.
template <typename Elt, int W>
__global__ void __launch_bounds__(256) eql_epi_bwd_kernel(const EpiBwdArgs a) {
  constexpr int V = W / (int)sizeof(Elt);  // elements per chunk
  constexpr int NWD = W >= 4 ? W / 4 : 1;  // words per chunk
  constexpr int U = 4;                     // rows per iteration and wave
  __shared__ float red[3][V][64];
  const int lane = (int)threadIdx.x & 63, wv = (int)threadIdx.x >> 6;
  const int cb = (int)blockIdx.x % a.chunkBlocks, rb = (int)blockIdx.x / a.chunkBlocks;
  const int chunk = cb * 64 + lane;
  const bool live = chunk < a.rowElems / V;
  // Row indices in 64 bits: N may come within a block of 2^31.
  const int64_t r0 = (int64_t)rb * a.rowsPerBlock, r1 = min((int64_t)a.N, r0 + a.rowsPerBlock);
  const size_t rowBytes = (size_t)a.rowElems * sizeof(Elt);
  const size_t colOff = (size_t)chunk * W;
  const bool gelu = a.act == 1;
  // Without an activation, dpre written over dy would rewrite the same values: skip it.
  const bool store = gelu || a.dpre != a.dy;
  float s[V];
#pragma unroll
  for (int v = 0; v < V; ++v) s[v] = 0.0f;

  // dpre in fp32, rounded once when stored; the bias sums take the fp32 values.
  auto row_step = [&](const uint32_t (&g)[NWD], const uint32_t (&p)[NWD], size_t off) __attribute__((always_inline)) {
    float d[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      d[v] = chunk_elt<Elt, W>(g, v);
      if (gelu) d[v] *= gelu_grad(chunk_elt<Elt, W>(p, v));
      s[v] += d[v];
    }
    if (store) {
      uint32_t o[NWD];
      pack_chunk<Elt, W>(d, o);
      store_chunk<W>(static_cast<char*>(a.dpre) + off, o);
    }
  };

  if (live) {
    const char* dy = static_cast<const char*>(a.dy);
    const char* pre = static_cast<const char*>(a.pre);
    int64_t r = r0 + wv;
    for (; r + 4 * (U - 1) < r1; r += 4 * U) {
      uint32_t g[U][NWD], p[U][NWD];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t off = (size_t)(r + 4 * u) * rowBytes + colOff;
        load_chunk<W>(dy + off, g[u]);
        if (gelu) load_chunk<W>(pre + off, p[u]);
        else
#pragma unroll
          for (int i = 0; i < NWD; ++i) p[u][i] = 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) row_step(g[u], p[u], (size_t)(r + 4 * u) * rowBytes + colOff);
    }
    for (; r < r1; r += 4) {
      const size_t off = (size_t)r * rowBytes + colOff;
      uint32_t g[NWD], p[NWD];
      load_chunk<W>(dy + off, g);
      if (gelu) load_chunk<W>(pre + off, p);
      else
#pragma unroll
        for (int i = 0; i < NWD; ++i) p[i] = 0;
      row_step(g, p, off);
    }
  }
  if (a.part) {
    if (wv > 0) {
#pragma unroll
      for (int v = 0; v < V; ++v) red[wv - 1][v][lane] = s[v];
    }
    __syncthreads();
    if (wv == 0 && live) {
      float* out = a.part + (size_t)rb * a.rowElems + (size_t)chunk * V;
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = ((s[v] + red[0][v][lane]) + red[1][v][lane]) + red[2][v][lane];
    }
  }
}

// dbias[d] from the row blocks' column sums.  A workgroup takes 16 channels x 16
// slices of the row blocks: slice l adds blocks l, l+16, l+32, ... in that order
// (each block's T positions in order, four blocks' loads in flight), and the 16
// slice sums of a channel are then added in slice order; rounded once to Elt.
template <int T, typename Elt>
__global__ void __launch_bounds__(256) eql_epi_bias_kernel(const EpiBwdArgs a) {
  __shared__ float red[16][16];
  const int c = (int)threadIdx.x & 15, sl = (int)threadIdx.x >> 4;
  const int d = (int)blockIdx.x * 16 + c;
  float s = 0.0f;
  if (d < a.Dp) {
    const float* p = a.part + (size_t)d * T;
    const size_t stride = (size_t)a.rowElems;
    auto block_sum = [&](int rb) __attribute__((always_inline)) {
      float v[T];
#pragma unroll
      for (int g = 0; g < T; ++g) v[g] = p[(size_t)rb * stride + g];
      float t = v[0];
#pragma unroll
      for (int g = 1; g < T; ++g) t += v[g];
      return t;
    };
    int rb = sl;
    for (; rb + 48 < a.rowBlocks; rb += 64) {
      const float t0 = block_sum(rb), t1 = block_sum(rb + 16), t2 = block_sum(rb + 32), t3 = block_sum(rb + 48);
      s = (((s + t0) + t1) + t2) + t3;
    }
    for (; rb < a.rowBlocks; rb += 16) s += block_sum(rb);
  }
  red[sl][c] = s;
  __syncthreads();
  if (sl == 0 && d < a.Dp) {
    float tot = red[0][c];
#pragma unroll
    for (int l = 1; l < 16; ++l) tot += red[l][c];
    static_cast<Elt*>(a.dbias)[d] = (Elt)tot;
  }
}

}  // namespace eql

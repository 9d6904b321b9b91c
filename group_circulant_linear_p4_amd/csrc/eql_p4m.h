// The equivariant layer over p4m's point group (dihedral D4: four rotations r^a and four
// reflections r^a s) evaluated as a C_4 layer on twice the channels.
//
// "Resumo Tecnico: Flash EQ-Linear" names other transformation groups, reflection groups
// among them, as future work ("Limitacoes e Trabalho Futuro"); the layer here keeps its
// construction: one set of shared parameters w[d][c][j], j over the 8 group elements,
// replicated into W[(d,g),(c,h)] = w[d][c][g h^-1].  The group axis lists r^0..r^3, then
// the reflections r^-m s for m = 0..3.  With that order a channel's 8 values are two
// channels of 4 values (its rotation half and its reflection half), and each of the four
// half-to-half blocks of W is a circular convolution along Z_4:
//     rotations   -> rotations  : kernel w(r^k)        (k = g - h on the half's index)
//     reflections -> rotations  : kernel w(r^k s)
//     rotations   -> reflections: kernel w(r^-k s)
//     reflections -> reflections: kernel w(r^-k)
// So the p4m layer with C' in and D' out channels is exactly the C_4 layer with 2C' in,
// 2D' out channels and the tied weight w4[2d+bo][2c+bi][k] built from those kernels, on
// the same memory layout of x and y.  eql_p4m_expand_kernel builds w4 (a gather); the C_4
// kernels do the rest; eql_p4m_fold_kernel turns the C_4 weight gradient into the p4m one
// (each parameter is tied into exactly two entries of w4).
#pragma once

#include "eql_device.h"

namespace eql {

struct P4mArgs {
  const void* src;
  void* dst;
  int Dp, Cp;
};

// Index in w's group axis of r^a s^b.
__device__ __forceinline__ int p4m_index(int a, int b) {
  a &= 3;
  return b == 0 ? a : 4 + ((-a) & 3);
}

// Thread per (d, c, bo, bi) of w4: its 4 values w4[2d+bo][2c+bi][0..3].
template <typename Elt>
__global__ void __launch_bounds__(256) eql_p4m_expand_kernel(const P4mArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.Dp * a.Cp * 4;
  if (t >= total) return;
  const int bi = (int)(t & 1), bo = (int)((t >> 1) & 1);
  const int64_t dc = t >> 2;
  const int64_t d = dc / a.Cp, c = dc - d * a.Cp;
  const Elt* w = static_cast<const Elt*>(a.src) + dc * 8;
  Elt* out = static_cast<Elt*>(a.dst) + ((2 * d + bo) * (2 * (int64_t)a.Cp) + 2 * c + bi) * 4;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // (bo, bi) = (0,0): r^k; (0,1): r^k s; (1,0): r^-k s; (1,1): r^-k.
    const int rot = bo == 0 ? k : -k;
    out[k] = w[p4m_index(rot, bo ^ bi)];
  }
}

// Thread per (d, c, j): dw[d][c][j] = the sum, in fp32 and rounded once, of the two
// entries of the C_4 gradient dw4 that parameter j is tied into.
template <typename Elt>
__global__ void __launch_bounds__(256) eql_p4m_fold_kernel(const P4mArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.Dp * a.Cp * 8;
  if (t >= total) return;
  const int j = (int)(t & 7);
  const int64_t dc = t >> 3;
  const int64_t d = dc / a.Cp, c = dc - d * a.Cp;
  const Elt* g = static_cast<const Elt*>(a.src);
  const int64_t C2 = 2 * (int64_t)a.Cp;
  auto at = [&](int bo, int bi, int k) { return (float)g[((2 * d + bo) * C2 + 2 * c + bi) * 4 + (k & 3)]; };
  float v;
  if (j < 4) {
    v = at(0, 0, j) + at(1, 1, -j);           // r^j as w4[0][0][k = j] and w4[1][1][k = -j]
  } else {
    const int m = j - 4;                      // element r^-m s
    v = at(0, 1, -m) + at(1, 0, m);           // w4[0][1][k] = w(r^k s), w4[1][0][k] = w(r^-k s)
  }
  static_cast<Elt*>(a.dst)[t] = (Elt)v;
}

}  // namespace eql

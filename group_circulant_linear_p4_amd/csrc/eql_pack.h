// Packing of the shared weight into its half spectrum along the group axis
// ("Abordagem Algoritmica" in "Resumo Tecnico: Flash EQ-Linear": the Fourier-domain
// products need the DFT of w, and conjugate symmetry keeps half of it).
//
// One thread per (out, in) pair of the packed matrix (plus the zero padding of both
// axes: output channels to a multiple of 32, input channels to the padded group
// count).  It reads the T shared parameters,
// transforms them in fp32 (p4: butterflies only), divides each plane by its share
// of the inverse transform's scale and rounds it once to the element type.  In the input-gradient mode the weight is the transposed,
// group-reversed w~[c][d][t] = w[d][c][(-t) mod T]; its spectrum is the conjugate,
// so the Im planes change sign.  One launch may write both packings (PackArgs::wp2).
#pragma once

#include "eql_device.h"

namespace eql {

struct PackArgs {
  const void* w;    // [Dp][Cp][T]
  void* wp;         // packed: packed_unit(o, i / G, p) * G + i % G
  int Dp, Cp, outCh, inCh, Jin, transposed;
  Twiddles tw;
  // Both packings in one launch: workgroups from blocks1 on write the input-gradient
  // packing (transposed) into wp2, whose input axis has Jin2 groups; 0 = one packing.
  void* wp2;
  int Jin2, blocks1;
};

// Output channels per block of the packed weight.
constexpr int kPackBlock = 32;

// 16-byte unit of the packed weight holding input-channel group j of plane p for
// output channel o.  Output channels form blocks of 32; a block's data is one chunk of
// T * 64 units per K stage (two groups), and inside a chunk the units are ordered
// [plane][channel of the block][group of the stage, XOR bit 3 of the channel].  A
// forward kernel stage then reads each block as one contiguous T KB run, and the
// fragment reads of 16 consecutive channels land on distinct LDS bank groups.
__host__ __device__ inline size_t packed_unit(int o, int j, int p, int T, int stages) {
  const int ob = o / kPackBlock, ol = o % kPackBlock, s = j >> 1, jj = j & 1;
  return (((size_t)ob * stages + s) * T + p) * 64 + (size_t)ol * 2 + (jj ^ ((ol >> 3) & 1));
}

template <int T, typename Elt>
__global__ void __launch_bounds__(256) eql_pack_kernel(const PackArgs a) {
  constexpr int G = EltT<Elt>::kPerUnit;
  constexpr int NR = n_real_planes(T);
  const bool second = a.blocks1 > 0 && (int)blockIdx.x >= a.blocks1;
  const int transposed = second ? 1 : a.transposed;
  const int outCh = second ? a.inCh : a.outCh, inCh = second ? a.outCh : a.inCh;
  const int Jin = second ? a.Jin2 : a.Jin;
  const size_t idx = (size_t)((int)blockIdx.x - (second ? a.blocks1 : 0)) * 256 + threadIdx.x;
  const size_t row = (size_t)Jin * G;
  const int outPad = (outCh + kPackBlock - 1) / kPackBlock * kPackBlock;
  if (idx >= (size_t)outPad * row) return;
  const int o = (int)(idx / row);
  const int i = (int)(idx - (size_t)o * row);
  float pl[T];
#pragma unroll
  for (int p = 0; p < T; ++p) pl[p] = 0.0f;
  if (i < inCh && o < outCh) {
    const int d = transposed ? i : o;
    const int c = transposed ? o : i;
    float v[T];
    load_group<T, Elt>(static_cast<const Elt*>(a.w) + ((size_t)d * a.Cp + c) * T, v);
    Dft<T>::run(v, pl, a.tw);
    // The inverse transform's scale lives in the weight: 1/T on the real planes,
    // 2/T on the complex ones (one correctly rounded division; exact for
    // power-of-two T), so the kernels that consume the packing multiply by nothing.
#pragma unroll
    for (int p = 0; p < T; ++p) pl[p] = (p < NR ? pl[p] : 2.0f * pl[p]) / (float)T;
    if (transposed) {
#pragma unroll
      for (int p = NR + 1; p < T; p += 2) pl[p] = -pl[p];
    }
  }
  Elt* out = static_cast<Elt*>(second ? a.wp2 : a.wp);
#pragma unroll
  for (int p = 0; p < T; ++p) out[packed_unit(o, i / G, p, T, Jin / 2) * G + (i % G)] = (Elt)pl[p];
}

}  // namespace eql

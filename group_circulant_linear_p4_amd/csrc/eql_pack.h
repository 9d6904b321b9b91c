// Packing of the shared weight into its half spectrum along the group axis
// ("Abordagem Algoritmica" in "Resumo Tecnico: Flash EQ-Linear": the Fourier-domain
// products need the DFT of w, and conjugate symmetry keeps half of it).
//
// One thread per (out, in) pair of the packed matrix (plus the zero padding of the
// input axis up to the padded group count).  It reads the T shared parameters,
// transforms them in fp32 (p4: butterflies only), divides each plane by its share
// of the inverse transform's scale and rounds it once to the element type.  In the input-gradient mode the weight is the transposed,
// group-reversed w~[c][d][t] = w[d][c][(-t) mod T]; its spectrum is the conjugate,
// so the Im planes change sign.
#pragma once

#include "eql_device.h"

namespace eql {

struct PackArgs {
  const void* w;    // [Dp][Cp][T]
  void* wp;         // packed: ((o * Jin + i / G) * T + p) * G + i % G
  int Dp, Cp, outCh, inCh, Jin, transposed;
  Twiddles tw;
};

template <int T, typename Elt>
__global__ void __launch_bounds__(256) eql_pack_kernel(const PackArgs a) {
  constexpr int G = EltT<Elt>::kPerUnit;
  constexpr int NR = n_real_planes(T);
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = (size_t)a.Jin * G;
  if (idx >= (size_t)a.outCh * row) return;
  const int o = (int)(idx / row);
  const int i = (int)(idx - (size_t)o * row);
  float pl[T];
#pragma unroll
  for (int p = 0; p < T; ++p) pl[p] = 0.0f;
  if (i < a.inCh) {
    const int d = a.transposed ? i : o;
    const int c = a.transposed ? o : i;
    float v[T];
    load_group<T, Elt>(static_cast<const Elt*>(a.w) + ((size_t)d * a.Cp + c) * T, v);
    Dft<T>::run(v, pl, a.tw);
    // The inverse transform's scale lives in the weight: 1/T on the real planes,
    // 2/T on the complex ones (one correctly rounded division; exact for
    // power-of-two T), so the kernels that consume the packing multiply by nothing.
#pragma unroll
    for (int p = 0; p < T; ++p) pl[p] = (p < NR ? pl[p] : 2.0f * pl[p]) / (float)T;
    if (a.transposed) {
#pragma unroll
      for (int p = NR + 1; p < T; p += 2) pl[p] = -pl[p];
    }
  }
  Elt* out = static_cast<Elt*>(a.wp) + (((size_t)o * a.Jin + i / G) * T) * G + (i % G);
#pragma unroll
  for (int p = 0; p < T; ++p) out[p * G] = (Elt)pl[p];
}

}  // namespace eql

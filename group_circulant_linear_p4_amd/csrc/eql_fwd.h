// Fused forward kernel of the EQ-Linear layer: y = x W^T evaluated as
// group DFT (prologue) -> per-frequency channel GEMMs on MFMA -> inverse DFT
// (epilogue), with no intermediate global writes ("Implementacao" in "Resumo
// Tecnico: Flash EQ-Linear": fused data flow, Fourier fragments kept in registers
// and shared memory).  The input-gradient pass runs the same kernel on the
// conjugate-transposed packed weight.
//
// Work decomposition (gfx950, wave64):
//   * a workgroup is 4 waves and owns 128 rows x BN = 32*NB output channels, for
//     all T planes;
//   * each wave owns 32 rows.  Its lanes load x straight into MFMA A-operand
//     order: lane l takes row l%32 and one 16-byte channel group (G channels, all
//     T group elements: 16*T contiguous bytes), runs the group DFT in fp32
//     registers and rounds once to the element type.  x never goes through LDS;
//   * the packed spectrum of w for the workgroup's BN channels is staged through
//     double-buffered LDS (one 16-byte unit per (channel, group, plane), rows
//     padded to an odd number of units so the 16-byte MFMA B-operand reads are
//     bank-conflict free) and shared by the 4 waves;
//   * per k-step and 32-column block: real planes take one MFMA, each complex
//     plane pair four (Re += Xr Wr + (-Xi) Wi, Im += Xi Wr + Xr Wi; the chains are
//     ordered so that the p4 path is exactly shift-equivariant);
//   * the epilogue reads the T accumulators of one (row, channel) from the same
//     register slot, applies the inverse DFT and stores T contiguous outputs;
//     adjacent lanes write adjacent channels.
#pragma once

#include "eql_device.h"

namespace eql {

struct FwdArgs {
  const void* x;    // [N][Cin*T]
  const void* wp;   // packed spectrum, out = Dout, in = Cin
  void* y;          // [N][Dout*T]
  int N, Cin, Dout, Jtot, colTiles, numTiles, aligned16;
  Twiddles tw;
};

constexpr int kFwdRows = 128;  // rows per workgroup (4 waves x 32)

template <int T, typename Elt, int NB, int JC>
__global__ void __launch_bounds__(256) eql_fwd_kernel(const FwdArgs a) {
  using E = EltT<Elt>;
  constexpr int G = E::kPerUnit;        // channels per 16-byte group
  constexpr int NR = n_real_planes(T);
  constexpr int NP = n_pairs(T);
  constexpr int KS = JC / 2;            // k-steps per chunk (two groups per k-step)
  constexpr int BN = 32 * NB;
  constexpr int ROWU = JC * T;          // LDS units per output channel per chunk
  constexpr int PITCH = ROWU + 1;       // odd: conflict-free 16-byte reads
  constexpr int UNITS = BN * ROWU;
  constexpr int UPT = (UNITS + 255) / 256;
  constexpr int WPR = 4 * T;            // 32-bit words of raw x per lane per k-step
  static_assert(JC % 2 == 0, "two channel groups per k-step");

  __shared__ u32x4 lds[2][BN * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, khalf = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, a.numTiles);
  const int rowTile = tile / a.colTiles, colTile = tile - rowTile * a.colTiles;
  const int row0 = rowTile * kFwdRows, col0 = colTile * BN;
  const int myRow = row0 + wave * 32 + lrow;
  const bool rowOk = myRow < a.N;
  const Elt* __restrict__ xrow =
      static_cast<const Elt*>(a.x) + (size_t)(rowOk ? myRow : 0) * (size_t)a.Cin * T;
  const u32x4* __restrict__ wp = static_cast<const u32x4*>(a.wp);
  const int nch = (a.Jtot + JC - 1) / JC;

  f32x16 acc[T][NB];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[p][nb][r] = 0.0f;

  uint32_t raw[KS][WPR];
  u32x4 af[KS][T + NP];
  u32x4 bst[UPT];

  // Raw x of chunk `ch` for this lane: k-step s covers channel group
  // ch*JC + 2s + khalf (G channels x T elements, contiguous).
  auto load_x = [&](int ch) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int cfirst = (ch * JC + 2 * s + khalf) * G;
      const Elt* src = xrow + (size_t)cfirst * T;
      if (a.aligned16) {
#pragma unroll
        for (int v = 0; v < T; ++v) {
          const int chv = cfirst + (v * G) / T;  // channel of the unit's first element
          u32x4 val = {0u, 0u, 0u, 0u};
          if (rowOk && chv < a.Cin) val = *reinterpret_cast<const u32x4*>(src + v * G);
          raw[s][4 * v + 0] = val[0];
          raw[s][4 * v + 1] = val[1];
          raw[s][4 * v + 2] = val[2];
          raw[s][4 * v + 3] = val[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < WPR; ++i) raw[s][i] = 0u;
#pragma unroll
        for (int e = 0; e < G * T; ++e) {
          if (rowOk && cfirst + e / T < a.Cin) {
            if constexpr (sizeof(Elt) == 2) {
              const uint32_t hv = *reinterpret_cast<const uint16_t*>(src + e);
              raw[s][e / 2] |= (e & 1) ? (hv << 16) : hv;
            } else {
              raw[s][e] = *reinterpret_cast<const uint32_t*>(src + e);
            }
          }
        }
      }
    }
  };

  // Group DFT of the raw chunk into A-operand units (one per plane, plus the
  // negated Im planes used by the real part of the complex products).
  auto transform = [&]() {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float pl[T][G];
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float v[T], o[T];
#pragma unroll
        for (int h = 0; h < T; ++h) {
          const int i = e * T + h;
          if constexpr (sizeof(Elt) == 2) {
            const uint16_t bits = (uint16_t)(raw[s][i / 2] >> ((i & 1) * 16));
            v[h] = (float)__builtin_bit_cast(_Float16, bits);
          } else {
            v[h] = __builtin_bit_cast(float, raw[s][i]);
          }
        }
        Dft<T, true>::run(v, o, a.tw);
#pragma unroll
        for (int p = 0; p < T; ++p) pl[p][e] = o[p];
      }
#pragma unroll
      for (int p = 0; p < T; ++p) af[s][p] = E::pack(pl[p]);
#pragma unroll
      for (int q = 0; q < NP; ++q) af[s][T + q] = neg_unit(af[s][NR + 2 * q + 1], E::kSignMask);
    }
  };

  auto load_b = [&](int ch) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      const int o = u / ROWU, r = u - o * ROWU;
      const int jj = r / T, p = r - jj * T;
      const int og = col0 + o, jg = ch * JC + jj;
      u32x4 val = {0u, 0u, 0u, 0u};
      if ((UNITS % 256 == 0 || u < UNITS) && og < a.Dout && jg < a.Jtot)
        val = wp[((size_t)og * a.Jtot + jg) * T + p];
      bst[i] = val;
    }
  };

  auto store_b = [&](int buf) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      if (UNITS % 256 == 0 || u < UNITS) {
        const int o = u / ROWU, r = u - o * ROWU;
        lds[buf][o * PITCH + r] = bst[i];
      }
    }
  };

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4* bsrc = &lds[buf][(nb * 32 + lrow) * PITCH + (2 * s + khalf) * T];
        u32x4 bf[T];
#pragma unroll
        for (int p = 0; p < T; ++p) bf[p] = bsrc[p];
#pragma unroll
        for (int p = 0; p < NR; ++p) E::mfma(acc[p][nb], af[s][p], bf[p]);
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const int re = NR + 2 * q, im = re + 1;
          E::mfma(acc[re][nb], af[s][re], bf[re]);
          E::mfma(acc[re][nb], af[s][T + q], bf[im]);
          E::mfma(acc[im][nb], af[s][im], bf[re]);
          E::mfma(acc[im][nb], af[s][re], bf[im]);
        }
      }
    }
  };

  if (nch > 0) {
    load_x(0);
    load_b(0);
    store_b(0);
    transform();
  }
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const bool more = ch + 1 < nch;
    if (more) {
      load_x(ch + 1);
      load_b(ch + 1);
    }
    compute(ch & 1);
    if (more) {
      store_b((ch + 1) & 1);
      transform();
    }
    __syncthreads();
  }

  // Epilogue: accumulator slot r of lane l holds row 8*(r/4) + 4*(l/32) + r%4 and
  // column l%32 of each 32x32 block.
  Elt* __restrict__ yout = static_cast<Elt*>(a.y);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = col0 + nb * 32 + lrow;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + wave * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      if (row < a.N && col < a.Dout) {
        float P[T], yv[T];
#pragma unroll
        for (int p = 0; p < T; ++p) P[p] = acc[p][nb][r];
        Idft<T, false>::run(P, yv, a.tw);
        store_group<T, Elt>(yout + ((size_t)row * a.Dout + col) * T, yv);
      }
    }
  }
}

}  // namespace eql

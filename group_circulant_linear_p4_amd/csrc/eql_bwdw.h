// Weight-gradient kernels of the EQ-Linear layer.
//
// dw[d][c][t] = sum_n sum_g dy[n][d][g] x[n][c][(g-t) mod T].  In the Fourier
// domain this is, per frequency k, G_k[d][c] = sum_n dY_k[n][d] conj(X_k[n][c]):
// one channel GEMM per plane with the reduction running over the N rows.  Real
// planes take one real product; a complex pair takes four:
//     Re G = dYr Xr + dYi Xi,      Im G = dYi Xr - dYr Xi.
// Kernel 1 (eql_bwdw_kernel) splits the N rows into S ranges and writes one fp32
// partial spectrum per range into the workspace.  Kernel 2 (eql_bwdw_reduce) sums
// the S partials in a fixed order (deterministic), applies the inverse group
// transform and rounds to the element type.
//
// Work decomposition of kernel 1 (gfx950, wave64): a workgroup owns 128 output
// channels d (4 waves x 32) and BN = 32*NB input channels c for one row range.
//   * A operand (dY): lane l of a wave takes channel d = l%32 and G consecutive
//     rows (the MFMA k index runs over rows), loads each row's T group values
//     (adjacent lanes read adjacent channels: coalesced), runs the group DFT in
//     registers and rounds once.  No LDS.
//   * B operand (X): produced the same way by all 256 threads for the
//     workgroup's BN channels and shared through double-buffered LDS, laid out
//     [k-step][plane][row half][channel] so both the writes and the 16-byte MFMA
//     reads are bank-conflict free.
#pragma once

#include "eql_device.h"

namespace eql {

struct BwdwArgs {
  const void* x;    // [N][Cp*T]
  const void* dy;   // [N][Dp*T]
  float* ws;        // [S][T][Dp][Cp] fp32 partial spectra
  int N, Cp, Dp, rowsPerSplit, cTiles, dTiles, numTiles;
  Twiddles tw;
};

struct BwdwReduceArgs {
  const float* ws;  // [S][T][Dp][Cp]
  void* dw;         // [Dp][Cp][T]
  int S, Dp, Cp;
  Twiddles tw;
};

constexpr int kBwdwRowsD = 128;  // output channels d per workgroup

template <int T, typename Elt, int NB, int KSC>
__global__ void __launch_bounds__(256) eql_bwdw_kernel(const BwdwArgs a) {
  using E = EltT<Elt>;
  constexpr int G = E::kPerUnit;       // rows per lane per k-step
  constexpr int KR = 2 * G;            // rows per k-step
  constexpr int CH = KSC * KR;         // rows per chunk
  constexpr int NR = n_real_planes(T);
  constexpr int NP = n_pairs(T);
  constexpr int BN = 32 * NB;
  constexpr int ITEMS = KSC * 2 * BN;  // producer items per chunk: (k-step, half, c)
  constexpr int IPT = (ITEMS + 255) / 256;
  constexpr int GB = T * (int)sizeof(Elt);  // bytes of one (row, channel) group vector
  constexpr int GW = (GB + 3) / 4;          // its 32-bit words
  constexpr int LOADW = pow2_part(GB);

  __shared__ u32x4 lds[2][KSC * T * 2 * BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lcol = lane & 31, khalf = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, a.numTiles);
  const int per = a.dTiles * a.cTiles;
  const int split = tile / per;
  const int rest = tile - split * per;
  const int dTile = rest / a.cTiles, cTile = rest - dTile * a.cTiles;
  const int d0 = dTile * kBwdwRowsD, c0 = cTile * BN;
  const int rb = split * a.rowsPerSplit;
  const int re = min(a.N, rb + a.rowsPerSplit);
  const int nch = re > rb ? (re - rb + CH - 1) / CH : 0;

  const int myD = d0 + wave * 32 + lcol;
  const bool dOk = myD < a.Dp;
  const Elt* __restrict__ dyp = static_cast<const Elt*>(a.dy);
  const Elt* __restrict__ xp = static_cast<const Elt*>(a.x);

  f32x16 acc[T][NB];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[p][nb][r] = 0.0f;

  uint32_t araw[KSC][G][GW];
  uint32_t braw[IPT][G][GW];
  u32x4 af[KSC][T + NP];

  auto load_vec = [&](const Elt* src, uint32_t (&w)[GW]) {
#pragma unroll
    for (int i = 0; i < GW; ++i) w[i] = 0u;
    if constexpr (LOADW >= 4) {
#pragma unroll
      for (int b = 0; b < GB; b += LOADW) load_bytes<LOADW>(reinterpret_cast<const char*>(src) + b, &w[b / 4]);
    } else {
#pragma unroll
      for (int e = 0; e < T; ++e) {
        const uint32_t hv = *reinterpret_cast<const uint16_t*>(src + e);
        w[e / 2] |= (e & 1) ? (hv << 16) : hv;
      }
    }
  };
  auto zero_vec = [&](uint32_t (&w)[GW]) {
#pragma unroll
    for (int i = 0; i < GW; ++i) w[i] = 0u;
  };
  auto to_float = [&](const uint32_t (&w)[GW], float (&v)[T]) {
#pragma unroll
    for (int e = 0; e < T; ++e) {
      if constexpr (sizeof(Elt) == 2) {
        const uint16_t bits = (uint16_t)(w[e / 2] >> ((e & 1) * 16));
        v[e] = (float)__builtin_bit_cast(_Float16, bits);
      } else {
        v[e] = __builtin_bit_cast(float, w[e]);
      }
    }
  };

  auto load_chunk = [&](int ch) {
    const int base = rb + ch * CH;
#pragma unroll
    for (int s = 0; s < KSC; ++s)
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const int n = base + s * KR + khalf * G + e;
        if (dOk && n < re) load_vec(dyp + ((size_t)n * a.Dp + myD) * T, araw[s][e]);
        else zero_vec(araw[s][e]);
      }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + 256 * i;
      const int c = it % BN, sh = it / BN;
      const int half = sh & 1, s = sh >> 1;
      const int cg = c0 + c;
      const bool ok = (ITEMS % 256 == 0 || it < ITEMS) && cg < a.Cp;
#pragma unroll
      for (int e = 0; e < G; ++e) {
        const int n = base + s * KR + half * G + e;
        if (ok && n < re) load_vec(xp + ((size_t)n * a.Cp + cg) * T, braw[i][e]);
        else zero_vec(braw[i][e]);
      }
    }
  };

  // DFT of the raw rows into A units (registers) and B units (LDS buffer `buf`).
  auto transform = [&](int buf) {
#pragma unroll
    for (int s = 0; s < KSC; ++s) {
      float pl[T][G];
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float v[T], o[T];
        to_float(araw[s][e], v);
        Dft<T, true>::run(v, o, a.tw);
#pragma unroll
        for (int p = 0; p < T; ++p) pl[p][e] = o[p];
      }
#pragma unroll
      for (int p = 0; p < T; ++p) af[s][p] = E::pack(pl[p]);
      // Negated Re planes: Im G = dYi Xr + (-dYr) Xi.
#pragma unroll
      for (int q = 0; q < NP; ++q) af[s][T + q] = neg_unit(af[s][NR + 2 * q], E::kSignMask);
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + 256 * i;
      if (ITEMS % 256 == 0 || it < ITEMS) {
        const int c = it % BN, sh = it / BN;
        const int half = sh & 1, s = sh >> 1;
        float pl[T][G];
#pragma unroll
        for (int e = 0; e < G; ++e) {
          float v[T], o[T];
          to_float(braw[i][e], v);
          Dft<T, true>::run(v, o, a.tw);
#pragma unroll
          for (int p = 0; p < T; ++p) pl[p][e] = o[p];
        }
#pragma unroll
        for (int p = 0; p < T; ++p) lds[buf][((s * T + p) * 2 + half) * BN + c] = E::pack(pl[p]);
      }
    }
  };

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < KSC; ++s) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        u32x4 bf[T];
#pragma unroll
        for (int p = 0; p < T; ++p) bf[p] = lds[buf][((s * T + p) * 2 + khalf) * BN + nb * 32 + lcol];
#pragma unroll
        for (int p = 0; p < NR; ++p) E::mfma(acc[p][nb], af[s][p], bf[p]);
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const int rp = NR + 2 * q, ip = rp + 1;
          E::mfma(acc[rp][nb], af[s][rp], bf[rp]);
          E::mfma(acc[rp][nb], af[s][ip], bf[ip]);
          E::mfma(acc[ip][nb], af[s][ip], bf[rp]);
          E::mfma(acc[ip][nb], af[s][T + q], bf[ip]);
        }
      }
    }
  };

  if (nch > 0) {
    load_chunk(0);
    transform(0);
  }
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const bool more = ch + 1 < nch;
    if (more) load_chunk(ch + 1);
    compute(ch & 1);
    if (more) transform((ch + 1) & 1);
    __syncthreads();
  }

  // Partial spectrum of this row range: slot r of lane l is output channel
  // d = 8*(r/4) + 4*(l/32) + r%4 (MFMA rows) and input channel c = l%32.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = c0 + nb * 32 + lcol;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = d0 + wave * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      if (d < a.Dp && c < a.Cp) {
#pragma unroll
        for (int p = 0; p < T; ++p)
          a.ws[(((size_t)split * T + p) * a.Dp + d) * a.Cp + c] = acc[p][nb][r];
      }
    }
  }
}

template <int T, typename Elt>
__global__ void __launch_bounds__(256) eql_bwdw_reduce(const BwdwReduceArgs a) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t plane = (size_t)a.Dp * a.Cp;
  if (idx >= plane) return;
  float P[T];
#pragma unroll
  for (int p = 0; p < T; ++p) P[p] = 0.0f;
  for (int s = 0; s < a.S; ++s) {
#pragma unroll
    for (int p = 0; p < T; ++p) P[p] += a.ws[((size_t)s * T + p) * plane + idx];
  }
  float g[T];
  Idft<T, true>::run(P, g, a.tw);
  store_group<T, Elt>(static_cast<Elt*>(a.dw) + idx * T, g);
}

}  // namespace eql

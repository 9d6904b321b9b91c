// Weight-gradient kernels of the EQ-Linear layer.
//
// dw[d][c][t] = sum_n sum_g dy[n][d][g] x[n][c][(g-t) mod T].  In the Fourier
// domain, per frequency k, G_k[d][c] = sum_n dY_k[n][d] conj(X_k[n][c]): one channel
// GEMM per plane with the reduction over the N rows (the gradient of the pointwise
// products of "Abordagem Algoritmica" in "Resumo Tecnico: Flash EQ-Linear").  Real
// planes take one real product; a complex pair takes four:
//     Re G = dYr Xr + dYi Xi,      Im G = dYi Xr - dYr Xi.
//
// Three kernels:
//   1. eql_spec_kernel: the group DFT of x and of dy, once per element, rounded once
//      to the element type and stored in the workspace as MFMA operand units: unit
//      (kg, p, half, k) holds plane p of channel k for the G rows
//      kg*2G + half*G .. +G (G = 16 / sizeof(element); rows past N are zero).
//      Layout [kg][p][half][k], so the units one k-step of a channel tile needs
//      form 2T contiguous runs.  Purely bandwidth bound.
//   2. eql_bwdw_gemm: the per-plane GEMMs.  A workgroup owns 128 output channels d
//      (4 waves x 32) by BN = 32*NB input channels c for one range of k-steps;
//      both operands stream into NS-deep LDS rings by buffer->LDS loads, so the
//      loop body is LDS reads and MFMAs only.  It writes one fp32 partial spectrum
//      per row range into the workspace.
//   3. eql_bwdw_reduce: sums the partials in a fixed order (deterministic), applies
//      the inverse group transform and rounds to the element type.
#pragma once

#include <type_traits>

#include "eql_device.h"
#include "eql_dma.h"

namespace eql {

struct SpecArgs {
  const void* m;    // [N][K*T]
  void* out;        // units [kgCount][T][2][K]
  int N, K, kgCount;
  Twiddles tw;
};

struct BwdwArgs {
  const void* dyh;  // dY units [kgCount][T][2][Dp]
  const void* xh;   // X units  [kgCount][T][2][Cp]
  float* ws;        // [S][T][Dp][Cp] fp32 partial spectra
  int Dp, Cp, kgCount, kgPerSplit, dTiles, cTiles, numItems;
};

struct BwdwReduceArgs {
  const float* ws;  // [S][T][Dp][Cp]
  void* dw;         // [Dp][Cp][T]
  int S, Dp, Cp;
  Twiddles tw;
};

constexpr int kBwdwRowsD = 128;  // output channels d per workgroup (4 waves x 32)

template <int T, typename Elt>
__global__ void __launch_bounds__(256) eql_spec_kernel(const SpecArgs a) {
  using E = EltT<Elt>;
  constexpr int G = E::kPerUnit;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)a.kgCount * 2 * a.K;
  if (idx >= total) return;
  const int k = (int)(idx % a.K);
  const size_t rest = idx / a.K;
  const int half = (int)(rest & 1);
  const int kg = (int)(rest >> 1);
  const int row0 = kg * 2 * G + half * G;
  float pl[T][G];
#pragma unroll
  for (int e = 0; e < G; ++e) {
    float v[T], o[T];
    const int row = row0 + e;
    if (row < a.N) {
      load_group<T, Elt>(static_cast<const Elt*>(a.m) + ((size_t)row * a.K + k) * T, v);
    } else {
#pragma unroll
      for (int h = 0; h < T; ++h) v[h] = 0.0f;
    }
    Dft<T, false>::run(v, o, a.tw);
#pragma unroll
    for (int p = 0; p < T; ++p) pl[p][e] = o[p];
  }
  u32x4* out = static_cast<u32x4*>(a.out);
#pragma unroll
  for (int p = 0; p < T; ++p) out[(((size_t)kg * T + p) * 2 + half) * a.K + k] = E::pack(pl[p]);
}

template <int T, typename Elt, int NB>
__global__ void __launch_bounds__(256) eql_bwdw_gemm(const BwdwArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using E = EltT<Elt>;
  constexpr int NR = n_real_planes(T);
  constexpr int NP = n_pairs(T);
  constexpr int BN = 32 * NB;
  constexpr int UA = 2 * T * kBwdwRowsD;   // A units per stage (one k-step)
  constexpr int UB = 2 * T * BN;           // B units per stage
  // ... padded to whole loads of 4 waves x 64 lanes
  constexpr int UAP = (UA + 255) / 256 * 256, UBP = (UB + 255) / 256 * 256;
  constexpr int NS = ((UAP + UBP) * 16 * 4 <= 160 * 1024) ? 4 : (((UAP + UBP) * 16 * 3 <= 160 * 1024) ? 3 : 2);
  constexpr int DIST = NS - 1;
  constexpr int IPWA = UAP / 256, IPWB = UBP / 256;  // DMA loads per wave per stage
  constexpr int WAIT_TOP = (DIST - 1) * (IPWA + IPWB);
  static_assert(NS * (UAP + UBP) * 16 <= 160 * 1024, "LDS budget");
  static_assert(WAIT_TOP < 64, "vmcnt range");

  __shared__ u32x4 ringA[NS][UAP];
  __shared__ u32x4 ringB[NS][UBP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lcol = lane & 31, khalf = lane >> 5;
  const int item = xcd_remap(blockIdx.x, a.numItems);
  const int per = a.dTiles * a.cTiles;
  const int split = item / per;
  const int rest = item - split * per;
  const int dTile = rest / a.cTiles, cTile = rest - dTile * a.cTiles;
  const int d0 = dTile * kBwdwRowsD, c0 = cTile * BN;
  const int kgBegin = split * a.kgPerSplit;
  const int kgEnd = min(a.kgCount, kgBegin + a.kgPerSplit);
  const int nst = max(0, kgEnd - kgBegin);

  // DMA source offsets within a stage block (unit P of the block is run
  // s = P / width, element j = P % width, i.e. global unit (kg*2T + s)*K + k0 + j).
  // Units past K read neighbouring data that only reaches output channels that are
  // never stored; the descriptor range keeps every access inside the buffer.
  uint32_t aOff[IPWA], bOff[IPWB];
#pragma unroll
  for (int i = 0; i < IPWA; ++i) {
    const int P = (wave * IPWA + i) * 64 + lane;
    const int s = P / kBwdwRowsD, j = P - s * kBwdwRowsD;
    aOff[i] = P < UA ? ((uint32_t)s * a.Dp + (uint32_t)(d0 + j)) * 16u : 0u;  // padding: any unit
  }
#pragma unroll
  for (int i = 0; i < IPWB; ++i) {
    const int P = (wave * IPWB + i) * 64 + lane;
    const int s = P / BN, j = P - s * BN;
    bOff[i] = P < UB ? ((uint32_t)s * a.Cp + (uint32_t)(c0 + j)) * 16u : 0u;
  }
  const uint64_t aBase = reinterpret_cast<uint64_t>(a.dyh), bBase = reinterpret_cast<uint64_t>(a.xh);
  const uint64_t aStage = (uint64_t)2 * T * a.Dp * 16, bStage = (uint64_t)2 * T * a.Cp * 16;
  const uint64_t aTotal = aStage * a.kgCount, bTotal = bStage * a.kgCount;

  // Stage j of this item (k-step kgBegin + j) into ring slot j % NS.  Stages past
  // the item read nothing (empty range), so every stage issues the same loads.
  auto issue = [&](int j) __attribute__((always_inline)) {
    const bool live = j < nst;
    const uint64_t kg = (uint64_t)(kgBegin + (live ? j : 0));
    {
      const uint64_t base = aBase + kg * aStage;
      const uint64_t left = aTotal - kg * aStage;
      const BufDesc d = desc_at(base, live ? (uint32_t)min(left, (uint64_t)0xFFFFFFF0u) : 0u);
      const uint32_t dst = lds_addr(&ringA[j % NS][wave * IPWA * 64]);
#pragma unroll
      for (int i = 0; i < IPWA; ++i) dma16(d, aOff[i], dst + i * 1024u);
    }
    {
      const uint64_t base = bBase + kg * bStage;
      const uint64_t left = bTotal - kg * bStage;
      const BufDesc d = desc_at(base, live ? (uint32_t)min(left, (uint64_t)0xFFFFFFF0u) : 0u);
      const uint32_t dst = lds_addr(&ringB[j % NS][wave * IPWB * 64]);
#pragma unroll
      for (int i = 0; i < IPWB; ++i) dma16(d, bOff[i], dst + i * 1024u);
    }
  };

  f32x16 acc[T][NB];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[p][nb][r] = 0.0f;

  // Pipeline: stage j is loaded DIST stages ahead, at the top of stage j - DIST,
  // into the slot of stage j - DIST - 1 (free once every wave passed that stage's
  // barrier).  At the top of stage j, the loads issued after it are those of
  // stages j+1 .. j+DIST-1: WAIT_TOP of them may still be outstanding.
#pragma unroll
  for (int j = 0; j < DIST; ++j) issue(j);

  for (int j = 0; j < nst; ++j) {
    wait_vmcnt<WAIT_TOP>();
    __builtin_amdgcn_s_barrier();
    issue(j + DIST);
    const u32x4* sa = ringA[j % NS];
    const u32x4* sb = ringB[j % NS];
    u32x4 af[T + NP];
#pragma unroll
    for (int p = 0; p < T; ++p) af[p] = sa[(p * 2 + khalf) * kBwdwRowsD + wave * 32 + lcol];
    // -dYr for Im G = dYi Xr + (-dYr) Xi.
#pragma unroll
    for (int q = 0; q < NP; ++q) af[T + q] = neg_unit(af[NR + 2 * q], E::kSignMask);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      u32x4 bf[T];
#pragma unroll
      for (int p = 0; p < T; ++p) bf[p] = sb[(p * 2 + khalf) * BN + nb * 32 + lcol];
#pragma unroll
      for (int p = 0; p < NR; ++p) E::mfma(acc[p][nb], af[p], bf[p]);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int rp = NR + 2 * q, ip = rp + 1;
        E::mfma(acc[rp][nb], af[rp], bf[rp]);
        E::mfma(acc[rp][nb], af[ip], bf[ip]);
        E::mfma(acc[ip][nb], af[ip], bf[rp]);
        E::mfma(acc[ip][nb], af[T + q], bf[ip]);
      }
    }
  }
  wait_vmcnt<0>();  // drain the look-ahead loads before the LDS is reused

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
#endif  // __HIP_DEVICE_COMPILE__
}

// Sum of the split partials, then the inverse group transform.  Both operands were
// transformed without scaling, so the inverse is the plain one:
//   dw[t] = (1/T) (G0 + (-1)^t G_{T/2} + 2 sum_k (cos Re G_k - sin Im G_k)).
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

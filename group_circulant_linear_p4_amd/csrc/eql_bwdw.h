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
//      kg*2G + half*G .. +G (G = 16 / sizeof(element); rows past N and channels
//      past the padded width are zero).  Channels are cut into tiles of the GEMM's
//      tile width W, layout [kg][k / W][p][half][k % W], so the units one k-step of
//      one channel tile needs are one contiguous block.  Purely bandwidth bound.
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
  void* out;        // units [kgCount][kTiles][T][2][W]
  int N, K, kgCount, W, kTiles;
  Twiddles tw;
};

struct BwdwArgs {
  const void* dyh;  // dY units [kgCount][dTiles][T][2][128]
  const void* xh;   // X units  [kgCount][cTiles][T][2][32 NB]
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
  const size_t width = (size_t)a.kTiles * a.W;  // padded channel count
  if (idx >= (size_t)a.kgCount * 2 * width) return;
  const int k = (int)(idx % width);
  const size_t rest = idx / width;
  const int half = (int)(rest & 1);
  const int kg = (int)(rest >> 1);
  const int row0 = kg * 2 * G + half * G;
  float pl[T][G];
#pragma unroll
  for (int e = 0; e < G; ++e) {
    float v[T], o[T];
    const int row = row0 + e;
    if (row < a.N && k < a.K) {
      load_group<T, Elt>(static_cast<const Elt*>(a.m) + ((size_t)row * a.K + k) * T, v);
    } else {
#pragma unroll
      for (int h = 0; h < T; ++h) v[h] = 0.0f;
    }
    Dft<T, false>::run(v, o, a.tw);
#pragma unroll
    for (int p = 0; p < T; ++p) pl[p][e] = o[p];
  }
  const int kt = k / a.W, kk = k - kt * a.W;
  u32x4* out = static_cast<u32x4*>(a.out) + (((size_t)kg * a.kTiles + kt) * T * 2 + half) * a.W + kk;
#pragma unroll
  for (int p = 0; p < T; ++p) out[(size_t)p * 2 * a.W] = E::pack(pl[p]);
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
  constexpr int IPWA = UAP / 256, IPWB = UBP / 256;  // DMA loads per wave per stage
  constexpr int IPW = IPWA + IPWB;
  // Register double buffering of the operand fragments (next k-step read from LDS
  // while this one's MFMAs run) when two fragment sets fit beside the address
  // registers; otherwise one set, read after the barrier of its own k-step.
  constexpr bool PIPE = 2 * (T + NB * T) * 4 <= 192;
  static_assert(NS * (UAP + UBP) * 16 <= 160 * 1024, "LDS budget");
  static_assert((NS - 1) * IPW < 64, "vmcnt range");

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

  // A stage block (one k-step of one channel tile) is contiguous in the workspace
  // and lands in the ring in the same order: unit P of the block at slot unit P.
  // Padding units of the last wave load (UBP > UB) re-read unit 0.
  uint32_t aOff[IPWA], bOff[IPWB];
#pragma unroll
  for (int i = 0; i < IPWA; ++i) {
    const int P = (wave * IPWA + i) * 64 + lane;
    aOff[i] = P < UA ? (uint32_t)P * 16u : 0u;
  }
#pragma unroll
  for (int i = 0; i < IPWB; ++i) {
    const int P = (wave * IPWB + i) * 64 + lane;
    bOff[i] = P < UB ? (uint32_t)P * 16u : 0u;
  }
  const uint64_t aBase = reinterpret_cast<uint64_t>(a.dyh) + (uint64_t)dTile * UA * 16;
  const uint64_t bBase = reinterpret_cast<uint64_t>(a.xh) + (uint64_t)cTile * UB * 16;
  const uint64_t aStage = (uint64_t)a.dTiles * UA * 16, bStage = (uint64_t)a.cTiles * UB * 16;

  // Stage j of this item (k-step kgBegin + j) into ring slot j % NS.  Stages past
  // the item read nothing (empty range), so every stage issues the same loads.
  // Loads 0 .. IPWA-1 fill the A block, IPWA .. IPW-1 the B block.
  struct StageDesc {
    BufDesc da, db;
    uint32_t dsta, dstb;
  };
  auto stage_desc = [&](int j) __attribute__((always_inline)) {
    const bool live = j < nst;
    const uint64_t kg = (uint64_t)(kgBegin + (live ? j : 0));
    StageDesc sd;
    sd.da = desc_at(aBase + kg * aStage, live ? (uint32_t)(UA * 16) : 0u);
    sd.db = desc_at(bBase + kg * bStage, live ? (uint32_t)(UB * 16) : 0u);
    sd.dsta = lds_addr(&ringA[j % NS][wave * IPWA * 64]);
    sd.dstb = lds_addr(&ringB[j % NS][wave * IPWB * 64]);
    return sd;
  };
  auto issue_one = [&](const StageDesc& sd, int i) __attribute__((always_inline)) {
    if (i < IPWA)
      dma16(sd.da, aOff[i], sd.dsta + i * 1024u);
    else
      dma16(sd.db, bOff[i - IPWA], sd.dstb + (i - IPWA) * 1024u);
  };
  auto issue = [&](int j) __attribute__((always_inline)) {
    const StageDesc sd = stage_desc(j);
#pragma unroll
    for (int i = 0; i < IPW; ++i) issue_one(sd, i);
  };

  f32x16 acc[T][NB];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[p][nb][r] = 0.0f;

  // Operand fragments of one k-step: lane (lcol, khalf) holds plane p of output
  // channel d0 + 32*wave + lcol (A) / input channel c0 + 32*nb + lcol (B) for rows
  // khalf*G .. +G of the step.
  struct Frags {
    u32x4 a[T];
    u32x4 b[NB][T];
  };
  auto read_frags = [&](int j, Frags& f) __attribute__((always_inline)) {
    const u32x4* sa = ringA[j % NS];
    const u32x4* sb = ringB[j % NS];
#pragma unroll
    for (int p = 0; p < T; ++p) f.a[p] = sa[(p * 2 + khalf) * kBwdwRowsD + wave * 32 + lcol];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int p = 0; p < T; ++p) f.b[nb][p] = sb[(p * 2 + khalf) * BN + nb * 32 + lcol];
  };
  // MFMAs of one k-step.  With `sd` given, the IPW loads of a later stage are issued
  // between them, one after every MFMAS / IPW MFMAs: issue is in order, so a burst
  // of loads would hold the MFMAs back until the address unit had taken every one
  // of them.  The scheduling barriers keep that order.
  constexpr int MFMAS = NB * (NR + 4 * NP);
  constexpr int EVERY = MFMAS / IPW > 0 ? MFMAS / IPW : 1;
  auto mma = [&](const Frags& f, const StageDesc* sd) __attribute__((always_inline)) {
    // -dYr for Im G = dYi Xr + (-dYr) Xi.
    u32x4 negr[NP > 0 ? NP : 1];
#pragma unroll
    for (int q = 0; q < NP; ++q) negr[q] = neg_unit(f.a[NR + 2 * q], E::kSignMask);
    int m = 0, ld = 0;
    auto after_mfma = [&]() __attribute__((always_inline)) {
      ++m;
      if (sd && m % EVERY == 0 && ld < IPW) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one(*sd, ld++);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int p = 0; p < NR; ++p) {
        E::mfma(acc[p][nb], f.a[p], f.b[nb][p]);
        after_mfma();
      }
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int rp = NR + 2 * q, ip = rp + 1;
        E::mfma(acc[rp][nb], f.a[rp], f.b[nb][rp]);
        after_mfma();
        E::mfma(acc[rp][nb], f.a[ip], f.b[nb][ip]);
        after_mfma();
        E::mfma(acc[ip][nb], f.a[ip], f.b[nb][rp]);
        after_mfma();
        E::mfma(acc[ip][nb], negr[q], f.b[nb][ip]);
        after_mfma();
      }
    }
    if (sd) {
#pragma unroll
      for (; ld < IPW; ++ld) issue_one(*sd, ld);
    }
  };

  if constexpr (PIPE) {
    // Slot j % NS holds stage j; it is refilled with stage j + NS at the top of
    // k-step j, once every wave has its fragments of stage j in registers (its LDS
    // reads returned: lgkmcnt(0) before the barrier).  At that point the loads
    // issued after stage j+1 are those of stages j+2 .. j+NS-1.
#pragma unroll
    for (int j = 0; j < NS; ++j) issue(j);
    wait_vmcnt<(NS - 1) * IPW>();
    __builtin_amdgcn_s_barrier();
    Frags f0, f1;
    read_frags(0, f0);
    auto step = [&](int j, const Frags& cur, Frags& nxt) __attribute__((always_inline)) {
      wait_vmcnt<(NS - 2) * IPW>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      const StageDesc sd = stage_desc(j + NS);
      read_frags(j + 1, nxt);
      mma(cur, &sd);
    };
    int j = 0;
    for (; j + 1 < nst; j += 2) {
      step(j, f0, f1);
      step(j + 1, f1, f0);
    }
    if (j < nst) step(j, f0, f1);
  } else {
    // Stage j is loaded NS-1 stages ahead, at the top of stage j-NS+1, into the
    // slot of stage j-NS (free once every wave passed that stage's barrier).  At
    // the top of stage j the loads issued after it are those of stages
    // j+1 .. j+NS-2.
    constexpr int DIST = NS - 1;
#pragma unroll
    for (int j = 0; j < DIST; ++j) issue(j);
    for (int j = 0; j < nst; ++j) {
      wait_vmcnt<(DIST - 1) * IPW>();
      __builtin_amdgcn_s_barrier();
      issue(j + DIST);
      Frags f;
      read_frags(j, f);
      mma(f, nullptr);
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

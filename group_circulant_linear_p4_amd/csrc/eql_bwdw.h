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
//      past the channel count are zero).  Layout [kg][p][half][Kpad] with the channel
//      axis padded to a multiple of the GEMM tile width, so a tile's units of one
//      k-step are 2 or 4 contiguous runs.  Purely bandwidth bound.
//   2. eql_bwdw_gemm<T, Elt, PAIR, DB, CB, WCN>: the per-frequency GEMMs, one plane
//      group per workgroup so that its output tile can be as large as the register
//      file allows: 2 x WCN waves, each with DB x CB blocks of 32 x 32 outputs per
//      plane (WCN = 2: one wave per SIMD; WCN = 4: two, each with half the columns).  For large channel counts a real plane takes a 256 (d) x
//      256 (c) tile and a complex pair a 256 x 128 tile of both planes (256
//      accumulator registers per lane either way); per MFMA that moves about
//      0.56-0.75x the operand bytes of a tile holding all T planes.  Narrow channel
//      axes take 64-wide tiles instead of padding to 256.  Both operands stream
//      into NS-deep LDS rings by buffer->LDS loads; the loop body is LDS reads and
//      MFMAs.  Each item writes the fp32 partial spectrum of one row range.
//   3. eql_bwdw_reduce: sums the partials in a fixed order (deterministic; with long
//      chains 4 or 16 phases of threads share the splits of 64 or 16 outputs, combined
//      in order), applies the inverse group transform and rounds to the element type.
#pragma once

#include <type_traits>

#include "eql_device.h"
#include "eql_dma.h"

namespace eql {

// Two matrices of N rows may share one launch: workgroups below `blocks1` transform
// (m, out, K, Kpad), the others (m2, out2, K2, Kpad2).
struct SpecArgs {
  const void* m;    // [N][K*T]
  void* out;        // units [kgCount][T][2][Kpad]
  int N, K, Kpad, kgCount;
  Twiddles tw;
  const void* m2;   // [N][K2*T] or null
  void* out2;       // units [kgCount][T][2][Kpad2]
  int K2, Kpad2, blocks1;
};

// One launch covers either every real plane (PAIR = false: planes 0 .. NR-1) or
// every complex pair (PAIR = true: planes NR .. T-1).
struct BwdwArgs {
  const void* dyh;  // dY units [kgCount][T][2][Dpad]
  const void* xh;   // X units  [kgCount][T][2][Cpad]
  float* ws;        // partials [S][planes of this launch][Dp][Cp]
  int Dp, Cp, Dpad, Cpad, kgCount, kgPerSplit, groups, dTiles, cTiles, numItems;
};

struct BwdwReduceArgs {
  const float* wsR;  // [SR][NR][Dp][Cp]
  const float* wsP;  // [SP][2 NP][Dp][Cp]
  void* dw;          // [Dp][Cp][T]
  int SR, SP, Dp, Cp;
  Twiddles tw;
};

template <int T, typename Elt>
__global__ void __launch_bounds__(256) eql_spec_kernel(const SpecArgs a) {
  using E = EltT<Elt>;
  constexpr int G = E::kPerUnit;
  const bool second = (int)blockIdx.x >= a.blocks1;
  const Elt* const m = static_cast<const Elt*>(second ? a.m2 : a.m);
  const int K = second ? a.K2 : a.K, Kpad = second ? a.Kpad2 : a.Kpad;
  const size_t idx = (size_t)((int)blockIdx.x - (second ? a.blocks1 : 0)) * 256 + threadIdx.x;
  if (idx >= (size_t)a.kgCount * 2 * Kpad) return;
  const int k = (int)(idx % Kpad);
  const size_t rest = idx / Kpad;
  const int half = (int)(rest & 1);
  const int kg = (int)(rest >> 1);
  const int row0 = kg * 2 * G + half * G;
  float pl[T][G];
#pragma unroll
  for (int e = 0; e < G; ++e) {
    float v[T], o[T];
    const int row = row0 + e;
    if (row < a.N && k < K) {
      load_group<T, Elt>(m + ((size_t)row * K + k) * T, v);
    } else {
#pragma unroll
      for (int h = 0; h < T; ++h) v[h] = 0.0f;
    }
    Dft<T>::run(v, o, a.tw);
#pragma unroll
    for (int p = 0; p < T; ++p) pl[p][e] = o[p];
  }
  // Non-temporal: the spectra are read back by the GEMMs only after the whole
  // transform, long after they would have left the caches.
  u32x4* out = static_cast<u32x4*>(second ? a.out2 : a.out) + ((size_t)kg * T * 2 + half) * Kpad + k;
#pragma unroll
  for (int p = 0; p < T; ++p) __builtin_nontemporal_store(E::pack(pl[p]), &out[(size_t)p * 2 * Kpad]);
}

template <int T, typename Elt, bool PAIR, int DB, int CB, int WCN>
__global__ void __launch_bounds__(128 * WCN) eql_bwdw_gemm(const BwdwArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using E = EltT<Elt>;
  constexpr int NR = n_real_planes(T);
  constexpr int NPL = PAIR ? 2 : 1;          // planes per item
  constexpr int WAVES = 2 * WCN;             // 2 x WCN waves
  constexpr int WD = 64 * DB;                // output channels d per workgroup
  constexpr int WC = 32 * CB * WCN;          // input channels c per workgroup
  constexpr int UA = NPL * 2 * WD;           // A units per stage (one k-step)
  constexpr int UB = NPL * 2 * WC;           // B units per stage
  // ... padded to whole loads of all waves x 64 lanes
  constexpr int LW = 64 * WAVES;
  constexpr int UAP = (UA + LW - 1) / LW * LW, UBP = (UB + LW - 1) / LW * LW;
  constexpr int NS = 4;
  constexpr int IPWA = UAP / LW, IPWB = UBP / LW;  // DMA loads per wave per stage
  constexpr int IPW = IPWA + IPWB;
  static_assert(NS * (UAP + UBP) * 16 <= 160 * 1024, "LDS budget");
  static_assert((NS - 1) * IPW < 64, "vmcnt range");

  __shared__ u32x4 ringA[NS][UAP];
  __shared__ u32x4 ringB[NS][UBP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wd = wave / WCN, wc = wave % WCN;  // 2 x WCN waves
  const int lcol = lane & 31, khalf = lane >> 5;
  const int item = xcd_remap(blockIdx.x, a.numItems);
  const int per = a.groups * a.dTiles * a.cTiles;
  const int split = item / per;
  int rest = item - split * per;
  const int grp = rest / (a.dTiles * a.cTiles);
  rest -= grp * (a.dTiles * a.cTiles);
  const int dTile = rest / a.cTiles, cTile = rest - dTile * a.cTiles;
  const int d0 = dTile * WD, c0 = cTile * WC;
  const int p0 = PAIR ? NR + 2 * grp : grp;  // first plane of the item
  const int kgBegin = split * a.kgPerSplit;
  const int kgEnd = min(a.kgCount, kgBegin + a.kgPerSplit);
  const int nst = max(0, kgEnd - kgBegin);

  // A stage is run s = plane*2 + half of the item's planes: A units d0 .. d0+WD-1
  // of that run, B units c0 .. c0+WC-1; unit P of the stage lands at ring unit P.
  // Padding positions of the last wave load (P >= UA or UB) re-read unit 0.
  uint32_t aOff[IPWA], bOff[IPWB];
#pragma unroll
  for (int i = 0; i < IPWA; ++i) {
    const int P = (wave * IPWA + i) * 64 + lane;
    const int s = P / WD, j = P - s * WD;
    aOff[i] = P < UA ? ((uint32_t)s * a.Dpad + (uint32_t)(d0 + j)) * 16u : 0u;
  }
#pragma unroll
  for (int i = 0; i < IPWB; ++i) {
    const int P = (wave * IPWB + i) * 64 + lane;
    const int s = P / WC, j = P - s * WC;
    bOff[i] = P < UB ? ((uint32_t)s * a.Cpad + (uint32_t)(c0 + j)) * 16u : 0u;
  }
  // Byte offset of k-step kg's first run, and the bytes the item's runs span.
  const uint64_t aBase = reinterpret_cast<uint64_t>(a.dyh), bBase = reinterpret_cast<uint64_t>(a.xh);
  const uint64_t aStep = (uint64_t)T * 2 * a.Dpad * 16, bStep = (uint64_t)T * 2 * a.Cpad * 16;
  const uint64_t aPlane = (uint64_t)p0 * 2 * a.Dpad * 16, bPlane = (uint64_t)p0 * 2 * a.Cpad * 16;
  const uint32_t aSpan = (uint32_t)NPL * 2 * a.Dpad * 16, bSpan = (uint32_t)NPL * 2 * a.Cpad * 16;

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
    sd.da = desc_at(aBase + kg * aStep + aPlane, live ? aSpan : 0u);
    sd.db = desc_at(bBase + kg * bStep + bPlane, live ? bSpan : 0u);
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

  f32x16 acc[NPL][DB][CB];
#pragma unroll
  for (int q = 0; q < NPL; ++q)
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int jc = 0; jc < CB; ++jc)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][i][jc][r] = 0.0f;

  // Operand fragments of one k-step: lane (lcol, khalf) holds plane q of output
  // channel d0 + (WD/2)*wd + 32*i + lcol (A) / input channel c0 + (WC/WCN)*wc + 32*jc
  // + lcol (B) for rows khalf*G .. +G of the step.
  struct Frags {
    u32x4 a[NPL][DB];
    u32x4 b[NPL][CB];
  };
  auto read_frags = [&](int j, Frags& f) __attribute__((always_inline)) {
    const u32x4* sa = ringA[j % NS];
    const u32x4* sb = ringB[j % NS];
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
#pragma unroll
      for (int i = 0; i < DB; ++i) f.a[q][i] = sa[(q * 2 + khalf) * WD + wd * (WD / 2) + i * 32 + lcol];
#pragma unroll
      for (int jc = 0; jc < CB; ++jc) f.b[q][jc] = sb[(q * 2 + khalf) * WC + wc * (WC / WCN) + jc * 32 + lcol];
    }
  };

  // MFMAs of one k-step, with the IPW loads of a later stage issued between them,
  // one after every MFMAS / IPW MFMAs (issue is in order: a burst of loads would
  // hold the MFMAs back until the address unit had taken every one of them).
  constexpr int MFMAS = DB * CB * (PAIR ? 4 : 1);
  constexpr int EVERY = MFMAS / IPW > 0 ? MFMAS / IPW : 1;
  auto mma = [&](const Frags& f, const StageDesc& sd) __attribute__((always_inline)) {
    int m = 0, ld = 0;
    auto after_mfma = [&]() __attribute__((always_inline)) {
      ++m;
      if (m % EVERY == 0 && ld < IPW) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one(sd, ld++);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      u32x4 negr;
      if constexpr (PAIR) negr = neg_unit(f.a[0][i], E::kSignMask);  // -dYr
#pragma unroll
      for (int jc = 0; jc < CB; ++jc) {
        if constexpr (PAIR) {
          E::mfma(acc[0][i][jc], f.a[0][i], f.b[0][jc]);  // Re += dYr Xr
          after_mfma();
          E::mfma(acc[0][i][jc], f.a[1][i], f.b[1][jc]);  //    + dYi Xi
          after_mfma();
          E::mfma(acc[1][i][jc], f.a[1][i], f.b[0][jc]);  // Im += dYi Xr
          after_mfma();
          E::mfma(acc[1][i][jc], negr, f.b[1][jc]);       //    - dYr Xi
          after_mfma();
        } else {
          E::mfma(acc[0][i][jc], f.a[0][i], f.b[0][jc]);
          after_mfma();
        }
      }
    }
#pragma unroll
    for (; ld < IPW; ++ld) issue_one(sd, ld);
  };

  // Slot j % NS holds stage j; it is refilled with stage j + NS at the top of
  // k-step j, once every wave has its fragments of stage j in registers (its LDS
  // reads returned: lgkmcnt(0) before the barrier).  At that point the loads
  // issued after stage j+1 are those of stages j+2 .. j+NS-1.
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const StageDesc sd = stage_desc(j);
#pragma unroll
    for (int i = 0; i < IPW; ++i) issue_one(sd, i);
  }
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
    mma(cur, sd);
  };
  int j = 0;
  for (; j + 1 < nst; j += 2) {
    step(j, f0, f1);
    step(j + 1, f1, f0);
  }
  if (j < nst) step(j, f0, f1);
  wait_vmcnt<0>();  // drain the look-ahead loads before the LDS is reused

  // Partial spectrum of this row range: slot r of lane l in block (i, jc) is output
  // channel d = 8*(r/4) + 4*(l/32) + r%4 (MFMA rows) and input channel c = l%32 of
  // the block.
  const int planes = PAIR ? 2 * n_pairs(T) : NR;
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    const int pidx = PAIR ? 2 * grp + q : grp;
    float* out = a.ws + ((size_t)split * planes + pidx) * a.Dp * a.Cp;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int jc = 0; jc < CB; ++jc) {
        const int c = c0 + wc * (WC / WCN) + jc * 32 + lcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = d0 + wd * (WD / 2) + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          if (d < a.Dp && c < a.Cp) out[(size_t)d * a.Cp + c] = acc[q][i][jc][r];
        }
      }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Sum of the split partials, then the inverse group transform.  WAVES = 1: one
// output per thread, all splits in one chain.  WAVES = 4 or 16 (for long chains):
// a workgroup covers 256 / WAVES consecutive (d, c) outputs, and the threads of
// phase w sum splits w, w + WAVES, ... for them (adjacent threads read adjacent
// outputs); the first phase adds the other phases' sums in a fixed order.  Either
// way the order depends only on the shape, so the result does not depend on
// timing.  Both operands were transformed
// without scaling, so the inverse is the plain one,
//   dw[t] = (1/T) (G0 + (-1)^t G_{T/2} + 2 sum_k (cos Re G_k - sin Im G_k)),
// followed by one rounding to the element type.
template <int T, typename Elt, int WAVES>
__global__ void __launch_bounds__(256) eql_bwdw_reduce(const BwdwReduceArgs a) {
  constexpr int NR = n_real_planes(T);
  constexpr int NC = T - NR;  // planes of the complex pairs
  constexpr int OUTS = 256 / WAVES;
  __shared__ float part[WAVES > 1 ? WAVES - 1 : 1][T][OUTS];
  const int lane = threadIdx.x % OUTS, w = threadIdx.x / OUTS;
  const size_t idx = (size_t)blockIdx.x * OUTS + lane;
  const size_t plane = (size_t)a.Dp * a.Cp;
  const bool live = idx < plane;
  float P[T];
#pragma unroll
  for (int p = 0; p < T; ++p) P[p] = 0.0f;
  if (live) {
    for (int s = w; s < a.SR; s += WAVES) {
#pragma unroll
      for (int p = 0; p < NR; ++p) P[p] += a.wsR[((size_t)s * NR + p) * plane + idx];
    }
    if constexpr (NC > 0) {
      for (int s = w; s < a.SP; s += WAVES) {
#pragma unroll
        for (int p = 0; p < NC; ++p) P[NR + p] += a.wsP[((size_t)s * NC + p) * plane + idx];
      }
    }
  }
  if constexpr (WAVES > 1) {
    if (w > 0) {
#pragma unroll
      for (int p = 0; p < T; ++p) part[w - 1][p][lane] = P[p];
    }
    __syncthreads();
    if (w == 0 && live) {
#pragma unroll
      for (int v = 0; v < WAVES - 1; ++v)
#pragma unroll
        for (int p = 0; p < T; ++p) P[p] += part[v][p][lane];
    }
  }
  if (w == 0 && live) {
    float g[T];
    Idft<T, true>::run(P, g, a.tw);
    store_group<T, Elt>(static_cast<Elt*>(a.dw) + idx * T, g);
  }
}

// Phases per output group of the reduce, from the loads one thread would chain
// (splits x planes) and the number of outputs: sharing the chain pays only when it
// is long (c5: 32 loads, one phase), and 16 phases give small layers with long
// chains enough workgroups to fill the chip (the C8 layer with 64 x 64 channels:
// 4096 outputs and 766 loads, 256 workgroups instead of 64).
__host__ __device__ constexpr int reduce_waves(int64_t chain, int64_t outputs) {
  return chain < 64 ? 1 : (chain >= 256 && outputs / 64 < 256 ? 16 : 4);
}

}  // namespace eql

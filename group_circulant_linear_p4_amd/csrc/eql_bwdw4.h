// Weight-gradient kernel with the group transform of dy fused into the GEMM, for
// T in {1, 2, 4} and 16-byte-aligned dy rows (the layers whose weight gradient is
// bound by HBM traffic rather than MFMA throughput).
//
// dw's spectrum per frequency is G_k[d][c] = sum_n dY_k[n][d] conj(X_k[n][c]) (the
// gradient of the pointwise products of "Abordagem Algoritmica" in "Resumo Tecnico:
// Flash EQ-Linear").  The separate path (eql_bwdw.h) first writes the spectra of x and
// dy to memory and reads them back.  Here only x's spectrum is pre-computed (the
// smaller operand in these layers); dy streams raw through an LDS ring, and each
// wave forms its dY operand fragments in registers from transposed LDS reads (G rows
// of one output channel per lane), with the same butterflies as the forward kernel.
// dy is thus read once from memory and its spectrum is never written ("Implementacao":
// fused data flow, no intermediate global writes).
//
// Work decomposition: an item is a 128 (d) x 32 NB (c) output tile for all T planes
// (NB = 2, 3 or 4, the width that pads C' least) and one range of k-steps (split-K
// over the rows); one workgroup of 4 waves per item, wave w owning output channels
// d0 + 32w .. +31 and all NB 32-channel blocks of c.  A k-step is 2G rows
// (G = 16 / sizeof(element)).  Per k-step the stage holds the raw dy rows' 128-channel
// chunks (4T KB) and x's spectrum units of the tile's 32 NB channels (T NB KB,
// [plane][half][channel]).  The ring, its 4-slot unrolled loop and
// the DMA issue follow eql_fwd4_kernel.  Each item writes its fp32 partial spectrum;
// eql_bwdw_reduce sums the items of a tile in a fixed order and applies the inverse.
#pragma once

#include <type_traits>

#include "eql_bwdw.h"
#include "eql_fwd.h"

namespace eql {

struct Bwdw4Args {
  const void* dy;   // [N][Dp*T] raw
  const void* xh;   // X units [kgCount][T][2][Cpad]
  float* wsR;       // partials of the real planes [S][NR][Dp][Cp]
  float* wsP;       // partials of the complex planes [S][T-NR][Dp][Cp]
  int N, Dp, Cp, Cpad, kgCount, kgPerSplit, dTiles, cTiles, numItems;
  Twiddles tw;
};

constexpr int kBwdw4Tile = 128;  // output channels per tile in d

// Ring depth: 5 slots (160 KB of LDS at T = 4) keep four stages in flight per CU; the
// kernel is bound by load latency, not bandwidth, at the layer shapes it serves.  The
// fp32 T = 4 instantiation keeps 4 (a fifth slot's registers would spill).
template <int T, typename Elt>
__host__ __device__ constexpr int bwdw4_slots() { return T == 4 ? (sizeof(Elt) == 2 ? 5 : 4) : 6; }

template <int T, typename Elt, int NB>
__global__ void __launch_bounds__(256) eql_bwdw4_kernel(const Bwdw4Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using E = EltT<Elt>;
  constexpr int G = E::kPerUnit;           // rows per operand unit
  constexpr int NR = n_real_planes(T);
  constexpr int NP = n_pairs(T);
  constexpr int CT = 32 * NB;              // input channels c per tile
  constexpr int ELT = (int)sizeof(Elt);
  constexpr int TB = T * ELT;              // bytes of one (row, channel) group
  constexpr int CHUNK = kBwdw4Tile * TB;   // bytes of one dy row's tile chunk
  constexpr int UPR = CHUNK / 16;          // 16-byte units per row chunk
  constexpr int ASLOT = 2 * G * CHUNK;     // raw dy bytes per stage (4T KB)
  constexpr int BSLOT = T * 2 * CT * 16;   // spectrum bytes per stage (T NB KB)
  constexpr int NS = bwdw4_slots<T, Elt>(), DIST = NS - 1;
  constexpr int U = NS % 2 ? 2 * NS : NS;   // loop unroll: slot and fragment buffer both fixed
  constexpr int SPLIT = NS / 2 + 1;         // slots SPLIT.. read from a second base register
  constexpr int IPA = ASLOT / 4096;        // dy DMA loads per wave per stage (T)
  constexpr int IPB = BSLOT / 4096;        // spectrum DMA loads per wave per stage
  static_assert(T == 1 || T == 2 || T == 4, "fused weight gradient: T in {1, 2, 4}");
  static_assert(IPA == 1 || IPA == 2 || IPA == 4, "dy loads per wave");
  static_assert(NB >= 2 && NB <= 4 && IPB * 4096 == BSLOT && IPB >= 1 && IPB <= 4, "spectrum loads per wave");
  static_assert(NS * (ASLOT + BSLOT) <= 160 * 1024, "LDS budget");
  static_assert((SPLIT - 1) * ASLOT + (G - 1) * CHUNK < 65536 && (NS - SPLIT - 1) * ASLOT + (G - 1) * CHUNK < 65536 &&
                    (SPLIT - 1) * BSLOT + (2 * T - 1) * CT * 16 + (NB - 1) * 512 < 65536,
                "ds_read immediate offsets");
  constexpr int WAIT_TOP = (DIST - 2) * (IPA + IPB);
  constexpr int WAIT_PRO = (DIST - 1) * (IPA + IPB);
  static_assert(WAIT_PRO < 64, "vmcnt range");

  __shared__ u32x4 ringA[NS][ASLOT / 16];
  __shared__ u32x4 ringB[NS][BSLOT / 16];

  // Items ordered split-major; consecutive ids (the tiles of one row range, which
  // share dy rows and x spectrum units) map to one XCD's L2.
  const int item = xcd_remap(blockIdx.x, a.numItems);
  const int tiles = a.dTiles * a.cTiles;
  const int split = item / tiles;
  const int tile = item - split * tiles;
  const int dTile = tile / a.cTiles, cTile = tile - dTile * a.cTiles;
  const int d0 = dTile * kBwdw4Tile, c0 = cTile * CT;
  const int kgBegin = split * a.kgPerSplit;
  const int nst = max(0, min(a.kgCount, kgBegin + a.kgPerSplit) - kgBegin);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const uint32_t rowBytes = (uint32_t)a.Dp * TB;
  const uint32_t dyBytes = (uint32_t)a.N * rowBytes;  // < 2^32 (checked by the host)

  // Lane state.
  int lane = lane_index();
  const int lrow = lane & 31, khalf = lane >> 5;
  // dy DMA: load i of the wave covers ring bytes (wave IPA + i) KB .. +1 KB of the stage,
  // i.e. unit P = (wave IPA + i) 64 + lane: row P / UPR, unit P % UPR of its chunk.
  // Units of channels past D' take an out-of-range offset.
  uint32_t aOff[IPA];
#pragma unroll
  for (int i = 0; i < IPA; ++i) {
    const int P = (wave * IPA + i) * 64 + lane;
    const int r = P / UPR, u = P - r * UPR;
    const int dl = (u * 16) / TB;  // first channel of the unit within the tile
    aOff[i] = d0 + dl < a.Dp ? (uint32_t)r * rowBytes + (uint32_t)(d0 * TB + u * 16) : kOob;
  }
  // Spectrum DMA: load i of the wave covers stage unit P = (wave IPB + i) 64 + lane,
  // which is channel c0 + P % CT of run P / CT = (plane, half).
  uint32_t bOff[IPB];
#pragma unroll
  for (int i = 0; i < IPB; ++i) {
    const int P = (wave * IPB + i) * 64 + lane;
    const int run = P / CT;
    bOff[i] = (uint32_t)run * (uint32_t)a.Cpad * 16u + (uint32_t)(c0 + P - run * CT) * 16u;
  }
  // Fragment reads: dY of output channel d0 + 32 wave + lrow, rows khalf G .. +G-1 of
  // the stage; X units of channel c0 + 32 nb + lrow, half khalf, plane p.
  // Slots 0 .. SPLIT-1 are read at immediate offsets from aRd / bRd, the others from
  // aRd2 / bRd2 (ds_read offsets stop at 64 KB).
  const uint32_t aRd = lds_addr(&ringA[0][0]) + (uint32_t)(khalf * G * CHUNK + (wave * 32 + lrow) * TB);
  const uint32_t bRd = lds_addr(&ringB[0][0]) + (uint32_t)((khalf * CT + lrow) * 16);
  const uint32_t aRd2 = aRd + (uint32_t)(SPLIT * ASLOT), bRd2 = bRd + (uint32_t)(SPLIT * BSLOT);

  // Issue side: the stage to load next; its dy rows start at aCur, its spectrum units
  // at bCur; past the item's last stage the loads have an empty range.
  int issSt = 0;
  const uint64_t aStep = (uint64_t)2 * G * rowBytes;
  const uint64_t bStep = (uint64_t)T * 2 * a.Cpad * 16;
  uint64_t aCur = reinterpret_cast<uint64_t>(a.dy) + (uint64_t)kgBegin * aStep;
  uint64_t bCur = reinterpret_cast<uint64_t>(a.xh) + (uint64_t)kgBegin * bStep;
  const uint64_t dyEnd = reinterpret_cast<uint64_t>(a.dy) + dyBytes;
  const uint32_t bRange = (uint32_t)(T * 2 * a.Cpad * 16);
  const uint32_t aDma = lds_addr(&ringA[0][0]) + (uint32_t)(wave * IPA * 1024);
  const uint32_t bDma = lds_addr(&ringB[0][0]) + (uint32_t)(wave * IPB * 1024);
  auto issue = [&](auto slotTag) __attribute__((always_inline)) {
    constexpr int S = decltype(slotTag)::value;
    const bool live = issSt < nst;
    // dy: the rows from this stage to the end of dy (rows past N read zero).
    const uint32_t aLen = live && aCur < dyEnd ? (uint32_t)(dyEnd - aCur) : 0u;
    dma16_each<IPA, S * ASLOT>(desc_words(aCur, aLen), aOff, aDma);
    dma16_each<IPB, S * BSLOT>(desc_words(bCur, live ? bRange : 0u), bOff, bDma);
    aCur += aStep;
    bCur += bStep;
    ++issSt;
  };

  auto rd16 = [&](uint32_t addr, int imm) __attribute__((always_inline)) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        (const __attribute__((address_space(3))) char*)(uintptr_t)addr + imm);
  };

  // Raw dy of this lane for one stage: G rows x TB bytes, as 32-bit words
  // (row j occupies words j TB/4 .. ; for TB < 4, one row per half word).
  constexpr int RW = G * TB / 4 > 0 ? G * TB / 4 : 1;
  uint32_t raw[RW];
  auto read_a = [&](auto slotTag) __attribute__((always_inline)) {
    constexpr int S = decltype(slotTag)::value;
    const __attribute__((address_space(3))) char* base =
        (const __attribute__((address_space(3))) char*)(uintptr_t)(S < SPLIT ? aRd : aRd2);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const __attribute__((address_space(3))) char* p = base + (S < SPLIT ? S : S - SPLIT) * ASLOT + j * CHUNK;
      if constexpr (TB == 16) {
        const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
        raw[4 * j + 0] = v[0];
        raw[4 * j + 1] = v[1];
        raw[4 * j + 2] = v[2];
        raw[4 * j + 3] = v[3];
      } else if constexpr (TB == 8) {
        const u32x2 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(p);
        raw[2 * j + 0] = v[0];
        raw[2 * j + 1] = v[1];
      } else if constexpr (TB == 4) {
        raw[j] = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(p);
      } else {
        const uint32_t h = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(p);
        if (j & 1) raw[j / 2] |= h << 16;
        else raw[j / 2] = h;
      }
    }
  };

  // dY operand units of the G rows: planes 0 .. T-1, then for each complex pair the
  // negated Re plane (Im G = dYi Xr - dYr Xi).
  u32x4 af[2][T + NP];
  auto transform = [&](auto abTag) __attribute__((always_inline)) {
    constexpr int ab = decltype(abTag)::value;
    if constexpr (T == 4 && ELT == 2) {
      u32x4 o[5];
      dft_p4_f16(raw, o);  // the G rows play the role of the forward's G channels
      af[ab][0] = o[0];
      af[ab][1] = o[1];
      af[ab][2] = o[2];
      af[ab][3] = o[3];
      af[ab][4] = neg_unit(o[2], E::kSignMask);
    } else {
      float pl[T][G];
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float v[T], o[T];
#pragma unroll
        for (int h = 0; h < T; ++h) {
          const int i = e * T + h;
          if constexpr (ELT == 2) v[h] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[i / 2] >> ((i & 1) * 16)));
          else v[h] = __builtin_bit_cast(float, raw[i]);
        }
        Dft<T>::run(v, o, a.tw);
#pragma unroll
        for (int p = 0; p < T; ++p) pl[p][e] = o[p];
      }
#pragma unroll
      for (int p = 0; p < T; ++p) af[ab][p] = E::pack(pl[p]);
#pragma unroll
      for (int q = 0; q < NP; ++q) af[ab][T + q] = neg_unit(af[ab][NR + 2 * q], E::kSignMask);
    }
  };

  f32x16 acc[T][NB];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) E::zero(acc[p][nb]);

  // Stage j of the unrolled loop: ring slot j % NS, fragment buffer j % 2.  Stage g
  // reads its first block's X fragments (landed before the previous barrier), waits
  // for this wave's loads of stage g+1, passes the barrier, issues stage g+DIST, reads
  // dy of stage g+1, then per 32-channel block of c: the next block's X fragments, the
  // block's MFMAs, and after block 0 the transform of dy stage g+1.
  auto stage = [&](auto jTag) __attribute__((always_inline)) {
    constexpr int J = decltype(jTag)::value;
    constexpr int S = J % NS;
    constexpr int cur = J & 1;
    constexpr int SB0 = (S < SPLIT ? S : S - SPLIT) * BSLOT;
    const uint32_t bBase = S < SPLIT ? bRd : bRd2;
    using Nxt = std::integral_constant<int, cur ^ 1>;
    using SN = std::integral_constant<int, (S + 1) % NS>;
    using SI = std::integral_constant<int, (S + DIST) % NS>;
    u32x4 bf[2][T];
#pragma unroll
    for (int p = 0; p < T; ++p) bf[0][p] = rd16(bBase, SB0 + p * 2 * CT * 16);
    wait_vmcnt<WAIT_TOP>();
    __builtin_amdgcn_s_barrier();
    issue(SI{});
    read_a(SN{});
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (nb + 1 < NB) {
#pragma unroll
        for (int p = 0; p < T; ++p) bf[(nb + 1) & 1][p] = rd16(bBase, SB0 + p * 2 * CT * 16 + (nb + 1) * 512);
      }
      const u32x4(&b)[T] = bf[nb & 1];
#pragma unroll
      for (int p = 0; p < NR; ++p) E::mfma(acc[p][nb], af[cur][p], b[p]);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int re = NR + 2 * q, im = re + 1;
        E::mfma(acc[re][nb], af[cur][re], b[re]);      // Re += dYr Xr
        E::mfma(acc[re][nb], af[cur][im], b[im]);      //    + dYi Xi
        E::mfma(acc[im][nb], af[cur][im], b[re]);      // Im += dYi Xr
        E::mfma(acc[im][nb], af[cur][T + q], b[im]);   //    - dYr Xi
      }
      if (nb == 0) transform(Nxt{});
    }
  };

  // Prologue: stages 0 .. DIST-1, then dy of stage 0 into fragment buffer 0.
  [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
    (issue(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, DIST>{});
  wait_vmcnt<WAIT_PRO>();
  __builtin_amdgcn_s_barrier();
  read_a(std::integral_constant<int, 0>{});
  transform(std::integral_constant<int, 0>{});
  int st = 0;
  for (; st + U <= nst; st += U) {
    [&]<int... J>(std::integer_sequence<int, J...>) __attribute__((always_inline)) {
      (stage(std::integral_constant<int, J>{}), ...);
    }(std::make_integer_sequence<int, U>{});
  }
  // The last nst % U stages (one workgroup per item: the ring always starts at slot 0).
  [&]<int... J>(std::integer_sequence<int, J...>) __attribute__((always_inline)) {
    ((st + J < nst ? (stage(std::integral_constant<int, J>{}), 0) : 0), ...);
  }(std::make_integer_sequence<int, U - 1>{});
  wait_vmcnt<0>();

  // Partial spectrum of this item: slot r of lane l in block nb is output channel
  // d = d0 + 32 wave + 8 (r/4) + 4 (l/32) + r%4 and input channel c = c0 + 32 nb + l%32.
  const size_t plane = (size_t)a.Dp * a.Cp;
  lane = lane_index();
#pragma unroll
  for (int p = 0; p < T; ++p) {
    float* out = p < NR ? a.wsR + ((size_t)split * NR + p) * plane
                        : a.wsP + ((size_t)split * (T - NR) + (p - NR)) * plane;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = c0 + 32 * nb + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = d0 + 32 * wave + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (d < a.Dp && c < a.Cp) out[(size_t)d * a.Cp + c] = acc[p][nb][r];
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace eql

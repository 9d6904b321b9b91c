// Fused forward kernel of the EQ-Linear layer: y = x W^T evaluated as
// group DFT (prologue) -> per-frequency channel GEMMs on MFMA -> inverse DFT
// (epilogue), with no intermediate global writes ("Implementacao" in "Resumo
// Tecnico: Flash EQ-Linear": fused data flow, Fourier fragments kept in registers
// and shared memory).  The input-gradient pass runs the same kernel on the
// conjugate-transposed packed weight.
//
// Work decomposition (gfx950, wave64, one 256-thread workgroup per CU):
//   * a workgroup owns 128 rows x BN = 32*NB output channels for all T planes;
//     each of its 4 waves owns 32 rows;
//   * the K loop runs over "stages" of JC 16-byte channel groups (two groups per
//     MFMA k-step);
//   * x goes straight from HBM/L2 into registers in MFMA A-operand order: lane l
//     takes row l%32 and channel group 2s + l/32 of k-step s (G channels x T group
//     elements, 16*T contiguous bytes), via bounds-checked buffer loads (rows past
//     N and channels past C' read as zero without branches).  The group DFT runs
//     in fp32 registers and rounds once to the element type; the negated Im planes
//     needed by the real part of each complex product are made by a sign flip;
//   * the packed spectrum of w for the workgroup's BN channels streams into an
//     NSTAGE-deep LDS ring with buffer loads that write LDS directly (no VGPR
//     staging).  A ring row holds the JC*T 16-byte units of one output channel,
//     XOR-swizzled so that the 16-byte MFMA B-operand reads of 16 consecutive
//     channels (one LDS cycle on the 64-bank LDS) touch 16 different 16-byte
//     bank groups;
//   * per k-step and 32-column block: real planes take one MFMA, a complex pair
//     four (Re += Xr Wr + (-Xi) Wi, Im += Xi Wr + Xr Wi);
//   * the epilogue reads the T accumulators of one (row, channel) from the same
//     register slot, applies the inverse DFT and stores T contiguous outputs;
//     adjacent lanes write adjacent channels.
#pragma once

#include <type_traits>

#include "eql_device.h"

namespace eql {

struct FwdArgs {
  const void* x;    // [N][Cin*T]
  const void* wp;   // packed spectrum, out = Dout, in = Cin (groups padded to Jpad)
  void* y;          // [N][Dout*T]
  int N, Cin, Dout, Jpad, colTiles, numTiles, loadMode;
  uint32_t wpBytes;  // size of the packed weight in bytes (< 2^32)
  Twiddles tw;
};

constexpr int kFwdRows = 128;   // rows per workgroup (4 waves x 32)
constexpr int kFwdStages = 4;   // depth of the LDS ring for the packed weight

// s_waitcnt on vector-memory loads only (lgkm and exp counters left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
#endif

// Offsets at or beyond this value are outside every buffer: the load returns zero.
constexpr uint32_t kOob = 0x80000000u;

// How x is read.
//   kLoadNarrow: rows are not 16-byte aligned; loads of the widest power of two
//                dividing T*sizeof(Elt), each checked against C'.
//   kLoadAligned: 16-byte loads, each checked against C' (the last stage is partial).
//   kLoadFull: 16-byte loads, C' fills every group of the packed weight (a multiple
//              of 4 groups): no per-load check.
enum : int { kLoadNarrow = 0, kLoadAligned = 1, kLoadFull = 2 };

// Swizzle of ring row o: XOR applied to the unit index so that 16 consecutive rows
// read at the same unit land on 16 distinct (unit mod 16) positions.
template <int RP>
__device__ __forceinline__ int ring_swz(int o) {
  if constexpr (RP == 8) return (o >> 1) & 7;
  else return o & 15;
}

template <int T, typename Elt, int NB, int JC, int LOAD>
__global__ void __launch_bounds__(256) eql_fwd_kernel(const FwdArgs a) {
  // The body uses AMDGPU-only types (buffer resources); the host pass only needs
  // the kernel's signature to emit its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using E = EltT<Elt>;
  constexpr int G = E::kPerUnit;          // channels per 16-byte group
  constexpr int NR = n_real_planes(T);
  constexpr int NP = n_pairs(T);
  constexpr int KS = JC / 2;              // k-steps per stage
  constexpr int BN = 32 * NB;
  constexpr int R = JC * T;               // units of one output channel per stage
  constexpr int RP = R <= 8 ? 8 : (R + 15) / 16 * 16;  // ... padded to the swizzle span
  constexpr int IPW = BN * RP / 256;      // direct-to-LDS loads per wave per stage
  constexpr int NS = kFwdStages;
  constexpr int ELT = (int)sizeof(Elt);
  constexpr int GB = G * T * ELT;         // bytes of one lane's x block per k-step (16*T)
  constexpr int NW = LOAD == kLoadNarrow ? pow2_part(T * ELT) : 16;  // x load width
  constexpr int XL = KS * GB / NW;        // x loads per stage
  // Loads issued after weight stage st when stage st starts: x of stages st..st+2
  // and weight stages st+1, st+2.
  constexpr int WAIT_B = 3 * XL + 2 * IPW;
  constexpr bool kWaitExact = WAIT_B < 64;
  static_assert(JC % 2 == 0 && (BN * RP) % 256 == 0, "tile shape");

  __shared__ u32x4 ring[NS][BN * RP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, khalf = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, a.numTiles);
  const int rowTile = tile / a.colTiles, colTile = tile - rowTile * a.colTiles;
  const int row0 = rowTile * kFwdRows, col0 = colTile * BN;
  const int nst = a.Jpad / JC;
  const uint32_t rowBytes = (uint32_t)a.Cin * T * ELT;

  // x rows of this workgroup: rows past N fall outside the descriptor and read 0.
  const int tileRows = min(kFwdRows, a.N - row0);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const char*>(a.x) + (size_t)row0 * rowBytes, (uint32_t)tileRows * rowBytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wpBytes);
  const uint32_t xLaneOff = (uint32_t)(wave * 32 + lrow) * rowBytes;

  // Direct-to-LDS source offsets: position P = (wave*IPW + i)*64 + lane of a stage
  // holds unit r = (P % RP) ^ ring_swz(o) of output channel o = P / RP.
  uint32_t bOff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int P = (wave * IPW + i) * 64 + lane;
    const int o = P / RP, pos = P - o * RP;
    const int r = pos ^ ring_swz<RP>(o);
    const int og = min(col0 + o, a.Dout - 1);
    const int rr = r < R ? r : 0;  // padding positions load an arbitrary valid unit
    bOff[i] = ((uint32_t)og * a.Jpad + rr / T) * T * 16u + (uint32_t)(rr % T) * 16u;
  }

  // Weight stage st into ring slot st % NS.  Stages past the end read nothing
  // (out-of-range offsets), so the loop body needs no branch.
  auto issue_b = [&](int st) {
    const uint32_t stOff = st < nst ? (uint32_t)st * JC * T * 16u : kOob;
    u32x4* dst = &ring[st % NS][wave * IPW * 64];
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (__attribute__((address_space(3))) void*)(dst + i * 64), 16, bOff[i] + stOff, 0, 0, 0);
  };

  uint32_t raw[2][KS][4 * T];
  u32x4 af[2][KS][T + NP];

  // x of stage st into raw buffer `rb`.  Channels past C' read as zero, except in
  // kLoadFull mode where the stages past the end read arbitrary in-bounds data
  // that is transformed but never multiplied.
  auto issue_x = [&](int st, auto rbTag) {
    constexpr int rb = decltype(rbTag)::value;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int cfirst = (st * JC + 2 * s + khalf) * G;
      const uint32_t base = xLaneOff + (uint32_t)cfirst * T * ELT;
#pragma unroll
      for (int b = 0; b < GB; b += NW) {
        const int chv = cfirst + b / (T * ELT);
        const uint32_t off = (LOAD == kLoadFull || chv < a.Cin) ? base + b : kOob;
        if constexpr (NW == 16) {
          const u32x4 val = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
          raw[rb][s][b / 4 + 0] = val[0];
          raw[rb][s][b / 4 + 1] = val[1];
          raw[rb][s][b / 4 + 2] = val[2];
          raw[rb][s][b / 4 + 3] = val[3];
        } else if constexpr (NW == 8) {
          const u32x2 val = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(xr, off, 0, 0));
          raw[rb][s][b / 4 + 0] = val[0];
          raw[rb][s][b / 4 + 1] = val[1];
        } else if constexpr (NW == 4) {
          raw[rb][s][b / 4] = __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
        } else {
          const uint32_t hv = __builtin_amdgcn_raw_buffer_load_b16(xr, off, 0, 0);
          if ((b & 2) == 0) raw[rb][s][b / 4] = hv;
          else raw[rb][s][b / 4] |= hv << 16;
        }
      }
    }
  };

  // Group DFT of raw buffer `rb` into A-operand buffer `ab`.
  auto transform = [&](auto rbTag, auto abTag) {
    constexpr int rb = decltype(rbTag)::value, ab = decltype(abTag)::value;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float pl[T][G];
#pragma unroll
      for (int e = 0; e < G; ++e) {
        float v[T], o[T];
#pragma unroll
        for (int h = 0; h < T; ++h) {
          const int i = e * T + h;
          if constexpr (ELT == 2) {
            const uint16_t bits = (uint16_t)(raw[rb][s][i / 2] >> ((i & 1) * 16));
            v[h] = (float)__builtin_bit_cast(_Float16, bits);
          } else {
            v[h] = __builtin_bit_cast(float, raw[rb][s][i]);
          }
        }
        Dft<T, true>::run(v, o, a.tw);
#pragma unroll
        for (int p = 0; p < T; ++p) pl[p][e] = o[p];
      }
#pragma unroll
      for (int p = 0; p < T; ++p) af[ab][s][p] = E::pack(pl[p]);
#pragma unroll
      for (int q = 0; q < NP; ++q) af[ab][s][T + q] = neg_unit(af[ab][s][NR + 2 * q + 1], E::kSignMask);
    }
  };

  f32x16 acc[T][NB];
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[p][nb][r] = 0.0f;

  auto load_bfrag = [&](u32x4 (&bf)[T], const u32x4* slot, int s, int nb) {
    const int o = nb * 32 + lrow;
#pragma unroll
    for (int p = 0; p < T; ++p) {
      const int r = (2 * s + khalf) * T + p;
      bf[p] = slot[o * RP + (r ^ ring_swz<RP>(o))];
    }
  };

  auto mfma_block = [&](const u32x4 (&bf)[T], auto abTag, int s, int nb) {
    constexpr int ab = decltype(abTag)::value;
#pragma unroll
    for (int p = 0; p < NR; ++p) E::mfma(acc[p][nb], af[ab][s][p], bf[p]);
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int re = NR + 2 * q, im = re + 1;
      E::mfma(acc[re][nb], af[ab][s][re], bf[re]);
      E::mfma(acc[re][nb], af[ab][s][T + q], bf[im]);
      E::mfma(acc[im][nb], af[ab][s][im], bf[re]);
      E::mfma(acc[im][nb], af[ab][s][re], bf[im]);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // Prologue: weight stages 0..2 and x stages 0, 1 in flight; x stage 0
  // transformed; x stage 2 in flight.
  issue_b(0);
  issue_b(1);
  issue_b(2);
  issue_x(0, I0{});
  issue_x(1, I1{});
  if constexpr (2 * XL < 64) wait_vmcnt<XL>();  // x stage 0 (and everything before it)
  else wait_vmcnt<0>();
  transform(I0{}, I0{});
  issue_x(2, I0{});

  // Stage st.  x stage j lives in raw[j & 1] and af[j & 1]; `cur` = st & 1 is a
  // compile-time constant so that the fragments stay in registers.  Every stage
  // issues the same loads (weight st+3, x st+3), in range or not, so the wait for
  // weight stage st is a constant count.
  auto stage = [&](int st, auto curTag) {
    constexpr int cur = decltype(curTag)::value;
    using Cur = std::integral_constant<int, cur>;
    using Nxt = std::integral_constant<int, cur ^ 1>;
    if constexpr (kWaitExact) wait_vmcnt<WAIT_B>();
    else wait_vmcnt<0>();
    // Plain barrier (no fence): the ring reads of stage st-1 have been consumed by
    // MFMAs, and a fence would also wait for the prefetches in flight.
    __builtin_amdgcn_s_barrier();
    issue_b(st + 3);  // refills the slot of stage st-1

    const u32x4* slot = ring[st % NS];
    u32x4 bcur[T], bnext[T];
    load_bfrag(bcur, slot, 0, 0);
#pragma unroll
    for (int idx = 0; idx < KS * NB; ++idx) {
      const int s = idx / NB, nb = idx % NB;
      if (idx + 1 < KS * NB) load_bfrag(bnext, slot, (idx + 1) / NB, (idx + 1) % NB);
      mfma_block(bcur, Cur{}, s, nb);
      if (idx == 0) transform(Nxt{}, Nxt{});  // x stage st+1; overlaps the MFMA chains
      if (idx + 1 < KS * NB) {
#pragma unroll
        for (int p = 0; p < T; ++p) bcur[p] = bnext[p];
      }
    }
    issue_x(st + 3, Nxt{});
  };

  int st = 0;
  for (; st + 1 < nst; st += 2) {
    stage(st, I0{});
    stage(st + 1, I1{});
  }
  if (st < nst) stage(st, I0{});
  // Drain the look-ahead loads (all out of range) before the workgroup's LDS can
  // be reused.
  wait_vmcnt<0>();

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
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace eql

// Fused forward kernel of the EQ-Linear layer: y = x W^T evaluated as
// group DFT (prologue) -> per-frequency channel GEMMs on MFMA -> inverse DFT
// (epilogue), with no intermediate global writes ("Implementacao" in "Resumo
// Tecnico: Flash EQ-Linear": fused data flow, Fourier fragments kept in registers
// and shared memory).  The input-gradient pass runs the same kernel on the
// conjugate-transposed packed weight.
//
// Work decomposition (gfx950, wave64, one persistent 256-thread workgroup per CU):
//   * an output tile is 128 rows x BN = 32*NB output channels for all T planes;
//     each of the 4 waves owns 32 rows; a workgroup walks its tiles as one stream
//     of K stages, so loads run ahead across tile boundaries;
//   * the K loop runs over "stages" of JC 16-byte channel groups (two groups per
//     MFMA k-step);
//   * x of a stage (the workgroup's 128 rows x JC groups) streams into its own
//     LDS ring the same way as the weight (16-byte rows only; otherwise each lane
//     loads its x straight into registers with narrower bounds-checked loads).
//     Lane l takes row l%32 and channel group 2s + l/32 of k-step s (G channels x
//     T group elements) in MFMA A-operand order; rows past N and channels past
//     C' read as zero without branches.  The group DFT runs in fp32 registers and
//     rounds once to the element type; the negated Im planes needed by the real
//     part of each complex product are made by a sign flip;
//   * the packed spectrum of w for the workgroup's BN channels streams into an
//     NS-deep LDS ring with buffer loads that write LDS directly (no VGPR
//     staging).  A ring row holds the JC*T 16-byte units of one output channel,
//     XOR-swizzled so that the 16-byte MFMA B-operand reads of 16 consecutive
//     channels (one LDS cycle on the 64-bank LDS) touch 16 different 16-byte
//     bank groups;
//   * per k-step and 32-column block: real planes take one MFMA, a complex pair
//     four (Re += Xr Wr + (-Xi) Wi, Im += Xi Wr + Xr Wi);
//   * the epilogue reads the T accumulators of one (row, channel) from the same
//     register slot, applies the inverse DFT (its 1/T and 2/T are in the packed
//     weight) and stores T contiguous outputs; adjacent lanes write adjacent
//     channels.  EPI = 1 adds a per-channel bias, GELU and a residual first.
#pragma once

#include <type_traits>

#include "eql_device.h"
#include "eql_dma.h"

namespace eql {

struct FwdArgs {
  const void* x;    // [N][Cin*T]
  const void* wp;   // packed spectrum, out = Dout, in = Cin (groups padded to Jpad)
  void* y;          // [N][Dout*T]
  int N, Cin, Dout, Jpad, colTiles, numTiles, loadMode;
  uint32_t wpBytes;  // size of the packed weight in bytes (< 2^32)
  Twiddles tw;
  // Fused epilogue (EPI = 1 instantiations only): y = act(x W^T + bias) + res.
  const void* bias;  // [Dout] or null
  const void* res;   // [N][Dout*T] or null (may equal y)
  void* pre;         // [N][Dout*T] or null: receives x W^T + bias (the activation's input)
  int act;           // 0 none, 1 GELU
};

constexpr int kFwdRows = 128;   // rows per workgroup (4 waves x 32)

#if defined(__HIP_DEVICE_COMPILE__)
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// p4 group DFT of 8 fp16 channels (raw[2e], raw[2e+1] hold (x0,x1), (x2,x3) of
// channel e) into the A-operand units X0, X2, Xr, Xi and -Xi (8 halves each).
//   Xr = x0 - x2 and -Xi = x1 - x3 come from one packed fp16 subtraction per
//   channel (a single rounding of the exact difference); X0 = (x0+x1) + (x2+x3)
//   and X2 = (x0-x1) + (x2-x3) are fp32 dot products of the fp16 pairs, rounded
//   once to fp16.  The 1/2 of the p4 forward transform is folded into the packed
//   weight's real planes.
// b.lo*c.lo + b.hi*c.hi in fp32: v_dot2_f32_f16 with the addend given as the inline
// constant 0 (the two-operand form accumulates into its destination, which then
// has to be zeroed by a separate move first).
__device__ __forceinline__ float dot2_f16(f16x2 b, f16x2 c) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ void dft_p4_f16(const uint32_t (&raw)[16], u32x4 (&out)[5]) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  const f16x2 pm = {(_Float16)1.0f, (_Float16)-1.0f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // channel pair (2q, 2q+1) -> word q of each unit
    const f16x2 a0 = __builtin_bit_cast(f16x2, raw[4 * q + 0]), b0 = __builtin_bit_cast(f16x2, raw[4 * q + 1]);
    const f16x2 a1 = __builtin_bit_cast(f16x2, raw[4 * q + 2]), b1 = __builtin_bit_cast(f16x2, raw[4 * q + 3]);
    const f16x2 d0 = a0 - b0, d1 = a1 - b1;  // (Xr, -Xi) of each channel
    const float x0e = __builtin_amdgcn_fdot2(a0, ones, dot2_f16(b0, ones), false);
    const float x0o = __builtin_amdgcn_fdot2(a1, ones, dot2_f16(b1, ones), false);
    const float x2e = __builtin_amdgcn_fdot2(a0, pm, dot2_f16(b0, pm), false);
    const float x2o = __builtin_amdgcn_fdot2(a1, pm, dot2_f16(b1, pm), false);
    const f16x2 X0 = {(_Float16)x0e, (_Float16)x0o};
    const f16x2 X2 = {(_Float16)x2e, (_Float16)x2o};
    const uint32_t nxi = __builtin_bit_cast(uint32_t, __builtin_shufflevector(d0, d1, 1, 3));
    out[0][q] = __builtin_bit_cast(uint32_t, X0);
    out[1][q] = __builtin_bit_cast(uint32_t, X2);
    out[2][q] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(d0, d1, 0, 2));
    out[3][q] = nxi ^ 0x80008000u;
    out[4][q] = nxi;
  }
}
#endif

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

// Largest power of two <= v (v >= 1).
constexpr int floor_pow2(int v) { return v >= 16 ? 16 : v >= 8 ? 8 : v >= 4 ? 4 : v >= 2 ? 2 : 1; }

// erf by formula 7.1.26 of Abramowitz and Stegun, Handbook of Mathematical
// Functions (|error| <= 1.5e-7 for the formula itself):
//   erf(a) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-a^2),
//   t = 1 / (1 + p a), a = |u|, extended as an odd function.
// The reciprocal and exp2 are the hardware approximations (about 1 ulp).
// erf_as_e takes exp(-u^2) from the caller (GELU's derivative needs it as well).
__device__ __forceinline__ float erf_as_e(float u, float e) {
  const float a = __builtin_fabsf(u);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, a, 1.0f));
  float q = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  q = __builtin_fmaf(q, t, 1.421413741f);
  q = __builtin_fmaf(q, t, -0.284496736f);
  q = __builtin_fmaf(q, t, 0.254829592f);
  return __builtin_copysignf(__builtin_fmaf(-q * t, e, 1.0f), u);
}

__device__ __forceinline__ float erf_as(float u) {
  const float a = __builtin_fabsf(u);
  return erf_as_e(u, __builtin_amdgcn_exp2f((-1.4426950408889634f * a) * a));  // exp(-a^2)
}

// GELU in its exact form, v * Phi(v) = v/2 (1 + erf(v / sqrt 2)), in fp32.
__device__ __forceinline__ float gelu_erf(float v) {
  const float h = 0.5f * v;
  return __builtin_fmaf(h, erf_as(v * 0.7071067811865475f), h);
}

// EPI = 1: the epilogue adds the per-channel bias, applies the activation and adds
// the residual (all in fp32) before the single rounding to Elt.
template <int T, typename Elt, int NB, int JC, int LOAD, int EPI>
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
  constexpr int R = JC * T;               // 16-byte units of one channel row per stage
  constexpr int RP = R <= 8 ? 8 : (R + 15) / 16 * 16;  // ... padded to the swizzle span
  constexpr int ELT = (int)sizeof(Elt);
  // x through an LDS ring (buffer loads straight into LDS) when rows are 16-byte
  // aligned and the ring fits; otherwise x is read into registers synchronously.
  constexpr bool XLDS = LOAD != kLoadNarrow && T <= 8;
  constexpr int STAGE_UNITS = BN * RP + (XLDS ? kFwdRows * RP : 0);
  constexpr int NS = (4 * STAGE_UNITS * 16 <= 160 * 1024) ? 4 : 3;  // ring depth
  constexpr int DIST = NS - 1;            // stages loaded ahead
  constexpr int IPW = BN * RP / 256;      // weight DMA loads per wave per stage
  constexpr int IPWX = XLDS ? 32 * RP / 64 : 0;  // x DMA loads per wave per stage
  constexpr int GB = G * T * ELT;         // bytes of one lane's x block per k-step (16*T)
  constexpr int NW = LOAD == kLoadNarrow ? pow2_part(T * ELT) : 16;  // register-path width
  constexpr int XL = XLDS ? 0 : KS * GB / NW;  // register-path x loads per stage
  static_assert(JC % 2 == 0 && (BN * RP) % 256 == 0 && (32 * RP) % 64 == 0, "tile shape");
  static_assert(NS * STAGE_UNITS * 16 <= 160 * 1024, "LDS budget");
  // vmcnt at the top of a stage (see the pipeline notes below); a count beyond the
  // counter's range falls back to waiting for every load.
  constexpr int WAIT_TOP_N = XLDS ? (DIST - 2) * (IPW + IPWX) : (DIST - 1) * (XL + IPW);
  constexpr int WAIT_TOP = WAIT_TOP_N < 64 ? WAIT_TOP_N : 0;
  constexpr int WAIT_PRO = XLDS ? (DIST - 1) * (IPW + IPWX) : 0;
  static_assert(WAIT_PRO < 64 && IPW < 64, "vmcnt range");

  __shared__ u32x4 ringB[NS][BN * RP];
  __shared__ u32x4 ringX[XLDS ? NS : 1][XLDS ? kFwdRows * RP : 1];

  // Persistent schedule: workgroup b takes the tiles xcd_remap(b + k*gridDim.x)
  // for k = 0, 1, ... and walks them as one stream of K stages, so the loads of a
  // tile's first stages overlap the previous tile's last stages and epilogue.  With
  // gridDim.x a multiple of 8, all of a workgroup's tiles map to its own XCD, and
  // the XCD's concurrent workgroups share row blocks of x in its L2.
  const int b0 = blockIdx.x, grid = gridDim.x;
  if (b0 >= a.numTiles) return;
  const int myTiles = (a.numTiles - b0 + grid - 1) / grid;
  const int nst = a.Jpad / JC;

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  // Lane-derived values are re-derived after every epilogue from a lane index the
  // compiler cannot hoist, so none of them (LDS addresses, DMA offsets) is live in
  // the epilogue, where every register is taken: a spill there would make the
  // compiler drain all outstanding loads at its reload.
  int lane = lane_index();
  int lrow = lane & 31, khalf = lane >> 5;
  const uint32_t rowBytes = (uint32_t)a.Cin * T * ELT;
  const uint32_t colStride = (uint32_t)a.Jpad * T * 16u;  // packed bytes per output channel

  auto tile_row0 = [&](int k) __attribute__((always_inline)) {
    return (xcd_remap(b0 + k * grid, a.numTiles) / a.colTiles) * kFwdRows;
  };
  auto tile_col0 = [&](int k) __attribute__((always_inline)) {
    const int t = xcd_remap(b0 + k * grid, a.numTiles);
    return (t - (t / a.colTiles) * a.colTiles) * BN;
  };

  // Weight ring: position P = (wave*IPW + i)*64 + lane of a stage holds unit
  // r = (P % RP) ^ ring_swz(o) of output channel o = P / RP.  Offsets are relative
  // to the stage's first byte in output channel col0; channels past D' fall
  // outside the descriptor and read zero.
  uint32_t bOff[IPW];
  uint32_t xOff[IPWX > 0 ? IPWX : 1];
  int xCh[IPWX > 0 ? IPWX : 1];
  auto lane_offsets = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int P = (wave * IPW + i) * 64 + lane;
      const int o = P / RP, pos = P - o * RP;
      const int r = pos ^ ring_swz<RP>(o);
      const int rr = r < R ? r : 0;  // padding positions load an arbitrary unit
      bOff[i] = (uint32_t)o * colStride + (uint32_t)rr * 16u;
    }
    // x ring (each wave loads and reads only its own 32 rows): position
    // P = wave*32*RP + i*64 + lane holds unit u = (P % RP) ^ ring_swz(row) of row
    // P / RP; unit u of a stage is bytes [16u, 16u+16) of the row's JC*G channels.
    // Rows past N fall outside the descriptor and read zero.
#pragma unroll
    for (int i = 0; i < IPWX; ++i) {
      const int P = wave * 32 * RP + i * 64 + lane;
      const int row = P / RP, pos = P - row * RP;
      const int u = pos ^ ring_swz<RP>(row);
      const int uu = u < R ? u : 0;
      xOff[i] = (uint32_t)row * rowBytes + (uint32_t)uu * 16u;
      xCh[i] = (uu * 16) / (T * ELT);  // channel (within the stage) of the unit's first element
    }
  };
  lane_offsets();

  // Stage g of the stream = stage st of this workgroup's tile k (g = k*nst + st).
  // Every stage issues the same loads; past the stream they have an empty range
  // and read nothing.  Tile geometry is recomputed only when the loader crosses
  // into the next tile; per stage only the scalar descriptor base moves.
  int issK = 0, issSt = 0;  // next stage to load
  uint64_t bTileBase = 0, xTileBase = 0;
  uint32_t bTileBytes = 0, xTileBytes = 0;
  auto set_issue_tile = [&](int k) __attribute__((always_inline)) {
    if (k < myTiles) {
      const int row0 = tile_row0(k), col0 = tile_col0(k);
      bTileBase = reinterpret_cast<uint64_t>(a.wp) + (uint64_t)col0 * colStride;
      bTileBytes = (uint32_t)(a.Dout - col0) * colStride;
      xTileBase = reinterpret_cast<uint64_t>(a.x) + (uint64_t)row0 * rowBytes;
      xTileBytes = (uint32_t)min(kFwdRows, a.N - row0) * rowBytes;
    } else {
      bTileBytes = 0;
      xTileBytes = 0;
    }
  };
  set_issue_tile(0);
  auto issue_stage = [&](int g) __attribute__((always_inline)) {
    {
      // Bytes left in the tile from this stage on (0 past the stream, and for x 0
      // once the stage starts beyond the row's last channel, in the padding).
      const uint32_t st0 = (uint32_t)issSt * JC * T * 16u;
      const BufDesc d = desc_at(bTileBase + st0, (issK < myTiles && bTileBytes > st0) ? bTileBytes - st0 : 0u);
      const uint32_t dst = lds_addr(&ringB[g % NS][wave * IPW * 64]);
      uint32_t l[IPW];
#pragma unroll
      for (int i = 0; i < IPW; ++i) l[i] = dst + i * 1024u;
      dma16_batch<IPW>(d, bOff, l);
    }
    if constexpr (XLDS) {
      const int c0 = issSt * JC * G;
      const uint32_t st0 = (uint32_t)c0 * T * ELT;
      const BufDesc d = desc_at(xTileBase + st0, (issK < myTiles && xTileBytes > st0) ? xTileBytes - st0 : 0u);
      const uint32_t dst = lds_addr(&ringX[g % NS][wave * 32 * RP]);
      uint32_t off[IPWX], l[IPWX];
#pragma unroll
      for (int i = 0; i < IPWX; ++i) {
        off[i] = (LOAD == kLoadFull || c0 + xCh[i] < a.Cin) ? xOff[i] : kOob;
        l[i] = dst + i * 1024u;
      }
      dma16_batch<IPWX>(d, off, l);
    }
    if (++issSt == nst) {
      issSt = 0;
      set_issue_tile(++issK);
    }
  };

  uint32_t raw[KS][4 * T];
  u32x4 af[2][KS][T + NP];

  // Register path: x of stream stage g for this lane (row lrow, group 2s+khalf).
  auto load_xreg = [&](int g) __attribute__((always_inline)) {
    if constexpr (!XLDS) {
      const int k = g / nst, st = g - k * nst;
      const bool live = k < myTiles;
      const int row0 = live ? tile_row0(k) : 0;
      const __amdgpu_buffer_rsrc_t xr =
          make_rsrc(static_cast<const char*>(a.x) + (size_t)row0 * rowBytes,
                    (uint32_t)max(0, min(kFwdRows, a.N - row0)) * rowBytes);
      const uint32_t xLaneOff = (uint32_t)(wave * 32 + lrow) * rowBytes;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int cfirst = (st * JC + 2 * s + khalf) * G;
        const uint32_t base = xLaneOff + (uint32_t)cfirst * T * ELT;
#pragma unroll
        for (int b = 0; b < GB; b += NW) {
          const int chv = cfirst + b / (T * ELT);
          const uint32_t off = (live && (LOAD == kLoadFull || chv < a.Cin)) ? base + b : kOob;
          if constexpr (NW == 16) {
            const u32x4 val = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
            raw[s][b / 4 + 0] = val[0];
            raw[s][b / 4 + 1] = val[1];
            raw[s][b / 4 + 2] = val[2];
            raw[s][b / 4 + 3] = val[3];
          } else if constexpr (NW == 8) {
            const u32x2 val = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(xr, off, 0, 0));
            raw[s][b / 4 + 0] = val[0];
            raw[s][b / 4 + 1] = val[1];
          } else if constexpr (NW == 4) {
            raw[s][b / 4] = __builtin_amdgcn_raw_buffer_load_b32(xr, off, 0, 0);
          } else {
            const uint32_t hv = __builtin_amdgcn_raw_buffer_load_b16(xr, off, 0, 0);
            if ((b & 2) == 0) raw[s][b / 4] = hv;
            else raw[s][b / 4] |= hv << 16;
          }
        }
      }
    }
  };

  // LDS path: this lane's x of stream stage g (k-step s: units (2s+khalf)*T .. +T).
  auto read_xlds = [&](int g) __attribute__((always_inline)) {
    if constexpr (XLDS) {
      const u32x4* slot = ringX[g % NS];
      const int row = wave * 32 + lrow;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int v = 0; v < T; ++v) {
          const int u = (2 * s + khalf) * T + v;
          const u32x4 val = slot[row * RP + (u ^ ring_swz<RP>(row))];
          raw[s][4 * v + 0] = val[0];
          raw[s][4 * v + 1] = val[1];
          raw[s][4 * v + 2] = val[2];
          raw[s][4 * v + 3] = val[3];
        }
    }
  };

  // Group DFT of the raw stage into A-operand buffer `ab`.
  auto transform = [&](auto abTag) __attribute__((always_inline)) {
    constexpr int ab = decltype(abTag)::value;
    if constexpr (T == 4 && ELT == 2) {
#pragma unroll
      for (int s = 0; s < KS; ++s) dft_p4_f16(raw[s], af[ab][s]);
      return;
    }
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
            const uint16_t bits = (uint16_t)(raw[s][i / 2] >> ((i & 1) * 16));
            v[h] = (float)__builtin_bit_cast(_Float16, bits);
          } else {
            v[h] = __builtin_bit_cast(float, raw[s][i]);
          }
        }
        Dft<T>::run(v, o, a.tw);
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
  // Clearing at the top of each tile.  Up to T = 6 each 32x32 tile is cleared by one
  // MFMA of zero operands; written as constants the clearing is emitted as two
  // register writes per accumulator.  From T = 7 on, the MFMA form leaves the
  // register allocator short and it spills, so the constant form is kept there.
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < T; ++p)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (T <= 6) E::zero(acc[p][nb]);
        else acc[p][nb] = (f32x16){};
      }
  };

  auto load_bfrag = [&](u32x4 (&bf)[T], const u32x4* slot, int s, int nb) __attribute__((always_inline)) {
    const int o = nb * 32 + lrow;
#pragma unroll
    for (int p = 0; p < T; ++p) {
      const int r = (2 * s + khalf) * T + p;
      bf[p] = slot[o * RP + (r ^ ring_swz<RP>(o))];
    }
  };

  auto mfma_block = [&](const u32x4 (&bf)[T], auto abTag, int s, int nb) __attribute__((always_inline)) {
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

  // Epilogue of tile k: accumulator slot r of lane l holds row 8*(r/4) + 4*(l/32) +
  // r%4 and column l%32 of each 32x32 block.  Stores go through a buffer
  // descriptor covering the tile's valid rows; columns past D' take an offset
  // beyond every range, so no store needs a branch.
  const uint32_t outRow = (uint32_t)a.Dout * T * ELT;  // bytes of one output row
  auto epilogue = [&](int k) __attribute__((always_inline)) {
    const int row0 = tile_row0(k), col0 = tile_col0(k);
    const uint32_t rows = (uint32_t)min(kFwdRows, a.N - row0);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(static_cast<char*>(a.y) + (size_t)row0 * outRow, rows * outRow);
    // The lane index is recomputed here rather than kept live through the main
    // loop, where every register is taken.
    const int ln = lane_index();
    const uint32_t laneOff = (uint32_t)(wave * 32 + 4 * (ln >> 5)) * outRow;
    // Fused epilogue operands: an absent bias or residual gets an empty range, so
    // its loads read zero.
    const __amdgpu_buffer_rsrc_t br = make_rsrc(a.bias, EPI && a.bias ? (uint32_t)a.Dout * ELT : 0u);
    const __amdgpu_buffer_rsrc_t rr =
        make_rsrc(EPI && a.res ? static_cast<const char*>(a.res) + (size_t)row0 * outRow : nullptr,
                  EPI && a.res ? rows * outRow : 0u);
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(EPI && a.pre ? static_cast<char*>(a.pre) + (size_t)row0 * outRow : nullptr,
                  EPI && a.pre ? rows * outRow : 0u);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = col0 + nb * 32 + (ln & 31);
      const uint32_t cOff = col < a.Dout ? laneOff + (uint32_t)col * T * ELT : kOob;
      float bv = 0.0f;
      if constexpr (EPI) {
        uint32_t b1[1];
        load_group_raw<1, Elt>(br, col < a.Dout ? (uint32_t)col * ELT : kOob, b1);
        float bf1[1];
        group_from_raw<1, Elt>(b1, bf1);
        bv = bf1[0];
      }
      // Fused epilogue: the residual groups of a chunk are loaded before any of its
      // stores (the compiler may not move a load above a store to y, which the
      // residual may alias), so one wait covers the chunk.
      constexpr int RW = group_words<T, Elt>();
      constexpr int CH = EPI ? floor_pow2(32 / RW < 1 ? 1 : (32 / RW > 16 ? 16 : 32 / RW)) : 16;
      static_assert(16 % CH == 0, "chunks must tile the 16 accumulator slots");
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += CH) {
        uint32_t rw[CH][RW];
        if constexpr (EPI) {
#pragma unroll
          for (int j = 0; j < CH; ++j)
            load_group_raw<T, Elt>(rr, cOff + (uint32_t)(8 * ((r0 + j) >> 2) + ((r0 + j) & 3)) * outRow, rw[j]);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const int r = r0 + j;
          float P[T], yv[T];
#pragma unroll
          for (int p = 0; p < T; ++p) P[p] = acc[p][nb][r];
          Idft<T, false>::run(P, yv, a.tw);
          const uint32_t off = cOff + (uint32_t)(8 * (r >> 2) + (r & 3)) * outRow;
          if constexpr (EPI) {
            float rv[T];
            group_from_raw<T, Elt>(rw[j], rv);
#pragma unroll
            for (int g = 0; g < T; ++g) yv[g] += bv;
            if (a.pre) store_group_buf<T, Elt>(pr, off, yv);
#pragma unroll
            for (int g = 0; g < T; ++g) {
              const float v = a.act == 1 ? gelu_erf(yv[g]) : yv[g];
              yv[g] = v + rv[g];
            }
          }
          store_group_buf<T, Elt>(yr, off, yv);
        }
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // Pipeline.  Stream stage j (weight, and x on the LDS path) is loaded DIST
  // stages ahead, at the top of stage j - DIST, into ring slot j % NS (the slot of
  // stage j - DIST - 1, which every wave has finished with once it passes that
  // stage's barrier).  Stage g multiplies weight stage g with the A fragments of x
  // stage g while the DFT of x stage g+1 (already in LDS) fills the other fragment
  // buffer.  At the top of stage g the loads issued after x stage g+1 are those of
  // stages g+2 .. g+DIST-1: WAIT_TOP of them may still be outstanding.  Register
  // path: x stage g+1 is loaded at the top of stage g, before the weight loads, and
  // waited for (all but the IPW weight loads behind it).
#pragma unroll
  for (int j = 0; j < DIST; ++j) issue_stage(j);
  if constexpr (XLDS) {
    wait_vmcnt<WAIT_PRO>();  // x stage 0
    read_xlds(0);
  } else {
    load_xreg(0);
    wait_vmcnt<0>();
  }
  transform(I0{});

  auto stage = [&](int g, auto curTag) __attribute__((always_inline)) {
    constexpr int cur = decltype(curTag)::value;
    using Cur = std::integral_constant<int, cur>;
    using Nxt = std::integral_constant<int, cur ^ 1>;
    wait_vmcnt<WAIT_TOP>();
    // Plain barrier (no fence): ring reads of stage g-1 have been consumed, and a
    // fence would also wait for the loads in flight.
    __builtin_amdgcn_s_barrier();
    if constexpr (XLDS) {
      issue_stage(g + DIST);
      read_xlds(g + 1);
    } else {
      load_xreg(g + 1);
      issue_stage(g + DIST);
      wait_vmcnt<IPW>();
    }

    const u32x4* slot = ringB[g % NS];
    u32x4 bcur[T], bnext[T];
    load_bfrag(bcur, slot, 0, 0);
#pragma unroll
    for (int idx = 0; idx < KS * NB; ++idx) {
      const int s = idx / NB, nb = idx % NB;
      if (idx + 1 < KS * NB) load_bfrag(bnext, slot, (idx + 1) / NB, (idx + 1) % NB);
      mfma_block(bcur, Cur{}, s, nb);
      if (idx == 0) transform(Nxt{});  // x stage g+1; overlaps the MFMA chains
      if (idx + 1 < KS * NB) {
#pragma unroll
        for (int p = 0; p < T; ++p) bcur[p] = bnext[p];
      }
    }
  };

  // nst is even (the packed input axis is a multiple of 4 groups, two per stage),
  // so every tile starts on fragment buffer 0.
  int g = 0;
  for (int k = 0; k < myTiles; ++k) {
    zero_acc();
    for (int st = 0; st < nst; st += 2, g += 2) {
      stage(g, I0{});
      stage(g + 1, I1{});
    }
    epilogue(k);
    lane = lane_index();
    lrow = lane & 31;
    khalf = lane >> 5;
    lane_offsets();
  }
  // Drain the look-ahead loads (all out of range) before the workgroup's LDS can
  // be reused.
  wait_vmcnt<0>();
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace eql

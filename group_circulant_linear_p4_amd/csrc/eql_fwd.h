// Fused forward kernels of the EQ-Linear layer: y = x W^T evaluated as
// group DFT (prologue) -> per-frequency channel GEMMs on MFMA -> inverse DFT
// (epilogue), with no intermediate global writes ("Implementacao" in "Resumo
// Tecnico: Flash EQ-Linear": fused data flow, Fourier fragments kept in registers
// and shared memory).  The input-gradient pass runs the same kernels on the
// conjugate-transposed packed weight.
//
// Work decomposition (gfx950, wave64, one persistent workgroup per CU):
//   * an output tile is 128 rows x BN = 32*NB output channels for all T planes; a
//     workgroup walks its tiles as one stream of K stages, so loads run ahead across
//     tile boundaries;
//   * a K stage is two 16-byte channel groups (one MFMA k-step);
//   * x of a stage (the tile's 128 rows x 2 groups) streams into an LDS ring by
//     buffer loads that write LDS directly (16-byte rows; otherwise each lane loads
//     its x straight into registers with narrower bounds-checked loads).  Lane l
//     takes row l%32 and channel group l/32 (G channels x T group elements) in MFMA
//     A-operand order; rows past N and channels past C' read as zero.  The group DFT
//     runs in fp32 registers and rounds once to the element type (p4 fp16: packed
//     fp16 butterflies, see dft_p4_f16); the negated Im planes needed by the real
//     part of each complex product are made by a sign flip;
//   * the packed spectrum of w streams into its own LDS ring, one contiguous run per
//     32-channel block and stage (see packed_unit);
//   * per k-step and 32-column block: real planes take one MFMA, a complex pair
//     four (Re += Xr Wr + (-Xi) Wi, Im += Xi Wr + Xr Wi);
//   * the epilogue reads the T accumulators of one (row, channel) from the same
//     register slot, applies the inverse DFT (its 1/T and 2/T are in the packed
//     weight) and stores T contiguous outputs; adjacent lanes write adjacent
//     channels.  EPI = 1 adds a per-channel bias, GELU and a residual first.
//
// eql_fwd4_kernel (T <= 4, 16-byte rows) is the fast path: a 4-slot ring walked by a
// loop unrolled over the slots, so every LDS read takes an immediate offset from one
// of two base registers and the stage bodies have no branches; 8 waves (two per SIMD,
// each with half the tile's columns) when the tile has two or more column blocks.
// eql_fwd_kernel serves every other T and unaligned rows.
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
  // Spectrum side output (eql_fwd4_kernel with SPEC = 1): the tiles of output column 0
  // also store the transformed input as weight-gradient operand units, unit
  // (kg, p, half, k) = plane p of input channel k for rows 16 kg + 8 half .. +7, at
  // byte ((kg T + p) 2 + half) specKpad 16 + 16 k; stores at or past specBytes are
  // dropped.
  void* spec;
  uint32_t specBytes;
  int specKpad;
  int specGrid;      // workgroups that take column 0's tiles (a multiple of 8)
};

constexpr int kFwdRows = 128;   // rows per workgroup (4 waves x 32)

#if defined(__HIP_DEVICE_COMPILE__)
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// p4 group DFT of 8 fp16 channels (raw[4q..4q+1] hold (x0,x1), (x2,x3) of channel 2q,
// raw[4q+2..4q+3] those of channel 2q+1) into the A-operand units X0, X2, Xr, Xi and
// -Xi (8 halves each), with instructions that issue alongside MFMAs (v_dot2 does not:
// on gfx950 it occupies the matrix pipeline and serialises with the MFMAs).
//   Everything is packed fp16 arithmetic, two channels or two group elements per op:
//   one addition per channel gives (x0 + x2, x1 + x3), one subtraction gives
//   (Xr, -Xi) = (x0 - x2, x1 - x3); X0 / X2 are the sum / difference of the two sums
//   (so X0 and X2 take two fp16 roundings, Xr and Xi one).  The 1/2 of the p4 forward
//   transform is folded into the packed weight's real planes.
__device__ __forceinline__ void dft_p4_f16(const uint32_t (&raw)[16], u32x4 (&out)[5]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // channel pair (2q, 2q+1) -> word q of each unit
    const uint32_t a0 = raw[4 * q + 0], b0 = raw[4 * q + 1];
    const uint32_t a1 = raw[4 * q + 2], b1 = raw[4 * q + 3];
    const f16x2 A0 = __builtin_bit_cast(f16x2, a0), B0 = __builtin_bit_cast(f16x2, b0);
    const f16x2 A1 = __builtin_bit_cast(f16x2, a1), B1 = __builtin_bit_cast(f16x2, b1);
    const f16x2 s0 = A0 + B0, s1 = A1 + B1;                  // (x0+x2, x1+x3) of channels 2q, 2q+1
    const f16x2 lo = __builtin_shufflevector(s0, s1, 0, 2);  // x0+x2 of both channels
    const f16x2 hi = __builtin_shufflevector(s0, s1, 1, 3);  // x1+x3 of both channels
    const f16x2 X0 = lo + hi, X2 = lo - hi;
    const f16x2 d0 = A0 - B0, d1 = A1 - B1;                  // (Xr, -Xi) of channels 2q, 2q+1
    const uint32_t nxi = __builtin_bit_cast(uint32_t, __builtin_shufflevector(d0, d1, 1, 3));
    out[0][q] = __builtin_bit_cast(uint32_t, X0);
    out[1][q] = __builtin_bit_cast(uint32_t, X2);
    out[2][q] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(d0, d1, 0, 2));
    out[3][q] = nxi ^ 0x80008000u;
    out[4][q] = nxi;
  }
}

// Transposes, in each aligned group of 8 lanes, the 8 x 8 block of 16-bit values
// held as four words per lane: on entry lane j holds row j (word q = elements 2q and
// 2q+1), on return column j (word q = rows 2q and 2q+1).  Three exchange rounds by
// DPP: lanes j and j^4 swap 4 x 4 blocks (row shifts by 4 lanes, each written only to
// the banks of 4 lanes that receive it), then inside each quad lanes r and r^2 swap
// 2 x 2 blocks and lanes r and r^1 swap 16-bit halves.  hi2: bit 1 of the lane index;
// sel: the last round's byte selector (0x05040100 on even lanes, 0x03020706 on odd).
__device__ __forceinline__ u32x4 transpose8_b16(const u32x4& v, bool hi2, uint32_t sel) {
  // Lanes 4-7 of each group take words 2, 3 of lane j-4 as their words 0, 1; lanes
  // 0-3 take words 0, 1 of lane j+4 as their words 2, 3.
  const uint32_t n0 = (uint32_t)__builtin_amdgcn_update_dpp((int)v[0], (int)v[2], 0x114, 0xf, 0xa, false);
  const uint32_t n1 = (uint32_t)__builtin_amdgcn_update_dpp((int)v[1], (int)v[3], 0x114, 0xf, 0xa, false);
  const uint32_t n2 = (uint32_t)__builtin_amdgcn_update_dpp((int)v[2], (int)v[0], 0x104, 0xf, 0x5, false);
  const uint32_t n3 = (uint32_t)__builtin_amdgcn_update_dpp((int)v[3], (int)v[1], 0x104, 0xf, 0x5, false);
  // A 4 x 4 block of one quad, lane r holding row r as words (a, b).
  auto quad = [&](uint32_t a, uint32_t b, uint32_t& oa, uint32_t& ob) __attribute__((always_inline)) {
    const uint32_t pa = (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x4E, 0xf, 0xf, false);  // lane r^2
    const uint32_t pb = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x4E, 0xf, 0xf, false);
    const uint32_t a2 = hi2 ? pb : a, b2 = hi2 ? b : pa;
    const uint32_t qa = (uint32_t)__builtin_amdgcn_mov_dpp((int)a2, 0xB1, 0xf, 0xf, false);  // lane r^1
    const uint32_t qb = (uint32_t)__builtin_amdgcn_mov_dpp((int)b2, 0xB1, 0xf, 0xf, false);
    oa = __builtin_amdgcn_perm(qa, a2, sel);
    ob = __builtin_amdgcn_perm(qb, b2, sel);
  };
  u32x4 o;
  uint32_t o0, o1, o2, o3;
  quad(n0, n1, o0, o1);
  quad(n2, n3, o2, o3);
  o[0] = o0;
  o[1] = o1;
  o[2] = o2;
  o[3] = o3;
  return o;
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

#if defined(__HIP_DEVICE_COMPILE__)
// Epilogue of one wave's part of a tile: rows row0 + rowOff .. +31, columns colBase ..
// colBase + 32 NBW - 1.  Accumulator slot r of lane l in block nb holds row
// 8 (r/4) + 4 (l/32) + r%4 and column colBase + 32 nb + l%32.  Stores go through a
// buffer descriptor covering the tile's valid rows; columns past D' take an offset
// beyond every range, so no store needs a branch.  EPI = 1 adds the per-channel bias,
// applies the activation and adds the residual (all in fp32) before the single
// rounding to Elt, and writes the activation's input to pre when that is given.
template <int T, typename Elt, int NBW, int EPI>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, const f32x16 (&acc)[T][NBW], int row0, int rowOff,
                                             int colBase) {
  constexpr int ELT = (int)sizeof(Elt);
  const uint32_t outRow = (uint32_t)a.Dout * T * ELT;  // bytes of one output row
  const uint32_t rows = (uint32_t)min(kFwdRows, a.N - row0);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(static_cast<char*>(a.y) + (size_t)row0 * outRow, rows * outRow);
  // The lane index is recomputed here rather than kept live through the main loop.
  const int ln = lane_index();
  const uint32_t laneOff = (uint32_t)(rowOff + 4 * (ln >> 5)) * outRow;
  // Fused epilogue operands: an absent bias or residual gets an empty range, so its
  // loads read zero.
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.bias, EPI && a.bias ? (uint32_t)a.Dout * ELT : 0u);
  const __amdgpu_buffer_rsrc_t rr =
      make_rsrc(EPI && a.res ? static_cast<const char*>(a.res) + (size_t)row0 * outRow : nullptr,
                EPI && a.res ? rows * outRow : 0u);
  const __amdgpu_buffer_rsrc_t pr =
      make_rsrc(EPI && a.pre ? static_cast<char*>(a.pre) + (size_t)row0 * outRow : nullptr,
                EPI && a.pre ? rows * outRow : 0u);
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int col = colBase + nb * 32 + (ln & 31);
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
    // stores (the compiler may not move a load above a store to y, which the residual
    // may alias), so one wait covers the chunk.
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
}
#endif

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
  static_assert(JC == 2 && (BN * RP) % 256 == 0 && (32 * RP) % 64 == 0, "tile shape (a stage is one packed chunk)");
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
  const uint32_t chunkBytes = (uint32_t)T * 1024u;         // one 32-channel block, one stage
  const uint32_t blockStride = (uint32_t)nst * chunkBytes;  // packed bytes per 32-channel block
  const int nblk = (a.Dout + 31) >> 5;

  auto tile_row0 = [&](int k) __attribute__((always_inline)) {
    return (xcd_remap(b0 + k * grid, a.numTiles) / a.colTiles) * kFwdRows;
  };
  auto tile_col0 = [&](int k) __attribute__((always_inline)) {
    const int t = xcd_remap(b0 + k * grid, a.numTiles);
    return (t - (t / a.colTiles) * a.colTiles) * BN;
  };

  // Weight ring: position P = (wave*IPW + i)*64 + lane of a stage holds unit
  // r = (P % RP) ^ ring_swz(o) (group r / T of the stage, plane r % T) of the tile's
  // output channel o = P / RP.  Offsets are relative to the stage's chunk of the
  // tile's first 32-channel block (see packed_unit); blocks past D' fall outside the
  // descriptor and read zero.
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
      const int ol = o & 31;
      bOff[i] = (uint32_t)(o >> 5) * blockStride + (uint32_t)(rr % T) * 1024u + (uint32_t)ol * 32u +
                (uint32_t)((rr / T) ^ ((ol >> 3) & 1)) * 16u;
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
      bTileBase = reinterpret_cast<uint64_t>(a.wp) + (uint64_t)(col0 >> 5) * blockStride;
      bTileBytes = (uint32_t)(min(NB, nblk - (col0 >> 5)) - 1) * blockStride + chunkBytes;
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
      // The tile's blocks from this stage's chunk on (an empty range past the stream).
      const BufDesc d = desc_at(bTileBase + (uint64_t)issSt * chunkBytes, issK < myTiles ? bTileBytes : 0u);
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

  auto epilogue = [&](int k) __attribute__((always_inline)) {
    fwd_epilogue<T, Elt, NB, EPI>(a, acc, tile_row0(k), wave * 32, tile_col0(k));
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

// Waves per workgroup of eql_fwd4_kernel: two per SIMD (each with half the tile's
// column blocks) when the tile has two column blocks or more, else one.  With T = 3 and
// four blocks the weight stage (12 KB) does not split into whole 1 KB loads over 8 waves.
__host__ __device__ constexpr int fwd4_waves(int T, int NB) { return NB >= 2 && !(T == 3 && NB == 4) ? 8 : 4; }

// The fast forward kernel for T <= 4 and 16-byte-aligned rows (see the file comment).
//   * Ring: 4 slots of (weight stage, x stage).  Stage g of the workgroup's stream
//     lives in slot g % 4 and is loaded 3 stages ahead.  The loop body is unrolled over
//     the 4 slots; nst is even, so a tile starts at slot 0 or 2 ("phase").  Slots 0, 1
//     of the body live at pair base A (physical slots phase, phase + 1), slots 2, 3 at
//     pair base B; both bases are kept per lane for reads and per wave for DMA, so every
//     LDS address is a base register plus an immediate.
//   * Weight DMA: a stage of the tile is NB contiguous T KB chunks (packed_unit); wave w
//     loads IPW consecutive KB of it with one M0 write.  x DMA: the tile's 128 rows x
//     128 bytes (p4 fp16) in 1 KB loads spread over the waves.
//   * Issue state (next stage's weight and x addresses, x bytes left in the tile) is
//     bumped by constants per stage; the one tile boundary the issue side crosses
//     during a compute tile switches to the next tile's state, prepared at the compute
//     tile's start, by scalar selects: the stage bodies have no branches, so the
//     compiler keeps the next stage's transform interleaved with the MFMAs.
//   * Stage g: read block 0's weight fragments (landed before the previous barrier),
//     wait for this wave's loads of stage g+1, barrier, issue stage g+3, read x of
//     stage g+1, then per column block: next block's fragments, the block's MFMAs,
//     and after block 0 the transform of x stage g+1 into the other fragment buffer.
//   * SPEC = 1 (p4 fp16, either epilogue): the workgroups below FwdArgs::specGrid take the
//     tiles of output column 0 and run the loop with the spectrum side output; the others
//     take the remaining columns with the plain loop.  In the storing loop each wave also
//     transposes its transformed x fragments (8 rows x 8 channels per 8 lanes, by DPP)
//     and stores them as weight-gradient operand units (FwdArgs::spec), two planes per
//     wave with 8 waves, at the end of each stage.  Vector-memory loads (LDS DMA
//     included) and stores retire in issue order on this counter, so each stage's
//     wait leaves the previous stage's stores outstanding as well as the next stage's
//     loads.
#if defined(__HIP_DEVICE_COMPILE__)
// One workgroup's persistent loop of eql_fwd4_kernel: workgroup b0 of `grid` takes the
// tiles xcd_remap(b0 + k grid) of `numTiles`, which cover output column tiles
// colTile0 .. colTile0 + colTiles - 1 of every row tile; LDS rings at byte addresses
// ldsB (weight) and ldsX (x).  SPEC: also store the transformed x (see above).
template <int T, typename Elt, int NB, int LOAD, int EPI, bool SPEC>
__device__ __forceinline__ void fwd4_body(const FwdArgs& a, uint32_t ldsB, uint32_t ldsX, int b0, int grid,
                                          int numTiles, int colTile0, int colTiles) {
  using E = EltT<Elt>;
  constexpr int WAVES = fwd4_waves(T, NB);
  constexpr int G = E::kPerUnit;
  constexpr int NR = n_real_planes(T);
  constexpr int NP = n_pairs(T);
  constexpr int BN = 32 * NB;
  constexpr int NBW = NB * 4 / WAVES;      // column blocks per wave
  constexpr int RP = 8;                    // x ring row: 2T <= 8 units
  constexpr int ELT = (int)sizeof(Elt);
  constexpr int NS = 4, DIST = 3;
  constexpr int BKB = NB * T;              // KB of packed weight per stage
  constexpr int BSLOT = BKB * 1024;
  constexpr int XSLOT = kFwdRows * RP * 16;
  constexpr int IPW = BKB >= WAVES ? BKB / WAVES : 1;  // weight DMA loads per wave per stage
  constexpr int IPWX = kFwdRows * RP / 64 / WAVES;     // x DMA loads per wave per stage
  constexpr int SB = 2 * G * T * ELT;                  // bytes of one x row per stage
  static_assert(T <= 4 && LOAD != kLoadNarrow && NBW >= 1, "fast path: T <= 4, 16-byte rows");
  static_assert(BKB < WAVES || BKB % WAVES == 0, "whole 1 KB weight loads per wave");
  // A wave's run of IPW KB starts at KB qw % T of a block's T KB chunk and must end
  // inside it: the packed weight is block-major, so the next KB belongs to another
  // stage (and past the last block, to no buffer at all).
  static_assert(BKB < WAVES || (IPW <= T && T % IPW == 0), "weight run inside one block's chunk");
  static_assert(IPW <= 4 || IPW == 6 || IPW == 8, "weight run length");
  static_assert(IPWX == 2 || IPWX == 4, "x loads per wave");
  static_assert(NS * (BSLOT + XSLOT) <= 160 * 1024, "LDS budget");
  // Per-slot immediate offsets stay below 64 KB: slot pairs are 2 slots apart.
  static_assert(BSLOT + BKB * 1024 <= 65536 && XSLOT + XSLOT <= 65536, "ds_read offset range");
  constexpr int WAIT_TOP = (DIST - 2) * (IPW + IPWX);
  constexpr int WAIT_PRO = (DIST - 1) * (IPW + IPWX);
  static_assert(WAIT_PRO < 64, "vmcnt range");
  static_assert(!SPEC || (T == 4 && ELT == 2), "spectrum side output: p4 fp16");

  if (b0 >= numTiles) return;
  const int myTiles = (numTiles - b0 + grid - 1) / grid;
  const int nst = a.Jpad / 2;
  const int nblk = (a.Dout + 31) >> 5;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rb = wave & 3;                 // 32-row block of the tile
  const int cb = WAVES == 8 ? wave >> 2 : 0;  // column half (8 waves)
  // This wave's weight KBs of a stage: q = qw .. qw + IPW - 1 (block q / T, KB q % T).
  const int qw = BKB >= WAVES ? wave * IPW : wave % BKB;
  const int cw = qw / T, kbw = qw - cw * T;
  const uint32_t rowBytes = (uint32_t)a.Cin * T * ELT;
  const uint64_t chunkStride = (uint64_t)T * 1024;
  const uint64_t blockStride = (uint64_t)nst * chunkStride;

  auto tile_of = [&](int k) __attribute__((always_inline)) { return xcd_remap(b0 + k * grid, numTiles); };

  // Lane-derived values, re-derived after every epilogue (none is live there; see
  // eql_fwd_kernel).
  int phase = 0;
  uint32_t bRdA, bRdB, xRdA[T], xRdB[T], bVoff, xOff[IPWX];
  int xCh[IPWX];
  auto lane_setup = [&]() __attribute__((always_inline)) {
    const int lane = lane_index();
    const int lrow = lane & 31, khalf = lane >> 5;
    bVoff = (uint32_t)lane * 16u;
    const uint32_t pa = (uint32_t)phase, pb = (uint32_t)((phase + 2) & 3);
    // Weight fragment (block 0, plane 0) of this lane: channel lrow of the block, group
    // khalf of the stage (packed_unit's order within a chunk).
    const uint32_t bl = (uint32_t)(lrow * 32 + ((khalf ^ ((lrow >> 3) & 1)) * 16));
    bRdA = ldsB + pa * BSLOT + bl;
    bRdB = ldsB + pb * BSLOT + bl;
    const int row = rb * 32 + lrow;
#pragma unroll
    for (int v = 0; v < T; ++v) {
      const int u = khalf * T + v;
      const uint32_t xl = (uint32_t)((row * RP + (u ^ ring_swz<RP>(row))) * 16);
      xRdA[v] = ldsX + pa * XSLOT + xl;
      xRdB[v] = ldsX + pb * XSLOT + xl;
    }
    // x DMA: ring position P = (wave IPWX + i) 64 + lane holds unit (P % RP) ^ swz of
    // row P / RP (padding units past 2T load an arbitrary unit of the row).
#pragma unroll
    for (int i = 0; i < IPWX; ++i) {
      const int P = (wave * IPWX + i) * 64 + lane;
      const int rw = P / RP, pos = P - rw * RP;
      const int u = pos ^ ring_swz<RP>(rw);
      const int uu = u < 2 * T ? u : 0;
      xOff[i] = (uint32_t)rw * rowBytes + (uint32_t)uu * 16u;
      xCh[i] = (uu * 16) / (T * ELT);
    }
  };
  lane_setup();

  // Issue side.
  int issSt = 0, issK = 0;
  uint64_t bCur = 0, xCur = 0, nbCur = 0, nxCur = 0;
  uint32_t bLen = 0, xLeft = 0, nbLen = 0, nxLeft = 0;
  auto tile_state = [&](int k, uint64_t& bc, uint32_t& bl, uint64_t& xc, uint32_t& xl) __attribute__((always_inline)) {
    if (k < myTiles) {
      const int t = tile_of(k);
      const int rt = t / colTiles;
      const int row0 = rt * kFwdRows, col0 = (colTile0 + t - rt * colTiles) * BN;
      const int ob = (col0 >> 5) + cw;
      bc = reinterpret_cast<uint64_t>(a.wp) + (uint64_t)ob * blockStride + (uint64_t)kbw * 1024;
      bl = ob < nblk ? (uint32_t)(IPW * 1024) : 0u;
      xc = reinterpret_cast<uint64_t>(a.x) + (uint64_t)row0 * rowBytes;
      xl = (uint32_t)min(kFwdRows, a.N - row0) * rowBytes;
    } else {
      bc = xc = 0;
      bl = xl = 0;
    }
  };
  tile_state(0, bCur, bLen, xCur, xLeft);
  uint32_t bDmaA, bDmaB, xDmaA, xDmaB;
  auto ring_setup = [&]() __attribute__((always_inline)) {
    const uint32_t pa = (uint32_t)phase, pb = (uint32_t)((phase + 2) & 3);
    bDmaA = ldsB + pa * BSLOT + (uint32_t)qw * 1024u;
    bDmaB = ldsB + pb * BSLOT + (uint32_t)qw * 1024u;
    xDmaA = ldsX + pa * XSLOT + (uint32_t)(wave * IPWX * 1024);
    xDmaB = ldsX + pb * XSLOT + (uint32_t)(wave * IPWX * 1024);
  };
  ring_setup();
  auto issue = [&](auto slotTag) __attribute__((always_inline)) {
    constexpr int S = decltype(slotTag)::value;
    dma16_run<IPW, (S & 1) * BSLOT>(desc_words(bCur, bLen), bVoff, S < 2 ? bDmaA : bDmaB);
    {
      uint32_t off[IPWX];
      const int c0 = issSt * 2 * G;
#pragma unroll
      for (int i = 0; i < IPWX; ++i) off[i] = (LOAD == kLoadFull || c0 + xCh[i] < a.Cin) ? xOff[i] : kOob;
      dma16_each<IPWX, (S & 1) * XSLOT>(desc_words(xCur, xLeft), off, S < 2 ? xDmaA : xDmaB);
    }
    bCur += chunkStride;
    xCur += SB;
    xLeft = xLeft > (uint32_t)SB ? xLeft - SB : 0u;
    const bool wrap = ++issSt == nst;
    issSt = wrap ? 0 : issSt;
    issK = wrap ? issK + 1 : issK;
    bCur = wrap ? nbCur : bCur;
    bLen = wrap ? nbLen : bLen;
    xCur = wrap ? nxCur : xCur;
    xLeft = wrap ? nxLeft : xLeft;
  };

  auto rd = [&](uint32_t addr, int imm) __attribute__((always_inline)) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        (const __attribute__((address_space(3))) char*)(uintptr_t)addr + imm);
  };

  uint32_t raw[4 * T];
  u32x4 af[2][T + NP];
  auto read_x = [&](auto slotTag) __attribute__((always_inline)) {
    constexpr int S = decltype(slotTag)::value;
#pragma unroll
    for (int v = 0; v < T; ++v) {
      const u32x4 val = rd(S < 2 ? xRdA[v] : xRdB[v], (S & 1) * XSLOT);
      raw[4 * v + 0] = val[0];
      raw[4 * v + 1] = val[1];
      raw[4 * v + 2] = val[2];
      raw[4 * v + 3] = val[3];
    }
  };
  auto transform = [&](auto abTag) __attribute__((always_inline)) {
    constexpr int ab = decltype(abTag)::value;
    if constexpr (T == 4 && ELT == 2) {
      dft_p4_f16(raw, af[ab]);
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
      for (int q = 0; q < NP; ++q) af[ab][T + q] = neg_unit(af[ab][NR + 2 * q + 1], E::kSignMask);
    }
  };

  // Spectrum side output state (SPEC: set at each tile's start, dead before its epilogue).
  uint32_t specCur = 0, specSel = 0;
  bool specHi2 = false;
  constexpr int PPW = WAVES == 8 ? T / 2 : T;  // planes stored per wave
  const uint32_t specRow = (uint32_t)a.specKpad * 16u;  // bytes of one (kg, p, half) run
  auto spec_setup = [&](int rt) __attribute__((always_inline)) {
    const int lane = lane_index();
    const int lrow = lane & 31;
    const int rbase = rt * kFwdRows + rb * 32 + (lrow & 24);  // first row of the lane's 8-row group
    specCur = ((uint32_t)(rbase >> 4) * (2u * T) + (uint32_t)((rbase >> 3) & 1)) * specRow +
              (uint32_t)((lane >> 5) * 8 + (lrow & 7)) * 16u;
    specHi2 = (lane & 2) != 0;
    specSel = (lane & 1) ? 0x03020706u : 0x05040100u;
  };
  auto store_spec = [&](const u32x4 (&f)[T + NP]) __attribute__((always_inline)) {
    if constexpr (SPEC) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(a.spec, a.specBytes);
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        u32x4 v;
        if constexpr (PPW == T) {
          v = f[i];
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) v[w] = cb ? f[PPW + i][w] : f[i][w];
        }
        const int p = cb * PPW + i;
        __builtin_amdgcn_raw_buffer_store_b128(transpose8_b16(v, specHi2, specSel), r, specCur,
                                               (int)((uint32_t)p * 2u * specRow), kStoreNT);
      }
      specCur += 2u * G * 16u;  // the next stage's 16 channels
    }
  };

  f32x16 acc[T][NBW];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < T; ++p)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) E::zero(acc[p][nb]);
  };

  auto stage = [&](auto slotTag) __attribute__((always_inline)) {
    constexpr int S = decltype(slotTag)::value;
    constexpr int cur = S & 1;
    using Nxt = std::integral_constant<int, cur ^ 1>;
    using SN = std::integral_constant<int, (S + 1) % NS>;
    using SI = std::integral_constant<int, (S + DIST) % NS>;
    u32x4 bf[2][T];
#pragma unroll
    for (int p = 0; p < T; ++p) bf[0][p] = rd(S < 2 ? bRdA : bRdB, (S & 1) * BSLOT + (cb * NBW * T + p) * 1024);
    // With the spectrum side output the previous stage's PPW stores were issued after
    // this stage's look-ahead loads; vector-memory operations retire in issue order, so
    // leaving them outstanding still means that stage g+1's loads have landed.
    wait_vmcnt<SPEC ? WAIT_TOP + PPW : WAIT_TOP>();
    // Plain barrier (no fence): the ring reads of stage g-1 are consumed, and a fence
    // would also wait for the loads in flight.
    __builtin_amdgcn_s_barrier();
    issue(SI{});
    read_x(SN{});
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (nb + 1 < NBW) {
#pragma unroll
        for (int p = 0; p < T; ++p)
          bf[(nb + 1) & 1][p] = rd(S < 2 ? bRdA : bRdB, (S & 1) * BSLOT + ((cb * NBW + nb + 1) * T + p) * 1024);
      }
      const u32x4(&b)[T] = bf[nb & 1];
#pragma unroll
      for (int p = 0; p < NR; ++p) E::mfma(acc[p][nb], af[cur][p], b[p]);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int re = NR + 2 * q, im = re + 1;
        E::mfma(acc[re][nb], af[cur][re], b[re]);
        E::mfma(acc[re][nb], af[cur][T + q], b[im]);
        E::mfma(acc[im][nb], af[cur][im], b[re]);
        E::mfma(acc[im][nb], af[cur][re], b[im]);
      }
      if (nb == 0) transform(Nxt{});  // x stage g+1; overlaps the MFMA chains
    }
    if constexpr (SPEC) store_spec(af[cur]);  // x stage g, as weight-gradient units
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // Prologue: stages 0..2 into slots 0..2 (with nst = 2 the third is tile 1's stage 0),
  // then x of stage 0.
  tile_state(1, nbCur, nbLen, nxCur, nxLeft);
  issue(I0{});
  issue(I1{});
  issue(I2{});
  wait_vmcnt<WAIT_PRO>();
  __builtin_amdgcn_s_barrier();
  read_x(I0{});
  transform(I0{});
  // The first stage's wait counts stores that were never issued: wait for stage 1 here.
  if constexpr (SPEC) wait_vmcnt<WAIT_TOP>();

  for (int k = 0; k < myTiles; ++k) {
    // During this tile's nst stages the issue side crosses exactly one tile boundary.
    tile_state(issK + 1, nbCur, nbLen, nxCur, nxLeft);
    zero_acc();
    if constexpr (SPEC) spec_setup(tile_of(k) / colTiles);
    int st = 0;
    for (; st + 4 <= nst; st += 4) {
      stage(I0{});
      stage(I1{});
      stage(I2{});
      stage(I3{});
    }
    if (st < nst) {  // nst = 2 (mod 4): the next tile starts two slots on
      stage(I0{});
      stage(I1{});
    }
    phase = (phase + nst) & 3;
    ring_setup();
    const int t = tile_of(k);
    const int rt = t / colTiles;
    fwd_epilogue<T, Elt, NBW, EPI>(a, acc, rt * kFwdRows, rb * 32,
                                   (colTile0 + t - rt * colTiles) * BN + cb * NBW * 32);
    lane_setup();
  }
  // Drain the look-ahead loads (all out of range) before the workgroup's LDS can be
  // reused.
  wait_vmcnt<0>();
}
#endif  // __HIP_DEVICE_COMPILE__

template <int T, typename Elt, int NB, int LOAD, int EPI, int SPEC = 0>
__global__ void __launch_bounds__(64 * fwd4_waves(T, NB)) eql_fwd4_kernel(const FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NS = 4;
  constexpr int BSLOT = NB * T * 1024;
  constexpr int XSLOT = kFwdRows * 8 * 16;
  __shared__ u32x4 ringB[NS][BSLOT / 16];
  __shared__ u32x4 ringX[NS][XSLOT / 16];
  const uint32_t lb = lds_addr(&ringB[0][0]), lx = lds_addr(&ringX[0][0]);
  const int b = blockIdx.x;
  if constexpr (SPEC) {
    // Workgroups below specGrid (a multiple of the 8 XCDs, as is the rest) take column
    // 0's tiles and store the spectrum; the others take the remaining columns.  Each
    // part walks its own tiles in the XCD-aware order, and both visit the row tiles in
    // the same order, so the two parts of an XCD read the same rows of x.
    const int rowTiles = a.numTiles / a.colTiles;
    if (b < a.specGrid)
      fwd4_body<T, Elt, NB, LOAD, EPI, true>(a, lb, lx, b, a.specGrid, rowTiles, 0, 1);
    else
      fwd4_body<T, Elt, NB, LOAD, EPI, false>(a, lb, lx, b - a.specGrid, (int)gridDim.x - a.specGrid,
                                              rowTiles * (a.colTiles - 1), 1, a.colTiles - 1);
  } else {
    fwd4_body<T, Elt, NB, LOAD, EPI, false>(a, lb, lx, b, (int)gridDim.x, a.numTiles, 0, a.colTiles);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace eql

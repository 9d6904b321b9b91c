// Device-side building blocks of the EQ-Linear kernels for gfx950: vector types,
// the MFMA step, the group-axis transforms and the vectorised loads/stores.
//
// Plane convention (the real half spectrum along the group axis, "Abordagem
// Algoritmica" in "Resumo Tecnico: Flash EQ-Linear"): a length-T group vector v is
// represented by T real planes
//   p = 0                    k = 0       sum_h v_h
//   p = 1 (even T > 1)       k = T/2     sum_h (-1)^h v_h
//   p = NR + 2q, NR + 2q + 1 k = q + 1   Re / Im of sum_h v_h exp(-2 pi i h k / T)
// where NR is the number of real planes.  The packed weight of the forward and
// input-gradient kernels carries the inverse transform's scale (1/T on the real
// planes, 2/T on the complex ones), so neither the activation transform nor the
// epilogue's inverse multiplies by it; for p4 every coefficient left is 0 or +-1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eql {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxT = 16;

__host__ __device__ constexpr int n_real_planes(int T) { return (T % 2 == 0 && T > 1) ? 2 : 1; }
__host__ __device__ constexpr int n_pairs(int T) { return (T - n_real_planes(T)) / 2; }

// cos / sin of 2*pi*m/T for m = 0..T-1, computed on the host in double and rounded
// once to float.  Passed as a kernel argument, so the values live in scalar
// registers.  Entries whose exact value is 0 or +-1 are never read: those cases are
// folded at compile time (see acc_cos / acc_msin).
struct Twiddles {
  float cs[kMaxT];
  float sn[kMaxT];
  float inv_t;  // 1/T rounded to float
};

// Twiddle sums.  s accumulates v * cos(2 pi m / T) (acc_cos) or -v * sin(2 pi m / T)
// (acc_msin), with the exact coefficient when it is 0 or +-1; `any` says whether s
// holds a term yet.  The first term is taken as it is rather than added to zero:
// 0 + t differs from t only in the sign of a zero, so the compiler may not drop
// that addition, and it would cost one instruction per sum.  m and `any` are
// compile-time constants once the callers' loops are unrolled.
template <int T>
__device__ __forceinline__ void acc_cos(float& s, bool& any, float v, int m, const Twiddles& tw) {
  m %= T;
  if (4 * m == T || 4 * m == 3 * T) return;
  if (m == 0) s = any ? s + v : v;
  else if (2 * m == T) s = any ? s - v : -v;
  else s = any ? __builtin_fmaf(v, tw.cs[m], s) : v * tw.cs[m];
  any = true;
}

template <int T>
__device__ __forceinline__ void acc_msin(float& s, bool& any, float v, int m, const Twiddles& tw) {
  m %= T;
  if (m == 0 || 2 * m == T) return;
  if (4 * m == T) s = any ? s - v : -v;
  else if (4 * m == 3 * T) s = any ? s + v : v;
  else s = any ? __builtin_fmaf(-v, tw.sn[m], s) : -v * tw.sn[m];
  any = true;
}

// ---------------------------------------------------------------------------
// Forward group transform of one length-T vector into T (unscaled) planes.
// ---------------------------------------------------------------------------
template <int T>
struct Dft {
  static __device__ __forceinline__ void run(const float (&v)[T], float (&out)[T],
                                             const Twiddles& tw) {
    constexpr int NR = n_real_planes(T);
#pragma unroll
    for (int p = 0; p < T; ++p) {
      const int k = p == 0 ? 0 : (p < NR ? T / 2 : (p - NR) / 2 + 1);
      const bool im = p >= NR && ((p - NR) & 1);
      float s = 0.0f;
      bool any = false;
#pragma unroll
      for (int h = 0; h < T; ++h) {
        if (im) acc_msin<T>(s, any, v[h], h * k, tw);
        else acc_cos<T>(s, any, v[h], h * k, tw);
      }
      out[p] = s;
    }
  }
};

// p4: butterflies only.  The additions are ordered so that a cyclic shift of v
// permutes / negates the outputs exactly in floating point:
//   shift by one maps (X0, X2, Xr, Xi) to (X0, -X2, Xi, -Xr).
template <>
struct Dft<4> {
  static __device__ __forceinline__ void run(const float (&v)[4], float (&out)[4], const Twiddles&) {
    const float s02 = v[0] + v[2], d02 = v[0] - v[2];
    const float s13 = v[1] + v[3], d13 = v[3] - v[1];
    out[0] = s02 + s13;
    out[1] = s02 - s13;
    out[2] = d02;
    out[3] = d13;
  }
};

// ---------------------------------------------------------------------------
// Inverse transform of T planes back to T group values.
// kPlain = true: the plain inverse of unscaled planes,
//   y_g = (1/T) (P0 + (-1)^g P_N + 2 sum_k (cos P_re - sin P_im)).
// kPlain = false: the forward / input-gradient epilogue, whose planes already
// carry 1/T (real) and 2/T (complex) from the packed weight,
//   y_g = P0 + (-1)^g P_N + sum_k (cos P_re - sin P_im).
// ---------------------------------------------------------------------------
template <int T, bool kPlain>
struct Idft {
  static __device__ __forceinline__ void run(const float (&P)[T], float (&y)[T], const Twiddles& tw) {
    constexpr int NR = n_real_planes(T);
#pragma unroll
    for (int g = 0; g < T; ++g) {
      float s = P[0];
      if (NR == 2) s = (g & 1) ? s - P[1] : s + P[1];
      float u = 0.0f;
      bool any = false;
#pragma unroll
      for (int q = 0; q < n_pairs(T); ++q) {
        acc_cos<T>(u, any, P[NR + 2 * q], g * (q + 1), tw);
        acc_msin<T>(u, any, P[NR + 2 * q + 1], g * (q + 1), tw);
      }
      if (any) s = kPlain ? s + 2.0f * u : s + u;
      y[g] = kPlain ? s * tw.inv_t : s;
    }
  }
};

// ---------------------------------------------------------------------------
// Element types.  A "unit" is 16 bytes: 8 fp16 or 4 fp32 values.
// ---------------------------------------------------------------------------
template <typename Elt>
struct EltT;

template <>
struct EltT<_Float16> {
  static constexpr int kPerUnit = 8;
  static constexpr uint32_t kSignMask = 0x80008000u;
  static __device__ __forceinline__ float get(const u32x4& u, int e) {
    return (float)__builtin_bit_cast(f16x8, u)[e];
  }
  static __device__ __forceinline__ u32x4 pack(const float (&v)[8]) {
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)v[e];
    return __builtin_bit_cast(u32x4, h);
  }
  // One k-step: 32x32 output tile += A(32 x 16) * B(16 x 32).
  static __device__ __forceinline__ void mfma(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
  // Clear a 32x32 tile with one MFMA of zero operands (exact +0).  The zero operand
  // comes from a volatile move, so separate tiles get separate MFMAs: a constant
  // would be rematerialised as 16 register writes per tile (and, as generated,
  // twice).  An MFMA that reads a VGPR written by a VALU instruction needs wait
  // states in between, and the compiler's hazard check does not see a VALU write
  // inside an asm statement (it then emitted a single wait state, and the MFMA
  // could read the register's previous contents), so the statement carries its
  // own: five, a margin over the two the hazard requires.
  static __device__ __forceinline__ void zero(f32x16& acc) {
    uint32_t z0;
    asm volatile("v_mov_b32 %0, 0\n\ts_nop 4" : "=v"(z0));
    const f16x8 z = __builtin_bit_cast(f16x8, (u32x4){z0, z0, z0, z0});
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, z, (f32x16){}, 0, 0, 0);
  }
};

template <>
struct EltT<float> {
  static constexpr int kPerUnit = 4;
  static constexpr uint32_t kSignMask = 0x80000000u;
  static __device__ __forceinline__ float get(const u32x4& u, int e) {
    return __builtin_bit_cast(f32x4, u)[e];
  }
  static __device__ __forceinline__ u32x4 pack(const float (&v)[4]) {
    f32x4 f = {v[0], v[1], v[2], v[3]};
    return __builtin_bit_cast(u32x4, f);
  }
  // One k-step: four 32x32x2 products; element e of each lane's unit feeds product e.
  static __device__ __forceinline__ void mfma(f32x16& acc, const u32x4& a, const u32x4& b) {
    const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[0], bf[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[1], bf[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[2], bf[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[3], bf[3], acc, 0, 0, 0);
  }
  static __device__ __forceinline__ void zero(f32x16& acc) {  // see EltT<_Float16>::zero
    float z0;
    asm volatile("v_mov_b32 %0, 0\n\ts_nop 4" : "=v"(z0));
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(z0, z0, (f32x16){}, 0, 0, 0);
  }
};

__device__ __forceinline__ u32x4 neg_unit(const u32x4& u, uint32_t mask) {
  return u ^ (u32x4){mask, mask, mask, mask};
}

// Largest power of two dividing n, capped at 16 (the widest global access).
__host__ __device__ constexpr int pow2_part(int n) {
  return (n % 16 == 0) ? 16 : (n % 8 == 0) ? 8 : (n % 4 == 0) ? 4 : (n % 2 == 0) ? 2 : 1;
}

// Load NB bytes (a power of two <= 16) from a suitably aligned address into the
// low bytes of a u32x4.
template <int NBYTES>
__device__ __forceinline__ void load_bytes(const void* p, uint32_t* dst) {
  if constexpr (NBYTES == 16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
  } else if constexpr (NBYTES == 8) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    dst[0] = v[0]; dst[1] = v[1];
  } else if constexpr (NBYTES == 4) {
    dst[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    static_assert(NBYTES == 2, "unsupported width");
    dst[0] = *reinterpret_cast<const uint16_t*>(p);
  }
}

// Read T contiguous elements starting at `p` (aligned to pow2_part(T*sizeof(Elt)))
// into floats.
template <int T, typename Elt>
__device__ __forceinline__ void load_group(const Elt* p, float (&v)[T]) {
  constexpr int BYTES = T * (int)sizeof(Elt);
  constexpr int W = pow2_part(BYTES);
  constexpr int WORDS = (BYTES + 3) / 4;
  uint32_t w[WORDS > 0 ? WORDS : 1];
#pragma unroll
  for (int i = 0; i < WORDS; ++i) w[i] = 0;
  if constexpr (W >= 4) {
#pragma unroll
    for (int b = 0; b < BYTES; b += W) load_bytes<W>(reinterpret_cast<const char*>(p) + b, &w[b / 4]);
  } else {
    // 2-byte granularity (fp16 with odd T): assemble half-words.
#pragma unroll
    for (int e = 0; e < T; ++e) {
      const uint32_t hv = *reinterpret_cast<const uint16_t*>(p + e);
      w[e / 2] |= (e & 1) ? (hv << 16) : hv;
    }
  }
#pragma unroll
  for (int e = 0; e < T; ++e) {
    if constexpr (sizeof(Elt) == 2) {
      const uint16_t bits = (uint16_t)(w[e / 2] >> ((e & 1) * 16));
      v[e] = (float)__builtin_bit_cast(_Float16, bits);
    } else {
      v[e] = __builtin_bit_cast(float, w[e]);
    }
  }
}

// Write T floats, rounded to Elt (nearest even), as contiguous elements at `p`
// (aligned to pow2_part(T*sizeof(Elt))).
template <int T, typename Elt>
__device__ __forceinline__ void store_group(Elt* p, const float (&v)[T]) {
  constexpr int BYTES = T * (int)sizeof(Elt);
  constexpr int W = pow2_part(BYTES);
  if constexpr (W >= 4) {
    constexpr int WORDS = BYTES / 4;
    uint32_t w[WORDS];
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      if constexpr (sizeof(Elt) == 2) {
        const _Float16 lo = (_Float16)v[2 * i], hi = (_Float16)v[2 * i + 1];
        w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      } else {
        w[i] = __builtin_bit_cast(uint32_t, v[i]);
      }
    }
    char* b = reinterpret_cast<char*>(p);
#pragma unroll
    for (int off = 0; off < BYTES; off += W) {
      if constexpr (W == 16) {
        *reinterpret_cast<u32x4*>(b + off) = (u32x4){w[off / 4], w[off / 4 + 1], w[off / 4 + 2], w[off / 4 + 3]};
      } else if constexpr (W == 8) {
        *reinterpret_cast<u32x2*>(b + off) = (u32x2){w[off / 4], w[off / 4 + 1]};
      } else {
        *reinterpret_cast<uint32_t*>(b + off) = w[off / 4];
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < T; ++e) p[e] = (Elt)v[e];
  }
}

// Index of the calling lane in its wave (0..63), computed afresh at each call: an
// asm statement, so the compiler cannot merge it with an earlier value and keep
// that one live instead.
__device__ __forceinline__ int lane_index() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// XCD-aware tile order.  Consecutive workgroup ids are dispatched round-robin over
// the 8 XCDs; this remaps them so that each XCD receives a contiguous range of
// logical tiles (and so shares row blocks of the input in its own L2).
__device__ __forceinline__ int xcd_remap(int b, int num) {
  constexpr int kXcd = 8;
  const int per = num / kXcd, rem = num % kXcd;
  const int xcd = b % kXcd, local = b / kXcd;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

}  // namespace eql

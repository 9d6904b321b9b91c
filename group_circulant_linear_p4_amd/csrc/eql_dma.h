// Buffer-descriptor loads, including loads that write LDS directly, for gfx950.
#pragma once

#include "eql_device.h"

namespace eql {

// s_waitcnt on vector-memory loads only (lgkm and exp counters left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): every LDS read of this wave has returned.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
}

// Cache-policy operand of a buffer store: NT (non-temporal) on gfx940-family parts.
constexpr int kStoreNT = 2;

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Stores the T values of one group (rounded to Elt) at byte offset `off` of buffer
// `r`; accesses at or beyond the buffer's range are dropped by the hardware, so the
// caller masks rows and columns through the offset instead of a branch.  The stores
// are non-temporal (cache policy NT): outputs are written once and not read again
// by the kernel, and streaming them past the caches leaves L2 to the operands.
template <int T, typename Elt>
__device__ __forceinline__ void store_group_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&v)[T]) {
  constexpr int BYTES = T * (int)sizeof(Elt);
  constexpr int W = pow2_part(BYTES);
  if constexpr (W >= 4) {
    constexpr int WORDS = BYTES / 4;
    uint32_t w[WORDS];
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      if constexpr (sizeof(Elt) == 2) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 pr = {(_Float16)v[2 * i], (_Float16)v[2 * i + 1]};  // one packed RNE convert
        w[i] = __builtin_bit_cast(uint32_t, pr);
      } else {
        w[i] = __builtin_bit_cast(uint32_t, v[i]);
      }
    }
#pragma unroll
    for (int b = 0; b < BYTES; b += W) {
      if constexpr (W == 16) {
        __builtin_amdgcn_raw_buffer_store_b128((u32x4){w[b / 4], w[b / 4 + 1], w[b / 4 + 2], w[b / 4 + 3]}, r,
                                               off + b, 0, kStoreNT);
      } else if constexpr (W == 8) {
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){w[b / 4], w[b / 4 + 1]}, r, off + b, 0, kStoreNT);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(w[b / 4], r, off + b, 0, kStoreNT);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < T; ++e)
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (Elt)v[e]), r, off + 2 * e, 0, kStoreNT);
  }
}

// Raw 32-bit words of one group (the counterpart of store_group_buf): T * size
// bytes in the widest aligned loads; with 2-byte loads, one value per word.
// Out-of-range accesses read zero.
template <int T, typename Elt>
__host__ __device__ constexpr int group_words() {
  return pow2_part(T * (int)sizeof(Elt)) >= 4 ? T * (int)sizeof(Elt) / 4 : T;
}

template <int T, typename Elt>
__device__ __forceinline__ void load_group_raw(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               uint32_t (&w)[group_words<T, Elt>()]) {
  constexpr int BYTES = T * (int)sizeof(Elt);
  constexpr int W = pow2_part(BYTES);
  if constexpr (W >= 4) {
#pragma unroll
    for (int b = 0; b < BYTES; b += W) {
      if constexpr (W == 16) {
        const u32x4 q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + b, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) w[b / 4 + i] = q[i];
      } else if constexpr (W == 8) {
        const u32x2 q = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off + b, 0, 0));
        w[b / 4] = q[0];
        w[b / 4 + 1] = q[1];
      } else {
        w[b / 4] = __builtin_amdgcn_raw_buffer_load_b32(r, off + b, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < T; ++e) w[e] = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * e, 0, 0);
  }
}

template <int T, typename Elt>
__device__ __forceinline__ void group_from_raw(const uint32_t (&w)[group_words<T, Elt>()], float (&v)[T]) {
  constexpr bool kWords = pow2_part(T * (int)sizeof(Elt)) >= 4;
#pragma unroll
  for (int e = 0; e < T; ++e) {
    if constexpr (sizeof(Elt) == 4) {
      v[e] = __builtin_bit_cast(float, w[e]);
    } else if constexpr (kWords) {
      v[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e / 2] >> ((e & 1) * 16)));
    } else {
      v[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)w[e]);
    }
  }
}
#endif

// Offsets at or beyond this value are outside every buffer: the load returns zero.
constexpr uint32_t kOob = 0x80000000u;

#if defined(__HIP_DEVICE_COMPILE__)
// Raw buffer descriptor words (gfx9 family: dword3 = 0x00020000).
struct BufDesc {
  u32x4 w;
};

// Debug builds (EQL_POISON_RING): before a DMA load fills a 1 KB LDS chunk, the
// issuing wave sets the chunk to all-ones bits (NaN in fp16 and fp32) and waits for
// that store.  A fragment read that runs ahead of its load, or a load that leaves its
// chunk unwritten (out-of-range lanes must write zeros), then shows up as NaN in the
// outputs instead of as plausible stale data.  Only the issuing wave touches the
// chunk, which the ring protocol has already freed, so the stores race with nothing.
#if defined(EQL_POISON_RING)
__device__ __forceinline__ void poison_chunk(uint32_t chunk) {
  __attribute__((address_space(3))) char* p = (__attribute__((address_space(3))) char*)(uintptr_t)chunk;
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p + 16 * lane_index()) = (u32x4){~0u, ~0u, ~0u, ~0u};
}
#define EQL_POISON_CHUNKS(N, base, stride)                                    \
  do {                                                                        \
    _Pragma("unroll") for (int i_ = 0; i_ < (N); ++i_) poison_chunk((base) + (uint32_t)i_ * (stride)); \
    wait_lgkm0();                                                             \
  } while (0)
#else
#define EQL_POISON_CHUNKS(N, base, stride) \
  do {                                      \
  } while (0)
#endif

// 16 bytes per lane from buffer offset `voff` straight into LDS at
// lds_base + 16 * lane (no VGPR destination).  Written as an asm statement so that
// the compiler does not add a wait for all LDS-bound loads before every later LDS
// read (it cannot tell the ring slots apart); completion is tracked explicitly
// with wait_vmcnt at the places that consume the data.
//   * The hazard recognizer does not look inside the statement, so it carries its
//     own wait states: 5 before the load (a VALU write of an SGPR read by a VMEM
//     instruction) and 1 between the M0 write and the load that reads it.
//   * The descriptor and LDS base are wave-uniform; readfirstlane keeps them in
//     SGPRs even where the compiler cannot prove uniformity.  M0 is reserved by
//     the compiler (never allocated to other values), so it needs no clobber.
__device__ __forceinline__ void dma16(const BufDesc& d, uint32_t voff, uint32_t lds_base) {
  EQL_POISON_CHUNKS(1, (uint32_t)__builtin_amdgcn_readfirstlane(lds_base), 1024u);
  const u32x4 w = {(uint32_t)__builtin_amdgcn_readfirstlane(d.w[0]), (uint32_t)__builtin_amdgcn_readfirstlane(d.w[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(d.w[2]), (uint32_t)__builtin_amdgcn_readfirstlane(d.w[3])};
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(w)
               : "memory");
}

// N loads of dma16 with one descriptor, lane offsets voff[i] and LDS bases
// lds[i], in one asm statement: its operands are all computed before it, so a
// single 5-wait-state gap covers the VALU-to-SGPR hazard for the whole batch
// (only the M0 writes inside it need their 1 wait state each).  M0 is written with
// s_mov only, so no scalar condition code is touched.
#define EQL_DMA_ONE(v, l) "s_mov_b32 m0, %" #l "\n\ts_nop 0\n\tbuffer_load_dwordx4 %" #v ", %[desc], 0 offen lds\n\t"
template <int N>
__device__ __forceinline__ void dma16_batch(const BufDesc& d, const uint32_t (&voff)[N], const uint32_t (&lds)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "batch size");
  const u32x4 w = {(uint32_t)__builtin_amdgcn_readfirstlane(d.w[0]), (uint32_t)__builtin_amdgcn_readfirstlane(d.w[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(d.w[2]), (uint32_t)__builtin_amdgcn_readfirstlane(d.w[3])};
  uint32_t l[N];
#pragma unroll
  for (int i = 0; i < N; ++i) l[i] = (uint32_t)__builtin_amdgcn_readfirstlane(lds[i]);
#if defined(EQL_POISON_RING)
#pragma unroll
  for (int i = 0; i < N; ++i) poison_chunk(l[i]);
  wait_lgkm0();
#endif
  if constexpr (N == 1) {
    asm volatile("s_nop 4\n\t" EQL_DMA_ONE(0, 1) : : "v"(voff[0]), "s"(l[0]), [desc] "s"(w) : "memory");
  } else if constexpr (N == 2) {
    asm volatile("s_nop 4\n\t" EQL_DMA_ONE(0, 2) EQL_DMA_ONE(1, 3)
                 : : "v"(voff[0]), "v"(voff[1]), "s"(l[0]), "s"(l[1]), [desc] "s"(w) : "memory");
  } else if constexpr (N == 4) {
    asm volatile("s_nop 4\n\t" EQL_DMA_ONE(0, 4) EQL_DMA_ONE(1, 5) EQL_DMA_ONE(2, 6) EQL_DMA_ONE(3, 7)
                 : : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
                     "s"(l[0]), "s"(l[1]), "s"(l[2]), "s"(l[3]), [desc] "s"(w) : "memory");
  } else {
    asm volatile("s_nop 4\n\t" EQL_DMA_ONE(0, 8) EQL_DMA_ONE(1, 9) EQL_DMA_ONE(2, 10) EQL_DMA_ONE(3, 11)
                 EQL_DMA_ONE(4, 12) EQL_DMA_ONE(5, 13) EQL_DMA_ONE(6, 14) EQL_DMA_ONE(7, 15)
                 : : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
                     "v"(voff[4]), "v"(voff[5]), "v"(voff[6]), "v"(voff[7]),
                     "s"(l[0]), "s"(l[1]), "s"(l[2]), "s"(l[3]), "s"(l[4]), "s"(l[5]), "s"(l[6]), "s"(l[7]),
                     [desc] "s"(w) : "memory");
  }
}
#undef EQL_DMA_ONE

// Descriptor words of `bytes` bytes at `base`, forced into scalar registers.  The
// address is below 2^48, so the stride field above it stays zero.
__device__ __forceinline__ u32x4 desc_words(uint64_t base, uint32_t bytes) {
  return (u32x4){(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)),
                 (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// N consecutive 1 KB loads (16 bytes per lane) from buffer offsets voff + 1024 i into
// LDS at ldsBase + OFF + 1024 i + 16 lane.  The instruction offset applies to both the
// buffer and the LDS address, so one M0 write serves a run of up to four loads; M0 is
// formed inside the statement (base register plus immediate), so the compiler keeps no
// per-slot copy of it live.  Wait states as dma16.
#define EQL_DMAO(v, i) "buffer_load_dwordx4 %[" #v "], %[desc], 0 offen offset:" #i " lds\n\t"
#define EQL_M0(o) "s_add_u32 m0, %[l], %[" #o "]\n\ts_nop 0\n\t"
template <int N, int OFF>
__device__ __forceinline__ void dma16_run(const u32x4& desc, uint32_t voff, uint32_t ldsBase) {
  static_assert(N >= 1 && N <= 8 && N != 5 && N != 7, "run length");
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane(ldsBase);
  EQL_POISON_CHUNKS(N, l + (uint32_t)OFF, 1024u);
  if constexpr (N == 1) {
    asm volatile("s_nop 4\n\t" EQL_M0(o) EQL_DMAO(v, 0)
                 : : [v] "v"(voff), [l] "s"(l), [o] "i"(OFF), [desc] "s"(desc) : "memory", "scc");
  } else if constexpr (N == 2) {
    asm volatile("s_nop 4\n\t" EQL_M0(o) EQL_DMAO(v, 0) EQL_DMAO(v, 1024)
                 : : [v] "v"(voff), [l] "s"(l), [o] "i"(OFF), [desc] "s"(desc) : "memory", "scc");
  } else if constexpr (N == 3) {
    asm volatile("s_nop 4\n\t" EQL_M0(o) EQL_DMAO(v, 0) EQL_DMAO(v, 1024) EQL_DMAO(v, 2048)
                 : : [v] "v"(voff), [l] "s"(l), [o] "i"(OFF), [desc] "s"(desc) : "memory", "scc");
  } else if constexpr (N == 4) {
    asm volatile("s_nop 4\n\t" EQL_M0(o) EQL_DMAO(v, 0) EQL_DMAO(v, 1024) EQL_DMAO(v, 2048) EQL_DMAO(v, 3072)
                 : : [v] "v"(voff), [l] "s"(l), [o] "i"(OFF), [desc] "s"(desc) : "memory", "scc");
  } else {
    // Past four loads the instruction offset would exceed its 12 bits: a second run
    // starts 4 KB on in both address spaces, from a second lane offset.
    const uint32_t voff2 = voff + 4096u;
    if constexpr (N == 6) {
      asm volatile("s_nop 4\n\t" EQL_M0(o) EQL_DMAO(v, 0) EQL_DMAO(v, 1024) EQL_DMAO(v, 2048) EQL_DMAO(v, 3072)
                   EQL_M0(o2) EQL_DMAO(v2, 0) EQL_DMAO(v2, 1024)
                   : : [v] "v"(voff), [v2] "v"(voff2), [l] "s"(l), [o] "i"(OFF), [o2] "i"(OFF + 4096),
                       [desc] "s"(desc) : "memory", "scc");
    } else {
      asm volatile("s_nop 4\n\t" EQL_M0(o) EQL_DMAO(v, 0) EQL_DMAO(v, 1024) EQL_DMAO(v, 2048) EQL_DMAO(v, 3072)
                   EQL_M0(o2) EQL_DMAO(v2, 0) EQL_DMAO(v2, 1024) EQL_DMAO(v2, 2048) EQL_DMAO(v2, 3072)
                   : : [v] "v"(voff), [v2] "v"(voff2), [l] "s"(l), [o] "i"(OFF), [o2] "i"(OFF + 4096),
                       [desc] "s"(desc) : "memory", "scc");
    }
  }
}

// N loads (1 to 4) of 16 bytes per lane with lane offsets voff[i] into LDS at
// ldsBase + OFF + 1024 i + 16 lane: one M0 write per load, formed inside the statement.
#define EQL_DMAX(k) EQL_M0(o##k) "buffer_load_dwordx4 %[v" #k "], %[desc], 0 offen lds\n\t"
template <int N, int OFF>
__device__ __forceinline__ void dma16_each(const u32x4& desc, const uint32_t (&voff)[N], uint32_t ldsBase) {
  static_assert(N >= 1 && N <= 4, "batch size");
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane(ldsBase);
  EQL_POISON_CHUNKS(N, l + (uint32_t)OFF, 1024u);
  if constexpr (N == 1) {
    asm volatile("s_nop 4\n\t" EQL_DMAX(0)
                 : : [v0] "v"(voff[0]), [l] "s"(l), [o0] "i"(OFF), [desc] "s"(desc) : "memory", "scc");
  } else if constexpr (N == 2) {
    asm volatile("s_nop 4\n\t" EQL_DMAX(0) EQL_DMAX(1)
                 : : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [l] "s"(l), [o0] "i"(OFF), [o1] "i"(OFF + 1024),
                     [desc] "s"(desc) : "memory", "scc");
  } else if constexpr (N == 3) {
    asm volatile("s_nop 4\n\t" EQL_DMAX(0) EQL_DMAX(1) EQL_DMAX(2)
                 : : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [l] "s"(l),
                     [o0] "i"(OFF), [o1] "i"(OFF + 1024), [o2] "i"(OFF + 2048), [desc] "s"(desc) : "memory", "scc");
  } else {
    asm volatile("s_nop 4\n\t" EQL_DMAX(0) EQL_DMAX(1) EQL_DMAX(2) EQL_DMAX(3)
                 : : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3]), [l] "s"(l),
                     [o0] "i"(OFF), [o1] "i"(OFF + 1024), [o2] "i"(OFF + 2048), [o3] "i"(OFF + 3072),
                     [desc] "s"(desc) : "memory", "scc");
  }
}
#undef EQL_DMAX
#undef EQL_M0
#undef EQL_DMAO

// Descriptor of `bytes` bytes at `base` (words built from scalar values).
__device__ __forceinline__ BufDesc desc_at(uint64_t base, uint32_t bytes) {
  BufDesc d;
  d.w = (u32x4){(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, bytes, 0x00020000u};
  return d;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
#endif

}  // namespace eql

// pivot_device.h -- device-side building blocks of the PIVOT indexer kernels
// (gfx950 / CDNA4, wave64).
//
// Score tiles use the 32x32 matrix-core instructions with the H indexer heads
// on the M axis and 32 keys on the N axis, so after the contraction over D each
// lane holds one key column and half of the heads' dot products.  The head
// reduction S = sum_h w[h] * max(0, dot_h) then runs inside the lane, with one
// swap across the two lane halves at the end, and never leaves registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pivot {

enum : int { kBF16 = 0, kFP8 = 1 };

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kTileN = 32;  // keys per matrix-core tile

// ---------------------------------------------------------------------------
// Operand formats.  A "fragment" is what one lane feeds one 32x32 instruction
// for one operand.  Lane l covers row/column (l % 32) and k-slice (l / 32).
// Mapping of a fragment to memory (shared by A = query heads and B = keys, so
// the contraction pairs equal d):  step ks, lane half hf ->
//   elements [hf*D/2 + ks*FRAG_ELEMS, +FRAG_ELEMS) of the D-vector.
// Each lane therefore reads one contiguous D/2-element half of a row.
// ---------------------------------------------------------------------------
template <int DT>
struct Fmt;

template <>
struct Fmt<kBF16> {
  static constexpr int ESZ = 2;          // bytes per element
  static constexpr int KSTEP = 16;       // contraction depth of one instruction
  static constexpr int FRAG_ELEMS = 8;   // elements per lane per instruction
  static constexpr int FRAG_BYTES = 16;
  using frag = i32x4;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Fmt<kFP8> {
  static constexpr int ESZ = 1;
  static constexpr int KSTEP = 64;
  static constexpr int FRAG_ELEMS = 32;
  static constexpr int FRAG_BYTES = 32;
  using frag = i32x8;
  // OCP E4M3 operands (format selector 0 for A and B), unit block scales
  // (E8M0 exponent 127 = 2^0).
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

template <int DT>
__device__ inline typename Fmt<DT>::frag load_frag(const uint8_t* p) {
  if constexpr (DT == kBF16) {
    return *reinterpret_cast<const i32x4*>(p);
  } else {
    i32x4 lo = *reinterpret_cast<const i32x4*>(p);
    i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

template <int DT>
__device__ inline typename Fmt<DT>::frag zero_frag() {
  return typename Fmt<DT>::frag{};
}

// s_waitcnt immediate that waits for every vector-memory operation of the
// wave (vmcnt 0) and leaves the export and LDS/scalar counters unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

// Direct-to-LDS buffer loads: lane l's 16 (or 4) bytes from voffset land at
// LDS byte address lds + 16*l (4*l); reads past the buffer's range write zeros.
// They are issued as inline assembly, outside the compiler's wait tracking, so
// the caller waits for them explicitly (lds_dma_wait) before reading the
// destination.  (The compiler's own builtin for these loads makes it wait for
// every load in flight before each later LDS atomic, which would drain the
// rings.)  The LDS address goes through M0, a register the compiler reserves:
// each statement saves M0 in a scratch SGPR and restores it afterwards, so the
// compiler's view of M0 is never invalidated.
//
// The buffer descriptor of these loads: base address, no stride, `bytes` of
// range, raw-buffer flags; every word made wave-uniform so it lives in SGPRs.
__device__ inline i32x4 dma_rsrc(const void* base, uint32_t bytes, int flags) {
  const uint64_t addr = (uint64_t)(uintptr_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)addr),
               __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32) & 0xffff),
               __builtin_amdgcn_readfirstlane((int)bytes), flags};
}
__device__ inline void lds_dma16(i32x4 rsrc, uint32_t lds, uint32_t voffset) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rsrc)
      : "memory");
}
__device__ inline void lds_dma4(i32x4 rsrc, uint32_t lds, uint32_t voffset) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rsrc)
      : "memory");
}
// Wait until at most N vector-memory operations of the wave are outstanding
// (they complete in issue order); a compiler barrier for memory accesses.
template <int N>
__device__ inline void lds_dma_wait() {
  static_assert(N >= 0 && N < 64);
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// LDS byte address of a pointer into a __shared__ array.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Byte offset, inside one D-row, of the fragment of step ks for lane half hf.
template <int DT, int D>
__device__ constexpr int frag_offset(int ks, int hf) {
  return (hf * (D / 2) + ks * Fmt<DT>::FRAG_ELEMS) * Fmt<DT>::ESZ;
}

// Row (M index inside a 32-row block) held by accumulator i of lane l in a
// 32x32 tile: blocks of 4 rows, alternating between the two lane halves.
__device__ constexpr int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// A raw buffer resource over `bytes` bytes at `base`: loads past the range
// return zeros and stores past it are dropped by the hardware range check.
constexpr uint32_t kBufferFlags = 0x00020000;  // raw 32-bit buffer, range-checked

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}

// ---------------------------------------------------------------------------
// Order-preserving 32-bit key of a float score (larger score -> larger key);
// -0 is folded onto +0 so equal scores get equal keys.
// ---------------------------------------------------------------------------
__device__ inline uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// The score a key stands for (the inverse of score_key; -0 comes back as +0).
__device__ inline float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// The value written where an output position is -1.
__device__ inline float no_score() { return __uint_as_float(0x7FC00000u); }

// ---------------------------------------------------------------------------
// Storage codecs used by the proxy step.
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t c) { return __uint_as_float((uint32_t)c << 16); }

// binary32 -> bf16 with round-to-nearest-even: add 0x7FFF plus the lowest
// kept bit, then truncate.
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Wave / block scans.
// ---------------------------------------------------------------------------
__device__ inline uint32_t wave_inclusive_sum(uint32_t v) {
  // Hillis-Steele within each row of 16 lanes (lanes shifted in from outside
  // the row read 0), then the row totals are carried forward: lane 15 of
  // rows 0 and 2 into rows 1 and 3, lane 31 (rows 0-1) into rows 2 and 3.
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Block-wide exclusive sum over NT threads; `scratch` holds NT/64 + 1 words.
// Returns the exclusive prefix; *total receives the block total.
template <int NT>
__device__ inline uint32_t block_exclusive_sum(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) scratch[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint32_t t = lane < NW ? scratch[lane] : 0u;
    uint32_t ti = wave_inclusive_sum(t);
    if (lane < NW) scratch[lane] = ti - t;
    if (lane == NW - 1) scratch[NW] = ti;
  }
  __syncthreads();
  uint32_t res = scratch[wid] + inc - v;
  *total = scratch[NW];
  __syncthreads();
  return res;
}

}  // namespace pivot

// Helpers shared by the prefill kernels (gfx950): LDS tile geometry and swizzles, the
// HBM -> LDS copy instructions, bf16 packing and the per-tile weight form.
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.hpp"

namespace fa {
namespace {

constexpr int KT = 64;                 // keys per sub-tile
constexpr int kRelposLdsMax = 3073;    // table entries staged in LDS (2R+1 <= this)
constexpr int kRelPad = 96;            // saturated copies staged on each side of that table
constexpr int kRelWin = 192;           // per-K-slot window of a larger table (>= 128 + 64 - 1)
constexpr float kRescaleThresh = 8.0f; // base-2 growth allowed before rescaling O

template <int D>
struct Lds {
  static constexpr int KROW = D * 2;          // bytes per K or V row
  static constexpr int TILE = KT * KROW;      // one K or one V sub-tile
  static constexpr int UNITS = D / 16;        // 32-byte units per V row
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kListCap = 512;   // block-list entries staged in LDS per pass over the row

// LDS swizzles.  The LDS serves 256 bytes (64 banks of 4 bytes) per cycle; a
// ds_read_b128 is served 16 lanes at a time, so the 16 keys that lanes 0-15 (or 16-31)
// read at one logical chunk must land on 16 distinct 16-byte bank groups.  Both
// patterns repeat every kSwzKeys keys.
constexpr int kSwzKeys = 16;
// K: XOR of the 16-byte chunk index.  256-byte rows (D = 128): key & 15 over the 16
// chunks of a row; 128-byte rows (D = 64, two rows per bank window): (key >> 1) & 7.
template <int D>
__device__ __forceinline__ constexpr int k_swz(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
// V: XOR of the 32-byte unit index.  The transposing reads of one instruction cover 8
// keys (4 per lane half) at two neighbouring units; for 256-byte rows the pattern
// 2 (key & 3) + ((key >> 2) & 1) puts those 16 (key, unit) pairs on distinct units.
template <int D>
__device__ __forceinline__ constexpr int v_swz(int key) {
  return D == 128 ? (((key & 3) << 1) | ((key >> 2) & 1)) : (key & 7);
}
// K: byte offset of physical 16-byte chunk of row `key` holding logical chunk `ch`
template <int D>
__device__ __forceinline__ int k_off(int key, int ch) { return key * (D * 2) + ((ch ^ k_swz<D>(key)) << 4); }
// V: byte offset of V[key][d] (d a multiple of 4)
template <int D>
__device__ __forceinline__ int v_off(int key, int d) {
  constexpr int UM = Lds<D>::UNITS - 1;
  return key * (D * 2) + ((((d >> 4) ^ v_swz<D>(key)) & UM) << 5) + ((d & 15) << 1);
}

// key offset (within the 64-key sub-tile) held by S^T register rr of M-tile mt,
// excluding the lane-half term 4*half
__device__ __forceinline__ constexpr int key_of(int mt, int rr) { return 32 * mt + 8 * (rr >> 2) + (rr & 3); }

// The lane's 32 score elements as bits of a word (bit 16 mt + rr for the key at offset
// key_of(mt, rr) from the lane's first key): the elements whose offset is at least a.
__device__ __forceinline__ uint32_t ge_bits(int a) {
  const int c = min(max(a, 0), 64);
  const int e0 = 4 * (c >> 3) + min(c & 7, 4);   // first element at or past offset c
  return (uint32_t)(~0ull << e0);
}

template <int... U, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, U...>, F&& f) {
  (f(std::integral_constant<int, U>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// LDS byte address of a __shared__ object (the M0 operand of the LDS-DMA loads)
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const lds_void*)ptr;
}

// wave-uniform value in scalar registers (the "s" operands below)
__device__ __forceinline__ uint32_t sreg(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const void* sreg(const void* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint64_t lo = sreg((uint32_t)v), hi = sreg((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(lo | (hi << 32));
}

// HBM -> LDS loads that bypass VGPRs (global_load_lds).  Lane l writes LDS bytes
// [m0 + IMM + 16 l, +16); the immediate offset applies to the global and the LDS side
// alike.  Issued from inline assembly so that every address is a scalar base plus one
// precomputed per-lane offset; the compiler does not see these loads, so the caller
// waits (vmcnt) before the barrier that publishes the tile.  One wait state separates
// the M0 write from the load that reads it.

template <int IMM>
__device__ __forceinline__ void dma16_s(uint32_t m0, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3"
               :: "s"(sreg(m0)), "v"(voff), "s"(sreg(sbase)), "i"(IMM) : "memory", "m0");
}
// the same with the non-temporal cache policy, for data read once: streaming reads of
// scattered regions run at about 5.2 TB/s without it and 6.9 TB/s with it on MI355X
template <int IMM>
__device__ __forceinline__ void dma16_s_nt(uint32_t m0, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3 nt"
               :: "s"(sreg(m0)), "v"(voff), "s"(sreg(sbase)), "i"(IMM) : "memory", "m0");
}
__device__ __forceinline__ void dma16_v(uint32_t m0, const void* gaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(sreg(m0)), "v"(gaddr) : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(uint32_t m0, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(sreg(m0)), "v"(voff), "s"(sreg(sbase)) : "memory", "m0");
}
__device__ __forceinline__ void dma4_v(uint32_t m0, const void* gaddr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(sreg(m0)), "v"(gaddr) : "memory", "m0");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// round-to-nearest-even pair conversion into one dword (v_cvt_pk_bf16_f32), low = a
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Per-tile evaluation of the weights from the stored value x of each element:
//   soft-cap kernels: P = exp2(add - 2 cap2 / (exp2(x capk) + one)), add = cap2 - m, and
//     one = 1 on tiles that hold raw scores; masked tiles hold
//     y = log2(exp2(s capk) + 1) / capk (-inf where masked) with one = 0, which gives the
//     same weight for allowed keys and exactly 0 where masked;
//   other kernels: P = exp2(fma(x, mul, add)).
struct TileMode {
  float mul;
  float add;   // includes -m
  float one;
};

}  // namespace
}  // namespace fa

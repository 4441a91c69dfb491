// Device-side helpers shared by the gfx950 kernels: bf16 conversions, MFMA
// operand vector types, wave reductions, and the pool geometry.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace pa {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern <-> float.  Widening is exact; narrowing is round to
// nearest even (NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element loads/stores for the two pool dtypes, through raw bit patterns.
template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elt<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// 2^x with the hardware instruction alone (v_exp_f32): results below 2^-126
// flush to 0 instead of going through the denormal-safe expansion exp2f
// adds around it.  Softmax weights that small are negligible next to the
// maximum weight 1.
__device__ __forceinline__ float exp2_flush(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (the same row of the four
// 16-lane groups), through gfx950's row-swap permutes: no LDS traffic, so no
// wait on the LDS / scalar-memory counter.  Each swap returns the pair
// {x_l, x_(l^16)} (resp. ^32) in some order; max and sum are symmetric.
__device__ __forceinline__ float rows4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Page layouts (offsets inside one (block, KV head) page; t = token within
// the block).  Each 16-token tile of a page is stored so that one wave load
// instruction of the decode kernel (64 lanes x 16 bytes) reads 1 KB of
// consecutive bytes, already in the MFMA operand order:
//
// bf16 K pages (block_size % 16 == 0, head_dim % 32 == 0): the 8 values
//   d = 32j + 8grp .. +7 of token t sit at element
//   (t / 16) * 16 D + ((j * 64 + grp * 16 + t % 16) * 8); other shapes are
//   row-major [block_size][head_dim].
__device__ __forceinline__ int k16_offset(int t, int d, int D, int BS) {
  if ((BS & 15) == 0 && (D & 31) == 0)
    return (t >> 4) * 16 * D + ((((d >> 5) * 64 + ((d & 31) >> 3) * 16 + (t & 15)) << 3) | (d & 7));
  return t * D + d;
}

// 8-bit K pages (head_dim % 64 == 0): lane grp of the QK contraction owns
//   d in [grp * D/4, +D/4); its 16-byte chunk w (d = grp * D/4 + 16w .. +15)
//   of token t sits at byte (t / 16) * 16 D + (w * 64 + grp * 16 + t % 16) * 16.
//   Other head_dims: row-major [block_size][head_dim].
__device__ __forceinline__ int k8_offset(int t, int d, int D) {
  if ((D & 63) == 0) {
    const int span = D >> 2;
    const int grp = d / span, c = d - grp * span;
    return (t >> 4) * 16 * D + ((((c >> 4) * 64 + grp * 16 + (t & 15)) << 4) | (c & 15));
  }
  return t * D + d;
}

// 8-bit V pages: the operand order of the P.V MFMA.  Within a 16-token tile,
//   row r = (t % 16) / 4 * 16 + d % 16 holds D/4 codes, byte c = (d / 16) * 4 +
//   t % 4 of the row; with head_dim % 64 == 0 chunk w = c / 16 of every row
//   sits at (w * 64 + r) * 16 + c % 16, otherwise rows are consecutive
//   (r * D/4 + c).
__device__ __forceinline__ int q8_v_offset(int t, int d, int D) {
  const int r = ((t & 15) >> 2) * 16 + (d & 15);
  const int c = (d >> 4) * 4 + (t & 3);
  if ((D & 63) == 0) return (t >> 4) * 16 * D + ((((c >> 4) * 64 + r) << 4) | (c & 15));
  return (t >> 4) * 16 * D + r * (D >> 2) + c;
}

// 4 int8 codes (one dword) -> 4 bf16 (exact: |code| <= 127 has 7 bits).
__device__ __forceinline__ s16x4 i8x4_to_bf16x4(uint32_t w) {
  s16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = static_cast<float>(static_cast<int8_t>(w >> (8 * i)));
    r[i] = static_cast<short>(__float_as_uint(f) >> 16);
  }
  return r;
}
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const s16x4 a = i8x4_to_bf16x4(lo), b = i8x4_to_bf16x4(hi);
  const short v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = __builtin_bit_cast(__bf16, v[i]);
  return r;
}

// 4 E4M3 codes (one dword; bit 7 sign, exponent bias 7, no infinities) ->
// 4 bf16, exact (every E4M3 value is a bf16): gfx950's scaled conversion
// with scale 1, two codes per instruction, each result a packed dword
// (byte 2i in the low half, byte 2i + 1 in the high half).  The results are
// moved as whole dwords: extracting their bf16 elements one by one has
// produced the low half twice.
__device__ __forceinline__ u32x2 f8x4_to_bf16x4_words(uint32_t w) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return u32x2{a, b};
}
__device__ __forceinline__ s16x4 f8x4_to_bf16x4(uint32_t w) {
  return __builtin_bit_cast(s16x4, f8x4_to_bf16x4_words(w));
}

// 8-bit codes of a page, by kind: Q8 = 1 int8 integers, 2 E4M3 floats.
template <int Q8>
__device__ __forceinline__ s16x4 codes4_to_bf16x4(uint32_t w) {
  if constexpr (Q8 == 2) return f8x4_to_bf16x4(w);
  else return i8x4_to_bf16x4(w);
}
template <int Q8>
__device__ __forceinline__ bf16x8 codes8_to_bf16x8(uint32_t lo, uint32_t hi) {
  if constexpr (Q8 == 2) {
    const u32x2 a = f8x4_to_bf16x4_words(lo), b = f8x4_to_bf16x4_words(hi);
    return __builtin_bit_cast(bf16x8, (u32x4{a[0], a[1], b[0], b[1]}));
  }
  const s16x4 a = codes4_to_bf16x4<Q8>(lo), b = codes4_to_bf16x4<Q8>(hi);
  const short v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = __builtin_bit_cast(__bf16, v[i]);
  return r;
}
template <int Q8>
__device__ __forceinline__ float code_value(uint8_t c) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(codes4_to_bf16x4<Q8>(c)[0])) << 16);
}

// Address spaces of the direct global-to-LDS load builtin.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory
// and `lgkm` LDS/scalar operations of this wave are outstanding (lgkm 15:
// LDS and scalar loads are not waited for).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | (((vm >> 4) & 3) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}

// Uniform value in a scalar register (the compiler cannot always prove it).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read-only int32 at a wave-uniform address through the constant address
// space, so it becomes a scalar load (counted by lgkmcnt, not vmcnt: it does
// not wait behind the wave's in-flight vector loads).
__device__ __forceinline__ int32_t scalar_load(const int32_t* base, int idx) {
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  return ((const const_i32*)base)[idx];  // C cast: generic -> constant address space
}

}  // namespace pa

// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;   // tokens per physical KV block
constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Element storage tags.  bf16 values travel as raw 16-bit patterns.
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};

// ---- bf16 <-> fp32 -------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Dot product of two bf16 pairs accumulated into fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// ---- cross-lane --------------------------------------------------------------

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane l -> 7-l within each group of 8
constexpr int kDppRowRor8 = 0x128;     // rotate right by 8 within a row of 16 (= xor 8)

template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8, 16, 32, 64); every lane
// of the group receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f32<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_f32<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_f32<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f32<kDppRowRor8>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- lanes 16 / 32 apart ---------------------------------------------------------
// v_permlane32_swap: lanes 32..63 of a <-> lanes 0..31 of b; v_permlane16_swap:
// odd 16-lane rows of a <-> even rows of b.  Summing or maxing the two results
// combines values 32 (resp. 16) lanes apart.
__device__ __forceinline__ void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// max / sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows); every lane gets the result.
__device__ __forceinline__ float rows_max(float v) {
  float a = v, b = v;
  swap32(a, b);
  v = fmaxf(a, b);
  a = v;
  b = v;
  swap16(a, b);
  return fmaxf(a, b);
}
// max / sum over lanes l and l^32 (the two 32-lane halves); every lane gets the result.
__device__ __forceinline__ float halves_max(float v) {
  float a = v, b = v;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float v) {
  float a = v, b = v;
  swap32(a, b);
  return a + b;
}
__device__ __forceinline__ float rows_sum(float v) {
  float a = v, b = v;
  swap32(a, b);
  v = a + b;
  a = v;
  b = v;
  swap16(a, b);
  return a + b;
}

// ---- wave-uniform values ----------------------------------------------------------
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uni_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uint32_t(uni(int(uint32_t(v)))), hi = uint32_t(uni(int(uint32_t(v >> 32))));
  return reinterpret_cast<T*>(lo | (hi << 32));
}

// Read-only metadata is read through the constant address space: the loads
// are then scalar (s_load) even when the kernel also stores to memory the
// compiler cannot prove disjoint from it.
typedef __attribute__((address_space(4))) const int32_t const_i32;

__device__ __forceinline__ int32_t load_const(const int32_t* p, int64_t i) { return ((const_i32*)(p))[i]; }
// Same, but the load may not be moved (sunk towards its use): for prefetches.
__device__ __forceinline__ int32_t load_const_early(const int32_t* p, int64_t i) {
  return ((volatile const_i32*)(p))[i];
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa

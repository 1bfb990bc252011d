// Device helpers shared by the gfx950 kernels of libv4attn.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <stdint.h>

namespace v4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define V4_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ float bf16_bits_to_f32(unsigned bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ unsigned f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return (unsigned)__builtin_bit_cast(unsigned short, h);
}

// Two floats -> two bf16 packed in a dword (lo in bits 0..15).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two floats -> two OCP E4M3FN codes in the low 16 bits, round to nearest
// even after clamping to +-448 (the converter itself does not saturate).
__device__ __forceinline__ unsigned pack_fp8x2(float a, float b) {
  a = fminf(fmaxf(a, -kFp8Max), kFp8Max);
  b = fminf(fmaxf(b, -kFp8Max), kFp8Max);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four E4M3FN codes (one dword) -> four bf16 (two dwords), exactly: every
// E4M3 value is representable in bf16.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(unsigned w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(unsigned, lo);
  r.y = __builtin_bit_cast(unsigned, hi);
  return r;
}

// Eight E4M3FN codes -> an MFMA bf16x8 operand.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 w) {
  u32x2 a = fp8x4_to_bf16x4(w.x);
  u32x2 b = fp8x4_to_bf16x4(w.y);
  u32x4 r = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float fp8_to_f32(unsigned code) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
  return v.x;
}

// Rotary frequencies of the R/2 = 32 pairs, in turns per position:
// base^(-2i/R) / (2 pi), formed once on the host in fp64.
struct RopeTurns {
  double t[32];
};

inline RopeTurns rope_turns(float base, int R) {
  RopeTurns r{};
  for (int i = 0; i < 32 && 2 * i < R; ++i)
    r.t[i] = std::pow((double)base, -2.0 * i / R) * 0.15915494309189533577;
  return r;
}

// Rotary angle of a pair at absolute position pos, as (cos, sin).  The angle
// is carried in turns in fp64, whose fraction is exact to ~1e-11 turns at a
// million positions; only the reduced angle in [-pi, pi] goes through the
// fp32 sincos (about 1e-7 rad), which avoids the large-argument fp64 path.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double turns_per_pos, float* c, float* s) {
  const double turns = (double)pos * turns_per_pos;
  const float r = (float)((turns - rint(turns)) * 6.283185307179586477);
  sincosf(r, s, c);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ unsigned wave_sum_u(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Order-preserving map of a float score to an unsigned key: larger float ->
// larger key.  -0 is folded into +0; NaN maps to 0, the "absent" key that is
// never selected (every other float maps above 0x007FFFFF).
__device__ __forceinline__ unsigned score_key(float f) {
  if (f != f) return 0u;
  unsigned u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(unsigned k) {
  unsigned u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

}  // namespace v4

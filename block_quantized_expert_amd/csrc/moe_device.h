// Device-side building blocks for gfx950 (CDNA4): block-format decode to
// bfloat16 with the hardware scaled converts, the 16x16x32 bf16 MFMA, and
// wavefront helpers.  Everything here is for 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Gate-first lazy skip: the largest |SiLU(g)| = |g / (1 + e^-g)| of four
// gate values, and that maximum merged over the four lane groups (lanes l,
// l^16, l^32, l^48: the 16 rows of a 16x16 MFMA tile's column l % 16).
// Every lane of the wavefront must call silu_col_max.
__device__ __forceinline__ float silu_abs_max4(f32x4 g) {
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(g[r] / (1.0f + expf(-g[r]))));
  return m;
}
__device__ __forceinline__ float silu_col_max(float m) {
  m = fmaxf(m, __shfl_xor(m, 16));
  return fmaxf(m, __shfl_xor(m, 32));
}

// UE8M0 byte u -> the fp32 number 2^(u-127) (u in 1..254).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t u) { return __uint_as_float(u << 23); }

__device__ __forceinline__ bf16x8 join(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Eight E2M1 codes packed in one little-endian word (element 2b in the low
// nibble of byte b) -> eight bf16 values, each times the power of two s.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float s) {
  return join(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
}

// Eight OCP E4M3 bytes (two little-endian words) -> eight bf16 values times s.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1, float s) {
  return join(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true));
}

// D = A * B + C on one 16x16x32 bf16 tile with fp32 accumulation.
// Operand lanes: lane l supplies A[l % 16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l % 16]; the result lane l holds D[4*(l/16) + r][l % 16]
// for r = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// D = A * B + C on one 16x16x128 tile with fp32 accumulation, A in E2M1
// (FA = 4) or E4M3 (FA = 0), B in E4M3, every 32 consecutive inputs of a row
// of A and of a column of B under one UE8M0 scale.  In natural K order:
//  - E2M1 operand, lane l: row l % 16, inputs 32*(l/16) .. +31 in its first
//    16 bytes (element 2i in the low nibble of byte i);
//  - E4M3 operand, lane l: row (or column) l % 16, bytes 0..15 = inputs
//    16*(l/16) .. +15, bytes 16..31 = inputs 64 + 16*(l/16) .. +15;
//  - scales: lane l carries the scale of inputs 32*(l/16) .. +31 of its row
//    of A (byte SA of sa) and of its column of B (byte SB of sb).
// The result lane l holds D[4*(l/16) + r][l % 16] for r = 0..3, as for
// mfma_bf16.  Checked on the hardware against the exact product; the sum
// of one tile's 128 products keeps about 14 bits relative to the largest.
template <int FA, int SA, int SB>
__device__ __forceinline__ f32x4 mfma_scaled(i32x8 a, i32x8 b, f32x4 c, uint32_t sa,
                                             uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, 0, SA, (int)sa, SB,
                                                         (int)sb);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Four floats kept to their top three bytes (sign, exponent and 15 stored
// mantissa bits, rounded to nearest; infinities and NaNs kept) and packed
// little-endian into three 32-bit words at w (4-byte aligned): the per-slot
// expert outputs between the down projection and the combine, 2^-16 of
// each value.
__device__ __forceinline__ uint32_t f24_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return ((u & 0x7F800000u) == 0x7F800000u ? u : u + 0x80u) >> 8;
}
__device__ __forceinline__ void store_f24x4(uint32_t* w, f32x4 v) {
  const uint32_t a = f24_bits(v[0]), b = f24_bits(v[1]), c = f24_bits(v[2]), d = f24_bits(v[3]);
  w[0] = a | (b << 24);
  w[1] = (b >> 8) | (c << 16);
  w[2] = (c >> 16) | (d << 8);
}
__device__ __forceinline__ f32x4 load_f24x4(const uint32_t* w) {
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
  return f32x4{__uint_as_float(w0 << 8), __uint_as_float(((w0 >> 24) | (w1 << 8)) << 8),
               __uint_as_float(((w1 >> 16) | (w2 << 16)) << 8), __uint_as_float(w2 & 0xFFFFFF00u)};
}

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi), both round to
// nearest even; hi + lo carries 16 significant bits of v.
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

}  // namespace moe

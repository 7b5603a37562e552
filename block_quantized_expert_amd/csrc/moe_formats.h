// Per-lane access to the block-quantized weight formats for the MFMA
// kernels, and wavefront-uniform helpers.
//
// In one reduction step of 128 inputs a lane (quarter g = lane/16 of the
// wavefront, row r16 = lane%16 of a 16-row block) owns the 32 consecutive
// inputs 32g .. 32g+31 of its row: one MXFP4 block (16 code bytes, one
// UE8M0 scale) or 32 fp8 bytes under the step's one scale.  Decoded, those
// are the A operands of four 16x16x32 MFMAs (sub-step j takes inputs
// 32g + 8j .. +7); the other operand is loaded with the same index map, so
// the products pair up.
#pragma once

#include "moe.h"
#include "moe_device.h"

namespace moe {
namespace {

// Values that are the same on every lane of a wavefront, moved to scalar
// registers so that branches on them are scalar branches: a batch of loads
// then sits in one basic block with no wait between its requests.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int wave_id() { return uniform(threadIdx.x >> 6); }

// Per reduction step a lane holds Q 16-byte code vectors and one scale.
template <int WT>
struct Fmt;

template <>
struct Fmt<MOE_W_MXFP4> {
  static constexpr int Q = 1;
  static constexpr int CH = 8;  // steps preloaded per chunk
  __device__ static int64_t row_bytes(int cols) { return cols / 2; }
  __device__ static int64_t scale_row_bytes(int cols) { return cols / 32; }
  __device__ static int code_off(int ks, int g) { return ks * 64 + g * 16; }
  __device__ static int scale_off(int ks, int g) { return ks * 4 + g; }
  __device__ static void decode(const u32x4 (&q)[Q], uint32_t u, bf16x8 (&a)[4]) {
    const float s = ue8m0_to_f32(u);
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = fp4x8_to_bf16(q[0][j], s);
  }
  // sub-step j only, with the scale already in fp32
  __device__ static bf16x8 decode_j(const u32x4 (&q)[Q], float s, int j) {
    return fp4x8_to_bf16(q[0][j], s);
  }
};

template <>
struct Fmt<MOE_W_FP8E4M3_B128> {
  static constexpr int Q = 2;
  static constexpr int CH = 4;
  __device__ static int64_t row_bytes(int cols) { return cols; }
  __device__ static int64_t scale_row_bytes(int cols) { return cols / 128; }
  __device__ static int code_off(int ks, int g) { return ks * 128 + g * 32; }
  __device__ static int scale_off(int ks, int) { return ks; }
  __device__ static void decode(const u32x4 (&q)[Q], uint32_t u, bf16x8 (&a)[4]) {
    const float s = ue8m0_to_f32(u);
    a[0] = fp8x8_to_bf16(q[0][0], q[0][1], s);
    a[1] = fp8x8_to_bf16(q[0][2], q[0][3], s);
    a[2] = fp8x8_to_bf16(q[1][0], q[1][1], s);
    a[3] = fp8x8_to_bf16(q[1][2], q[1][3], s);
  }
  __device__ static bf16x8 decode_j(const u32x4 (&q)[Q], float s, int j) {
    return fp8x8_to_bf16(q[j >> 1][2 * (j & 1)], q[j >> 1][2 * (j & 1) + 1], s);
  }
};

template <int WT>
__device__ __forceinline__ void load_codes(const uint8_t* crow, const uint8_t* srow, int ks,
                                           int g, u32x4 (&q)[Fmt<WT>::Q], uint32_t& u) {
  const uint8_t* c = crow + Fmt<WT>::code_off(ks, g);
#pragma unroll
  for (int i = 0; i < Fmt<WT>::Q; ++i) q[i] = load16(c + 16 * i);
  u = srow[Fmt<WT>::scale_off(ks, g)];
}

}  // namespace
}  // namespace moe

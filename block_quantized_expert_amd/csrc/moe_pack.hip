// Packed copy of a layer's expert matrices for the batched gate/up and down
// (declared in include/moe.h): the same code and scale bytes, reordered so
// that one 128-input step of a 16-row block is one contiguous KiB (two for
// fp8) in the matrix instruction's lane order, and a lane's scale bytes of
// four steps are one 32-bit word.
//
// "DeepSeek V4 target engine (CPU + optional CUDA tier)", introduction and
// GPU coverage: routed experts in MXFP4 (E2M1 codes, one UE8M0 scale per 32
// inputs); the order below is this library's.
#include <hip/hip_runtime.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_host.h"

namespace moe {
namespace {

constexpr int kPackThreads = 256;
constexpr int64_t kPackMaxBlocks = 1 << 16;

// Codes: output unit u (16 bytes) is block b = u / (S*64), step s, lane l =
// 16 g + r of that block: row 16 b + r, bytes 64 s + 16 g .. +15 of the row
// (S = cols / 128 steps, cols / 2 bytes per row).
__global__ __launch_bounds__(kPackThreads) void pack_codes_kernel(const uint8_t* __restrict__ src,
                                                                  uint8_t* __restrict__ dst,
                                                                  int64_t units, int cols) {
  const int64_t steps = cols / 128, per_block = steps * 64, row_bytes = cols / 2;
  for (int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * kPackThreads) {
    const int64_t b = u / per_block, rem = u - b * per_block;
    const int64_t s = rem >> 6;
    const int l = (int)(rem & 63), g = l >> 4, r = l & 15;
    const int64_t off = (16 * b + r) * row_bytes + 64 * s + 16 * g;
    *reinterpret_cast<u32x4*>(dst + 16 * u) = *reinterpret_cast<const u32x4*>(src + off);
  }
}

// Scales: output unit u (4 bytes) is block b, chunk c of four steps, lane
// l = 16 g + r: byte t is the scale of row 16 b + r for inputs
// 128 (4c + t) + 32 g .. +31, i.e. scale byte 4 (4c + t) + g of the row.
__global__ __launch_bounds__(kPackThreads) void pack_scales_kernel(const uint8_t* __restrict__ src,
                                                                   uint32_t* __restrict__ dst,
                                                                   int64_t units, int cols) {
  const int64_t chunks = cols / 512, per_block = chunks * 64, row_bytes = cols / 32;
  for (int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * kPackThreads) {
    const int64_t b = u / per_block, rem = u - b * per_block;
    const int64_t c = rem >> 6;
    const int l = (int)(rem & 63), g = l >> 4, r = l & 15;
    const uint8_t* row = src + (16 * b + r) * row_bytes + 16 * c + g;
    dst[u] = (uint32_t)row[0] | ((uint32_t)row[4] << 8) | ((uint32_t)row[8] << 16) |
             ((uint32_t)row[12] << 24);
  }
}

// fp8 codes: unit u (16 bytes) is block b, step s, half h, lane l = 16 g + r:
// row 16 b + r, bytes 128 s + 64 h + 16 g .. +15 (the two 16-byte groups an
// E4M3 operand lane holds), at ((b S + s) 2 + h) KiB + 16 l.
__global__ __launch_bounds__(kPackThreads) void pack_codes_fp8_kernel(
    const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t units, int cols) {
  const int64_t steps = cols / 128, per_block = steps * 128;
  for (int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * kPackThreads) {
    const int64_t b = u / per_block, rem = u - b * per_block;
    const int64_t s = rem >> 7;
    const int h = (int)((rem >> 6) & 1), l = (int)(rem & 63), g = l >> 4, r = l & 15;
    const int64_t off = (16 * b + r) * cols + 128 * s + 64 * h + 16 * g;
    *reinterpret_cast<u32x4*>(dst + 16 * u) = *reinterpret_cast<const u32x4*>(src + off);
  }
}

// fp8 scales (one byte per 128 inputs of a row): unit u (4 bytes) is block
// b, chunk c, lane l = 16 g + r: byte t is row 16 b + r's scale of step
// 4c + t (the four lanes of a row hold the same word).
__global__ __launch_bounds__(kPackThreads) void pack_scales_fp8_kernel(
    const uint8_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t units, int cols) {
  const int64_t chunks = cols / 512, per_block = chunks * 64, row_bytes = cols / 128;
  for (int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * kPackThreads) {
    const int64_t b = u / per_block, rem = u - b * per_block;
    const int64_t c = rem >> 6;
    const int r = (int)(rem & 15);
    const uint8_t* row = src + (16 * b + r) * row_bytes + 4 * c;
    dst[u] = (uint32_t)row[0] | ((uint32_t)row[1] << 8) | ((uint32_t)row[2] << 16) |
             ((uint32_t)row[3] << 24);
  }
}

unsigned pack_grid(int64_t units) {
  const int64_t blocks = (units + kPackThreads - 1) / kPackThreads;
  return (unsigned)(blocks < kPackMaxBlocks ? blocks : kPackMaxBlocks);
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_packed_experts_bytes(const moe_layer* layer) {
  if (layer == nullptr) return 0;
  moe_layer plain = *layer;
  plain.packed_experts = nullptr;
  moe::PackPlan pk;
  if (moe::check_layer(&plain) != MOE_OK || moe::plan_pack(&plain, &pk) != MOE_OK) return 0;
  return pk.total;
}

extern "C" moe_status moe_pack_experts(const moe_layer* layer, void* packed, size_t packed_bytes,
                                       hipStream_t stream) {
  if (layer == nullptr) return MOE_ERR_INVALID;
  moe_layer plain = *layer;
  plain.packed_experts = nullptr;
  moe_status s = moe::check_layer(&plain);
  if (s != MOE_OK) return s;
  moe::PackPlan pk;
  if ((s = moe::plan_pack(&plain, &pk)) != MOE_OK) return s;
  if (packed == nullptr || reinterpret_cast<uintptr_t>(packed) % 256 != 0 ||
      packed_bytes < pk.total)
    return MOE_ERR_INVALID;
  const moe_proj* src[6] = {&layer->gate,        &layer->up,        &layer->down,
                            &layer->shared_gate, &layer->shared_up, &layer->shared_down};
  uint8_t* base = static_cast<uint8_t*>(packed);
  for (int m = 0; m < 6; ++m) {
    if (pk.codes[m] < 0) continue;
    const int cols = pk.cols[m];
    // 16-byte code units (rows x cols/2 bytes MXFP4, rows x cols fp8) and
    // 4-byte scale words (64 lanes x cols/512 per 16-row block, both types)
    const bool fp4 = pk.type[m] == MOE_W_MXFP4;
    const int64_t code_units = pk.rows[m] * (fp4 ? cols / 2 : cols) / 16;
    const int64_t scale_units = pk.rows[m] / 16 * 64 * (cols / 512);
    hipLaunchKernelGGL(fp4 ? moe::pack_codes_kernel : moe::pack_codes_fp8_kernel,
                       dim3(moe::pack_grid(code_units)), dim3(moe::kPackThreads), 0, stream,
                       src[m]->codes, base + pk.codes[m], code_units, cols);
    hipLaunchKernelGGL(fp4 ? moe::pack_scales_kernel : moe::pack_scales_fp8_kernel,
                       dim3(moe::pack_grid(scale_units)), dim3(moe::kPackThreads), 0, stream,
                       src[m]->scales, reinterpret_cast<uint32_t*>(base + pk.scales[m]),
                       scale_units, cols);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

// A plain streaming read over a large buffer, and independent scaled
// matrix instructions: the measured ceilings of the HBM read rate and of the
// matrix-core issue rate on this GPU (declared in include/moe_probe.h).
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_probe.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerCu = 8;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                   int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = u32x4{0, 0, 0, 0};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == kProbeMagic) sink[0] = v;
}

// Independent accumulators per wavefront (no dependence between
// consecutive instructions), operands built from the lane index; the fold
// at the end keeps every instruction live.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int FA, int FB, bool BIG>
__global__ __launch_bounds__(kProbeThreads) void mfma_rate_kernel(float* __restrict__ out,
                                                                  int iters) {
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)(kProbeMagic * (threadIdx.x + i)) | 0x01010101;
    b[i] = (int)(kProbeMagic ^ (i * 77 + threadIdx.x));
  }
  float s = 0.0f;
  if constexpr (BIG) {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], FA, FB, 0, 127, 0,
                                                                  127);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
  } else {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], FA, FB, 0, 127, 0,
                                                                   127);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

template <bool BIG>
hipError_t mfma_rate_launch(int fa, int fb, unsigned blocks, int iters, float* out,
                            hipStream_t stream) {
  // the formats of the instruction: E4M3 (0), E2M3 (2), E2M1 (4)
  const dim3 g(blocks), t(kProbeThreads);
#define MOE_RATE_CASE(A, B)                                                               \
  if (fa == A && fb == B) {                                                               \
    hipLaunchKernelGGL((mfma_rate_kernel<A, B, BIG>), g, t, 0, stream, out, iters);        \
    return hipGetLastError();                                                             \
  }
  MOE_RATE_CASE(0, 0) MOE_RATE_CASE(0, 2) MOE_RATE_CASE(0, 4)
  MOE_RATE_CASE(2, 0) MOE_RATE_CASE(2, 2) MOE_RATE_CASE(2, 4)
  MOE_RATE_CASE(4, 0) MOE_RATE_CASE(4, 2) MOE_RATE_CASE(4, 4)
#undef MOE_RATE_CASE
  return hipErrorInvalidValue;
}

int probe_blocks() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus * kProbeBlocksPerCu;
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_mfma_rate_out_floats(void) {
  return (size_t)moe::probe_blocks() * moe::kProbeThreads;
}

extern "C" moe_status moe_mfma_rate(int shape, int fmt_a, int fmt_b, int iters, float* out,
                                    hipStream_t stream) {
  auto fmt_ok = [](int f) { return f == 0 || f == 2 || f == 4; };
  if ((shape != 16 && shape != 32) || !fmt_ok(fmt_a) || !fmt_ok(fmt_b) || iters < 1 ||
      out == nullptr)
    return MOE_ERR_INVALID;
  const int blocks = moe::probe_blocks();
  if (blocks <= 0) return MOE_ERR_DEVICE;
  const hipError_t e =
      shape == 32 ? moe::mfma_rate_launch<true>(fmt_a, fmt_b, (unsigned)blocks, iters, out, stream)
                  : moe::mfma_rate_launch<false>(fmt_a, fmt_b, (unsigned)blocks, iters, out, stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                      hipStream_t stream) {
  if (src == nullptr || sink == nullptr || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3) != 0 || bytes % 16 != 0)
    return MOE_ERR_INVALID;
  if (bytes == 0) return MOE_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_DEVICE;
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (int64_t)cus * moe::kProbeBlocksPerCu;
  const int64_t need = (n16 + moe::kProbeThreads - 1) / moe::kProbeThreads;
  if (blocks > need) blocks = need;
  hipLaunchKernelGGL(moe::stream_read_kernel, dim3((unsigned)blocks), dim3(moe::kProbeThreads), 0,
                     stream, static_cast<const moe::u32x4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// A plain streaming read over a large buffer: the measured ceiling of the
// HBM read rate on this GPU (declared in include/moe_probe.h).
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

}  // namespace
}  // namespace moe

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

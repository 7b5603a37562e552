// Routers: learned sqrt(softplus) top-k and token-id hash lookup.
//
// "DeepSeek-V4-Flash 284B -- Deep-Dive Mathematical & Kernel Guide",
// section 1 (SQRT_SOFTPLUS gating for the learned layers, ffn_gate_tid2eid
// for the hash layers) and section 3.2 (routed weights sum to 1.5).
#include <hip/hip_runtime.h>
#include <limits.h>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {
namespace {

// One wavefront per token; each lane holds PER logits (expert e = j*64 + lane).
// top_k rounds of a wave-wide arg-max on (value, lower index), then the
// weights of the winners in fp64, summed in rank order.
template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int n_tokens, int n_experts, int top_k,
                                                         float routed_scale,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tokens) return;  // whole wavefront leaves together
  const float* row = logits + (size_t)t * n_experts;
  float v[PER];
  bool live[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = j * kWave + lane;
    live[j] = e < n_experts;
    v[j] = live[j] ? row[e] : 0.0f;
  }
  int my_id = -1;
  float my_v = 0.0f;
  for (int r = 0; r < top_k; ++r) {
    // best live entry of this lane: j ascending means index ascending, so a
    // strict '>' keeps the lower index on ties
    float bv = 0.0f;
    int bi = INT_MAX;
    int have = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (live[j] && (!have || v[j] > bv)) {
        bv = v[j];
        bi = j * kWave + lane;
        have = 1;
      }
    }
    // butterfly arg-max: (larger value, then lower index) is a total order,
    // so every lane ends with the same winner
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const int oh = __shfl_xor(have, off);
      if (oh && (!have || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
        have = 1;
      }
    }
    if (lane == r) {
      my_id = bi;
      my_v = bv;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (j * kWave + lane == bi) live[j] = false;
  }
  double s = 0.0;
  if (lane < top_k) {
    const double l = (double)my_v;
    s = sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
  }
  double total = 0.0;
  for (int r = 0; r < top_k; ++r) total += __shfl(s, r);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    w[(size_t)t * top_k + lane] = (float)((double)routed_scale * s / total);
  }
}

__global__ __launch_bounds__(256) void route_hash_kernel(const int32_t* __restrict__ token_ids,
                                                         int n_tokens,
                                                         const int32_t* __restrict__ tid2eid,
                                                         const float* __restrict__ tid2w,
                                                         int vocab, int n_experts, int top_k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w,
                                                         int32_t* __restrict__ dev_error) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n_tokens * top_k) return;
  const int64_t t = i / top_k;
  const int j = (int)(i - t * top_k);
  const int tok = token_ids[t];
  int32_t id = -1;
  float wt = 0.0f;
  int err = 0;
  if (tok < 0 || tok >= vocab) {
    err = MOE_DEVERR_TOKEN_ID;
  } else {
    id = tid2eid[(int64_t)tok * top_k + j];
    wt = tid2w[(int64_t)tok * top_k + j];
    if (id < 0 || id >= n_experts) {
      id = -1;
      wt = 0.0f;
      err = MOE_DEVERR_EXPERT_ID;
    }
  }
  ids[i] = id;
  w[i] = wt;
  if (err && dev_error) atomicOr(dev_error, err);
}

}  // namespace

hipError_t launch_route(const float* logits, int n_tokens, int n_experts, int top_k,
                        float routed_scale, int32_t* ids, float* w, hipStream_t stream) {
  const dim3 grid((n_tokens + 3) / 4), block(256);
  const int per = (n_experts + kWave - 1) / kWave;
  if (per <= 1)
    route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, n_tokens, n_experts, top_k, routed_scale, ids, w);
  else if (per <= 2)
    route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, n_tokens, n_experts, top_k, routed_scale, ids, w);
  else if (per <= 4)
    route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, n_tokens, n_experts, top_k, routed_scale, ids, w);
  else if (per <= 8)
    route_topk_kernel<8><<<grid, block, 0, stream>>>(logits, n_tokens, n_experts, top_k, routed_scale, ids, w);
  else
    route_topk_kernel<16><<<grid, block, 0, stream>>>(logits, n_tokens, n_experts, top_k, routed_scale, ids, w);
  return hipGetLastError();
}

hipError_t launch_route_hash(const int32_t* token_ids, int n_tokens, const int32_t* tid2eid,
                             const float* tid2w, int vocab, int n_experts, int top_k,
                             int32_t* ids, float* w, int32_t* dev_error, hipStream_t stream) {
  const int64_t n = (int64_t)n_tokens * top_k;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  route_hash_kernel<<<grid, block, 0, stream>>>(token_ids, n_tokens, tid2eid, tid2w, vocab,
                                                n_experts, top_k, ids, w, dev_error);
  return hipGetLastError();
}

}  // namespace moe

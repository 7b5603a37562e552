// Wavefront-level learned routing shared by the router kernels and the
// fused decode kernel: top-k of one token's logits with sqrt(softplus)
// weights.
//
// "DeepSeek-V4-Flash 284B -- Deep-Dive Mathematical & Kernel Guide",
// section 1 (SQRT_SOFTPLUS gating) and section 3.2 (routed weights sum to
// the routed scale, 1.5).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "moe_device.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

__device__ __forceinline__ int read_lane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts by 1, 2, 4
// and 8 inside each row of 16 lanes, then the last lane of row 0 (of rows
// 0-1) is added into rows 1 and 3 (rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// A float as an unsigned key with the same order (larger value, larger
// key); -0 is first made +0, so the two compare equal as they do as floats.
// Every key is at least 1: 0 marks padding lanes and experts already chosen,
// which must stay below every live key (only the negative NaN with all
// mantissa bits set would map to 0; it shares 1 with its neighbour NaN).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return k > 1u ? k : 1u;
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Maximum of an unsigned value over the 64 lanes (an inclusive max-scan
// with the shifts of wave_incl_scan; lane 63 ends with the maximum).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)read_lane((int)v, 63);
}

// One token's logits as keys: lane l holds experts j*64 + l; experts past
// n_experts get key 0, below every live key.  All PER loads are issued
// before any is used (a load under the e < E branch would be waited for on
// its own).
template <int PER>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int n_experts, int lane,
                                          uint32_t (&key)[PER]) {
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = row[min(j * kWave + lane, n_experts - 1)];
#pragma unroll
  for (int j = 0; j < PER; ++j) key[j] = j * kWave + lane < n_experts ? order_key(v[j]) : 0u;
}

// Top-k selection by one wavefront (section 1 of the guide: the k largest
// gate scores; sqrt(softplus(.)) is increasing, so the logits give the same
// order), ties to the lower expert index.  Round r takes the largest key
// left (wave_max), the lowest expert index holding it (the first ballot in
// index order), and removes it; lane r receives that expert and key.  So
// lane r < k ends with the expert of rank r in (larger value, lower index)
// order.  Needs at least top_k live keys.
template <int PER>
__device__ __forceinline__ void route_select(uint32_t (&key)[PER], int top_k, int lane,
                                             int& out_id, uint32_t& out_key) {
  out_id = -1;
  out_key = 0u;
  for (int r = 0; r < top_k; ++r) {
    uint32_t m = key[0];
#pragma unroll
    for (int j = 1; j < PER; ++j) m = max(m, key[j]);
    const uint32_t top = wave_max(m);
    int e = -1;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint64_t b = __ballot(key[j] == top);
      if (e < 0 && b != 0) e = j * kWave + __builtin_ctzll(b);
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (e == j * kWave + lane) key[j] = 0u;
    if (lane == r) {
      out_id = e;
      out_key = top;
    }
  }
}

// s = sqrt(softplus(l)) in fp64 (section 1 of the guide).
__device__ __forceinline__ double gate_score(double l) {
  return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
}

// The routed weight of a winner with score s: routed_scale * s / total,
// where total is the sum of the k winners' scores taken in rank order in
// fp64; rounded to fp32 once (section 3.2 of the guide: the routed weights
// sum to the routed scale).
__device__ __forceinline__ float routed_weight(double s, double total, float routed_scale) {
  return (float)((double)routed_scale * s / total);
}

// Top-k of one token's keys (load_keys) with weights: lane r < k returns
// the expert of rank r and its weight (route_select, then routed_weight).
template <int PER>
__device__ __forceinline__ void route_keys(uint32_t (&key)[PER], int top_k, float routed_scale,
                                           int lane, int& out_id, float& out_w) {
  uint32_t out_key;
  route_select<PER>(key, top_k, lane, out_id, out_key);
  const double s = lane < top_k ? gate_score((double)key_value(out_key)) : 0.0;
  const long long sb = __double_as_longlong(s);
  auto s_of_rank = [&](int i) {
    const uint32_t lo = (uint32_t)read_lane((int)(uint32_t)sb, i);
    const uint32_t hi = (uint32_t)read_lane((int)(uint32_t)(sb >> 32), i);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  };
  double total = 0.0;
  for (int i = 0; i < top_k; ++i) total += s_of_rank(i);
  out_w = lane < top_k ? routed_weight(s, total, routed_scale) : 0.0f;
}

// route_keys of the token whose logits start at row.
template <int PER>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int n_experts,
                                            int top_k, float routed_scale, int lane,
                                            int& out_id, float& out_w) {
  uint32_t key[PER];
  load_keys<PER>(row, n_experts, lane, key);
  route_keys<PER>(key, top_k, routed_scale, lane, out_id, out_w);
}

}  // namespace
}  // namespace moe

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
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Top-k of one token's logits by one wavefront; lane l holds experts
// j*64 + l.  Selection runs on the logits themselves (sqrt(softplus(.)) is
// increasing, so the order is the same) with ties to the lower expert index.
//  1. The k-th largest key t, one bit at a time from the top: a bit stays
//     set while at least k keys are >= the candidate (counted with ballots,
//     so the whole search runs on the scalar unit).
//  2. The winners are every key above t and, in index order, as many keys
//     equal to t as are still missing; lane c collects the c-th winner in
//     index order.
//  3. A winner's slot is the number of winners before it in (larger value,
//     lower index) order.  Lane r < k returns slot r: its expert and its
//     weight routed_scale * s_r / sum_i s_i with s = sqrt(softplus(logit)),
//     in fp64 with the sum taken in slot order, rounded to fp32 once.
template <int PER>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int n_experts,
                                            int top_k, float routed_scale, int lane,
                                            int& out_id, float& out_w) {
  // all PER loads are issued before any is used (a load under the e < E
  // branch would be waited for on its own)
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = row[min(j * kWave + lane, n_experts - 1)];
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j)
    key[j] = j * kWave + lane < n_experts ? order_key(v[j]) : 0u;  // every live key is > 0
  uint32_t t = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) n += __popcll(__ballot(key[j] >= c));
    if (n >= top_k) t = c;
  }
  int above = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) above += __popcll(__ballot(key[j] > t));
  const int need = top_k - above;
  int eq_seen = 0, c = 0;
  uint32_t my_key = 0u;
  int my_idx = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint64_t eq = __ballot(key[j] == t);
    const int r = eq_seen + __popcll(eq & lanemask_lt(lane));
    eq_seen += __popcll(eq);
    uint64_t m = __ballot(key[j] > t || (key[j] == t && r < need));
    while (m) {
      const int l = __builtin_ctzll(m);
      m &= m - 1;
      const uint32_t kv = (uint32_t)read_lane((int)key[j], l);
      if (lane == c) {
        my_key = kv;
        my_idx = j * kWave + l;
      }
      ++c;
    }
  }
  int rank = 0;
  for (int q = 0; q < top_k; ++q) {
    const uint32_t kq = (uint32_t)read_lane((int)my_key, q);
    rank += (kq > my_key || (kq == my_key && q < lane)) ? 1 : 0;
  }
  uint32_t out_key = 0u;
  out_id = -1;
  for (int q = 0; q < top_k; ++q) {
    const int rq = read_lane(rank, q);
    const uint32_t kq = (uint32_t)read_lane((int)my_key, q);
    const int iq = read_lane(my_idx, q);
    if (lane == rq) {
      out_key = kq;
      out_id = iq;
    }
  }
  double s = 0.0;
  if (lane < top_k) {
    const double l = (double)key_value(out_key);
    s = sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
  }
  const long long sb = __double_as_longlong(s);
  double total = 0.0;
  for (int r = 0; r < top_k; ++r) {
    const uint32_t lo = (uint32_t)read_lane((int)(uint32_t)sb, r);
    const uint32_t hi = (uint32_t)read_lane((int)(uint32_t)(sb >> 32), r);
    total += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  }
  out_w = lane < top_k ? (float)((double)routed_scale * s / total) : 0.0f;
}

}  // namespace
}  // namespace moe

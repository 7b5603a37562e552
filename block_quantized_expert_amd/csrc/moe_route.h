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
#include "moe_kernels.h"

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

// ------------------------------------------------------------ routing options

__device__ __forceinline__ bool opts_select_on_logits(const RouteOpts& o) {
  return o.n_group <= 1 && o.bias == nullptr;
}
__device__ __forceinline__ bool opts_prune(const RouteOpts& o, int top_k) {
  return o.keep_max < top_k || o.min_w > 0.0f;
}

// A double as an unsigned 64-bit key with the same order; -0 is made +0 and
// every key is at least 1 (0 marks padding and removed entries).
__device__ __forceinline__ uint64_t order_key64(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  if (b == 0x8000000000000000ull) b = 0ull;
  const uint64_t k = (b & 0x8000000000000000ull) ? ~b : (b | 0x8000000000000000ull);
  return k > 1ull ? k : 1ull;
}

__device__ __forceinline__ double key_value64(uint64_t k) {
  return __longlong_as_double(
      (long long)((k & 0x8000000000000000ull) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}

// One DPP step of a 64-bit max-scan: both halves move with the same control
// (lanes without a source read 0, below every key), then the larger wins.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ uint64_t dpp_max64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK,
                                                            0xF, BOUND);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL,
                                                            ROW_MASK, 0xF, BOUND);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Maximum of a 64-bit value over the wavefront, in every lane: the max-scan
// of wave_max on both halves (row shifts, then row broadcasts; lane 63 ends
// with the maximum), read back from lane 63.  DPP moves stay inside the
// register file; cross-lane shuffles through LDS cost tens of cycles each.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
  v = dpp_max64<0x111, 0xF, true>(v);   // row_shr:1
  v = dpp_max64<0x112, 0xF, true>(v);   // row_shr:2
  v = dpp_max64<0x114, 0xF, true>(v);   // row_shr:4
  v = dpp_max64<0x118, 0xF, true>(v);   // row_shr:8
  v = dpp_max64<0x142, 0xA, false>(v);  // row_bcast:15
  v = dpp_max64<0x143, 0xC, false>(v);  // row_bcast:31
  const uint32_t lo = (uint32_t)read_lane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)read_lane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double read_lane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)read_lane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)read_lane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ float read_lane_f32(float v, int l) {
  return __int_as_float(read_lane(__float_as_int(v), l));
}

// route_select on 64-bit keys.
template <int PER>
__device__ __forceinline__ void route_select64(uint64_t (&key)[PER], int top_k, int lane,
                                               int& out_id) {
  out_id = -1;
  for (int r = 0; r < top_k; ++r) {
    uint64_t m = key[0];
#pragma unroll
    for (int j = 1; j < PER; ++j) m = key[j] > m ? key[j] : m;
    const uint64_t top = wave_max64(m);
    int e = -1;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint64_t b = __ballot(key[j] == top);
      if (e < 0 && b != 0) e = j * kWave + __builtin_ctzll(b);
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (e == j * kWave + lane) key[j] = 0ull;
    if (lane == r) out_id = e;
  }
}

// Group-limited top-k with a selection-only bias ("Deep-Dive Mathematical &
// Kernel Guide", section 1: SQRT_SOFTPLUS with expert group top-k selection;
// the pages give no group parameters, so the groups are contiguous runs of
// n_experts / n_group experts scored by the sum of their two largest keys).
// Every expert's score s = sqrt(softplus(l)) is taken in fp64, its key is
// s + bias; the topk_group groups of largest score are kept (ties to the
// lower group), and the top_k largest keys among their experts are chosen
// (ties to the lower expert).  Lane r < top_k returns the expert of rank r
// and its weight routed_scale * s_r / sum of the chosen s (unbiased).
// The selection itself, from the scores s (lane l holds experts j*64 + l)
// and the selection bias bv of the same experts.  kbuf: this wavefront's LDS
// room for n_experts doubles (used when there are groups): the keys go there
// and lane g scans the members of group g for its two largest, so every group
// is scored at once (one full-wavefront reduction per group cost ~0.7 us
// each at eight groups).
template <int PER>
__device__ void route_select_grouped(const double (&s)[PER], const float (&bv)[PER],
                                     int n_experts, int top_k, float routed_scale,
                                     const RouteOpts& o, int lane, double* kbuf, int& out_id,
                                     float& out_w) {
  uint64_t key[PER];
  double kv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool live = j * kWave + lane < n_experts;
    kv[j] = s[j] + (double)bv[j];
    key[j] = live ? order_key64(kv[j]) : 0ull;
  }
  if (o.n_group > 1) {
    const int gsize = n_experts / o.n_group;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (j * kWave + lane < n_experts) kbuf[j * kWave + lane] = kv[j];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wavefront's keys are in LDS
    __builtin_amdgcn_wave_barrier();
    // lane g: the two largest keys of group g (equal ones both count), their
    // sum largest first
    uint64_t gkey = 0ull;
    if (lane < o.n_group) {
      const double* kg = kbuf + lane * gsize;
      double t1 = -INFINITY, t2 = -INFINITY;
      // eight loads in flight at a time; the comparisons follow in order
      int i = 0;
      for (; i + 8 <= gsize; i += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = kg[i + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (v[u] > t1) {
            t2 = t1;
            t1 = v[u];
          } else if (v[u] > t2) {
            t2 = v[u];
          }
        }
      }
      for (; i < gsize; ++i) {
        const double v = kg[i];
        if (v > t1) {
          t2 = t1;
          t1 = v;
        } else if (v > t2) {
          t2 = v;
        }
      }
      gkey = order_key64(gsize > 1 ? t1 + t2 : t1);
    }
    uint64_t chosen = 0ull;  // bit g: group g kept
    for (int r = 0; r < o.topk_group; ++r) {
      const uint64_t top = wave_max64(gkey);
      const int g = __builtin_ctzll(__ballot(lane < o.n_group && gkey == top));
      chosen |= 1ull << g;
      if (lane == g) gkey = 0ull;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = j * kWave + lane;
      if (e < n_experts && !((chosen >> (e / gsize)) & 1ull)) key[j] = 0ull;
    }
  }
  route_select64<PER>(key, top_k, lane, out_id);
  // the unbiased score of the expert of each rank, from the lane that holds it
  double my_s = 0.0;
  for (int r = 0; r < top_k; ++r) {
    const int e = read_lane(out_id, r);
    const int jj = e / kWave;
    double sv = s[0];
#pragma unroll
    for (int j = 1; j < PER; ++j) sv = jj == j ? s[j] : sv;
    const double val = read_lane_f64(sv, e % kWave);
    if (lane == r) my_s = val;
  }
  double total = 0.0;
  for (int i = 0; i < top_k; ++i) total += read_lane_f64(my_s, i);
  out_w = lane < top_k ? routed_weight(my_s, total, routed_scale) : 0.0f;
}

// route_select_grouped of the token whose logits start at row, its scores
// computed here.
template <int PER>
__device__ void route_token_grouped(const float* __restrict__ row, int n_experts, int top_k,
                                    float routed_scale, const RouteOpts& o, int lane,
                                    double* kbuf, int& out_id, float& out_w) {
  float v[PER], bv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = row[min(j * kWave + lane, n_experts - 1)];
#pragma unroll
  for (int j = 0; j < PER; ++j)
    bv[j] = o.bias ? o.bias[min(j * kWave + lane, n_experts - 1)] : 0.0f;
  double s[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j)
    s[j] = j * kWave + lane < n_experts ? gate_score((double)v[j]) : 0.0;
  route_select_grouped<PER>(s, bv, n_experts, top_k, routed_scale, o, lane, kbuf, out_id,
                            out_w);
}

// Tail pruning with L2-quadrature rescaling ("Deep-Dive Mathematical &
// Kernel Guide", section 3.2 item 3; "[RFC / Benchmarks] Fitting 284B
// DeepSeek-V4-Flash in 57.61 GiB RAM", section 5) of one token's routed
// experts, lane r < top_k holding slot r: the slots whose weight is not
// below min_w are candidates, at most keep_max of them are kept (the largest
// weights, ties to the lower slot) and at least one (the largest weight);
// kept weights are multiplied by alpha = sqrt(sum_all w^2 / sum_kept w^2)
// (fp64 from the fp32 weights, sums in slot order), dropped slots become
// id -1 with weight 0.
__device__ void prune_slots(int top_k, int keep_max, float min_w, int lane, int& id, float& w) {
  const float wv = lane < top_k ? w : -1.0f;
  int better = 0, cbetter = 0;
  for (int i = 0; i < top_k; ++i) {
    const float wi = read_lane_f32(w, i);
    const bool beats = wi > wv || (wi == wv && i < lane);
    better += beats ? 1 : 0;
    cbetter += (beats && wi >= min_w) ? 1 : 0;
  }
  bool kept = lane < top_k && wv >= min_w && cbetter < keep_max;
  if (__ballot(kept) == 0) kept = lane < top_k && better == 0;
  const uint64_t km = __ballot(kept);
  double all_sq = 0.0, kept_sq = 0.0;
  for (int i = 0; i < top_k; ++i) {
    const double wi = (double)read_lane_f32(w, i);
    all_sq += wi * wi;
    if ((km >> i) & 1ull) kept_sq += wi * wi;
  }
  const double alpha = sqrt(all_sq / kept_sq);
  if (lane < top_k) {
    if (kept) {
      w = (float)((double)w * alpha);
    } else {
      id = -1;
      w = 0.0f;
    }
  }
}

// One token's routing with options: plain top-k on the logits, or the
// group-limited top-k with the selection-only bias; then tail pruning when
// asked.  Lane r < top_k returns slot r's expert (-1 when pruned) and weight.
template <int PER>
__device__ void route_token_opts(const float* __restrict__ row, int n_experts, int top_k,
                                 float routed_scale, const RouteOpts& o, int lane, double* kbuf,
                                 int& out_id, float& out_w) {
  if (opts_select_on_logits(o))
    route_token<PER>(row, n_experts, top_k, routed_scale, lane, out_id, out_w);
  else
    route_token_grouped<PER>(row, n_experts, top_k, routed_scale, o, lane, kbuf, out_id, out_w);
  if (opts_prune(o, top_k)) prune_slots(top_k, o.keep_max, o.min_w, lane, out_id, out_w);
}

}  // namespace
}  // namespace moe

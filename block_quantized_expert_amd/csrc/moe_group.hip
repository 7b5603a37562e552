// Token-to-expert grouping: histogram -> exclusive scan -> stable scatter.
//
// This is the bucketing behind MUL_MAT_ID "row-group reuse" and "expert
// bucket aggregation" in "DeepSeek-V4-Flash 284B -- Deep-Dive Mathematical &
// Kernel Guide" (section 2, tables A and B; section 6 item 2): tokens are
// grouped by expert so that each expert's weights stream once per batch.
//
// One 1024-thread workgroup does the whole job in LDS.  The scatter is
// deterministic: the position of flat index f inside its expert's segment is
// the number of earlier flat indices with the same expert, computed from
// per-wavefront match masks and a per-expert prefix over wavefronts, never
// from the order in which atomics land.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids,
                                                              int nk, int n_experts,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv_perm,
                                                              int32_t* __restrict__ dev_error) {
  // s_count holds the histogram, later each expert's count in the current
  // round; s_next the next free position of each expert; s_wave[w][e] the
  // count of wavefront w, then its offset inside the round (<= 1024).
  __shared__ int s_count[MOE_MAX_EXPERTS];
  __shared__ int s_next[MOE_MAX_EXPERTS];
  __shared__ uint16_t s_wave[kGroupWaves][MOE_MAX_EXPERTS];
  __shared__ int s_wave_sum[kGroupWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < n_experts; e += kGroupThreads) s_count[e] = 0;
  for (int i = tid; i < kGroupWaves * MOE_MAX_EXPERTS; i += kGroupThreads) (&s_wave[0][0])[i] = 0;
  __syncthreads();

  // 1. histogram (order-free)
  int bad = 0;
  for (int f = tid; f < nk; f += kGroupThreads) {
    const int e = ids[f];
    if (e >= 0 && e < n_experts)
      atomicAdd(&s_count[e], 1);
    else
      bad = 1;
  }
  __syncthreads();

  // 2. exclusive scan over experts (n_experts <= 1024: one per thread)
  const int c = tid < n_experts ? s_count[tid] : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) s_wave_sum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave_sum[w];
  incl += before;
  const int excl = incl - c;
  if (tid < n_experts) {
    counts[tid] = c;
    offsets[tid] = excl;
    s_next[tid] = excl;
    if (tid == n_experts - 1) offsets[n_experts] = incl;
  }
  __syncthreads();

  // 3. stable scatter, 1024 flat indices per round, in ascending order
  int nbits = 0;
  while ((1 << nbits) < n_experts) ++nbits;
  for (int base = 0; base < nk; base += kGroupThreads) {
    const int f = base + tid;
    const int e = f < nk ? ids[f] : -1;
    const bool valid = e >= 0 && e < n_experts;
    // lanes of this wavefront holding the same expert
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lanemask_lt(lane));
    const bool last = valid && (same >> lane) == 1ull;
    if (last) s_wave[wave][e] = (uint16_t)(rank + 1);
    __syncthreads();
    // per expert: wavefront counts -> offsets inside this round
    for (int x = tid; x < n_experts; x += kGroupThreads) {
      int run = 0;
#pragma unroll
      for (int w = 0; w < kGroupWaves; ++w) {
        const int cnt = s_wave[w][x];
        s_wave[w][x] = (uint16_t)run;
        run += cnt;
      }
      s_count[x] = run;
    }
    __syncthreads();
    if (valid) {
      const int p = s_next[e] + (int)s_wave[wave][e] + rank;
      perm[p] = f;
      inv_perm[f] = p;
    } else if (f < nk) {
      inv_perm[f] = -1;
    }
    __syncthreads();
    for (int x = tid; x < n_experts; x += kGroupThreads) {
      s_next[x] += s_count[x];
#pragma unroll
      for (int w = 0; w < kGroupWaves; ++w) s_wave[w][x] = 0;
    }
    __syncthreads();
  }
  if (bad && dev_error) atomicOr(dev_error, MOE_DEVERR_EXPERT_ID);
}

}  // namespace

hipError_t launch_group(const int32_t* ids, int n_tokens, int top_k, int n_experts,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        int32_t* dev_error, hipStream_t stream) {
  const int nk = n_tokens * top_k;
  group_kernel<<<1, kGroupThreads, 0, stream>>>(ids, nk, n_experts, counts, offsets, perm,
                                                inv_perm, dev_error);
  return hipGetLastError();
}

}  // namespace moe

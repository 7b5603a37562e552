// Routers (learned sqrt(softplus) top-k, token-id hash lookup) and the
// token-to-expert grouping (histogram -> exclusive scan -> stable scatter).
//
// "DeepSeek-V4-Flash 284B -- Deep-Dive Mathematical & Kernel Guide":
//   section 1: SQRT_SOFTPLUS gating for the learned layers, ffn_gate_tid2eid
//     for the hash layers; section 3.2: routed weights sum to 1.5;
//   section 2 (tables A and B) and section 6 item 2: MUL_MAT_ID groups tokens
//     by expert so each expert's weights stream once per batch.
//
// The grouping is deterministic: the position of flat index f inside its
// expert's segment is the number of earlier flat indices with the same
// expert, from per-wavefront match masks and a per-expert prefix over
// wavefronts, never from the order in which atomics land.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "moe_device.h"
#include "moe_kernels.h"
#include "moe_route.h"

namespace moe {
namespace {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;
// flat indices held in LDS by the fused route+group kernel, and its tokens
// (four per wavefront)
constexpr int kFusedMaxFlat = 4096;
constexpr int kFusedMaxTokens = 4 * kGroupWaves;
// flat indices scattered per grouping workgroup (at least), and the most
// workgroups
constexpr int kGroupChunk = 1024;
constexpr int kGroupMaxBlocks = 64;
static_assert(kGroupWaves * 8 * kWave * sizeof(double) <= kGroupWaves * MOE_MAX_EXPERTS * sizeof(int),
              "group keys of 512 experts per wavefront fit in the grouping's counts");

// ---------------------------------------------------------------- routing

template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int n_tokens, int n_experts, int top_k,
                                                         float routed_scale, RouteOpts opts,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  __shared__ double s_kb[4][PER * kWave];  // each wavefront's keys for group scoring
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tokens) return;  // the whole wavefront leaves together
  int id;
  float wt;
  route_token_opts<PER>(logits + (size_t)t * n_experts, n_experts, top_k, routed_scale, opts,
                        lane, s_kb[threadIdx.x >> 6], id, wt);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = id;
    w[(size_t)t * top_k + lane] = wt;
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

// ---------------------------------------------------------------- grouping

struct GroupShared {
  // s_base[w][e]: how many entries of wavefront w's segment go to expert e,
  // then the position of the next one
  int s_base[kGroupWaves][MOE_MAX_EXPERTS];
  // entries of each expert before and after the workgroup's range
  int s_pre[MOE_MAX_EXPERTS];
  int s_post[MOE_MAX_EXPERTS];
  int s_wave_sum[kGroupWaves];
};

// The grouping of the flat indices [blk_lo, blk_hi) of nk by one 1024-thread
// workgroup.  `ids` may point at global memory or LDS.  Several workgroups
// split the indices with no memory shared between them: each one counts
// every index outside its range per expert itself (those before it and
// those after it apart), so it knows where each expert's entries of its
// range start.  Only the `writer` stores counts, offsets and the error flag.
//
// Inside the range, wavefront w owns one contiguous segment (segments in
// ascending order, a multiple of 64 long).  It counts its segment per
// expert; one scan over (expert, wavefront) gives each wavefront the first
// position of each expert; then every wavefront scatters its segment in
// ascending order, 64 indices at a time, with no further barrier.  The rank
// of an index inside its batch of 64 is the number of earlier lanes holding
// the same expert, from ballots of the expert's bits.
__device__ void group_block(const int32_t* ids, int nk, int blk_lo, int blk_hi, bool writer,
                            int n_experts, int32_t* __restrict__ counts,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                            int32_t* __restrict__ inv_perm, int32_t* __restrict__ dev_error,
                            GroupShared& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kLoads = 8;  // batches of 64 requested before the first is used

  for (int e = tid; e < n_experts; e += kGroupThreads) {
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) sh.s_base[w][e] = 0;
    sh.s_pre[e] = 0;
    sh.s_post[e] = 0;
  }
  const int blen = blk_hi - blk_lo;
  const int64_t seg = ((int64_t)blen + kGroupThreads - 1) / kGroupThreads * kWave;
  const int lo = blk_lo + (int)min<int64_t>((int64_t)wave * seg, blen);
  const int len = blk_lo + (int)min<int64_t>((int64_t)wave * seg + seg, blen) - lo;
  const int32_t* sid = ids + lo;
  // the first kLoads batches of the wavefront's segment, loaded by the
  // histogram and used again by the scatter
  int keep[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) keep[j] = -1;
  __syncthreads();

  // 1. histograms: the indices outside the range (any thread takes any),
  // then each wavefront's own segment
  int bad = 0;
  const int n_out = nk - blen;
  for (int d = 0; d < n_out; d += kGroupThreads * kLoads) {
    int ev[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int g = d + kGroupThreads * j + tid;
      ev[j] = g < n_out ? ids[g < blk_lo ? g : g + blen] : 0;
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int g = d + kGroupThreads * j + tid;
      if (g < n_out) {
        const int e = ev[j];
        if (e >= 0 && e < n_experts)
          atomicAdd(g < blk_lo ? &sh.s_pre[e] : &sh.s_post[e], 1);
        else if (e != -1)  // -1: a slot dropped by tail pruning, no expert
          bad = 1;
      }
    }
  }
  for (int d = 0; d < len; d += kWave * kLoads) {
    int ev[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int o = d + kWave * j + lane;
      ev[j] = o < len ? sid[o] : -1;
      if (d == 0) keep[j] = ev[j];
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      if (d + kWave * j + lane < len) {
        const int e = ev[j];
        if (e >= 0 && e < n_experts)
          atomicAdd(&sh.s_base[wave][e], 1);
        else if (e != -1)
          bad = 1;
      }
    }
  }
  __syncthreads();

  // 2. per expert (one per thread, n_experts <= 1024): the prefix of its
  // range count over wavefronts, its total, then the exclusive scan of the
  // totals over experts
  int c = 0;
  int pre = 0;
  if (tid < n_experts) {
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
      const int v = sh.s_base[w][tid];
      sh.s_base[w][tid] = c;
      c += v;
    }
    pre = sh.s_pre[tid];
    c += pre + sh.s_post[tid];
  }
  int incl = wave_incl_scan(c);
  if (lane == kWave - 1) sh.s_wave_sum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += sh.s_wave_sum[w];
  incl += before;
  const int excl = incl - c;
  if (tid < n_experts) {
    if (writer) {
      counts[tid] = c;
      offsets[tid] = excl;
      if (tid == n_experts - 1) offsets[n_experts] = incl;
    }
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) sh.s_base[w][tid] += excl + pre;
  }
  __syncthreads();

  // 3. stable scatter of each segment; s_base[wave] is touched by this
  // wavefront only from here on
  int nbits = 0;
  while ((1 << nbits) < n_experts) ++nbits;
  for (int d = 0; d < len; d += kWave * kLoads) {
    int ev[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int o = d + kWave * j + lane;
      ev[j] = d == 0 ? keep[j] : (o < len ? sid[o] : -1);
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      if (d + kWave * j >= len) break;
      const int o = d + kWave * j + lane;
      const int e = ev[j];
      const bool valid = e >= 0 && e < n_experts;
      uint64_t same = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
      }
      const int r = __popcll(same & lanemask_lt(lane));
      const int run = valid ? sh.s_base[wave][e] : 0;  // read by every lane first
      const bool last = valid && (same >> lane) == 1ull;
      if (last) sh.s_base[wave][e] = run + r + 1;
      if (valid) {
        perm[run + r] = lo + o;
        inv_perm[lo + o] = run + r;
      } else if (o < len) {
        inv_perm[lo + o] = -1;
      }
    }
  }
  if (bad && writer && dev_error) atomicOr(dev_error, MOE_DEVERR_EXPERT_ID);
}

__global__ __launch_bounds__(kGroupThreads) void group_kernel(
    const int32_t* __restrict__ ids, int nk, int blk, int n_experts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ dev_error) {
  __shared__ GroupShared sh;
  const int lo = (int)min<int64_t>((int64_t)blockIdx.x * blk, nk);
  const int hi = (int)min<int64_t>((int64_t)lo + blk, nk);
  group_block(ids, nk, lo, hi, blockIdx.x == 0, n_experts, counts, offsets, perm, inv_perm,
              dev_error, sh);
}

// Learned routing and grouping of a small batch by one workgroup: the
// sixteen wavefronts route the tokens (token t by wavefront t % 16, at most
// TPW each, all their logits requested before the first selection), keep
// the ids in LDS, then group them.
template <int PER, int TPW>
__global__ __launch_bounds__(kGroupThreads) void route_group_kernel(
    const float* __restrict__ logits, int n_tokens, int n_experts, int top_k, float routed_scale,
    RouteOpts opts, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ dev_error) {
  __shared__ GroupShared sh;
  __shared__ int32_t s_ids[kFusedMaxFlat];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool on_logits = opts_select_on_logits(opts);
  const bool prune = opts_prune(opts, top_k);
  uint32_t key[TPW][PER];
  if (on_logits) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = min(wave + kGroupWaves * i, n_tokens - 1);  // past the end: a repeat, unused
      load_keys<PER>(logits + (size_t)t * n_experts, n_experts, lane, key[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave + kGroupWaves * i;
    if (t < n_tokens) {
      int id;
      float wt;
      if (on_logits)
        route_keys<PER>(key[i], top_k, routed_scale, lane, id, wt);
      else  // group keys in the grouping's LDS, which is not in use yet
        route_token_grouped<PER>(logits + (size_t)t * n_experts, n_experts, top_k, routed_scale,
                                 opts, lane,
                                 reinterpret_cast<double*>(&sh.s_base[0][0]) + wave * PER * kWave,
                                 id, wt);
      if (prune) prune_slots(top_k, opts.keep_max, opts.min_w, lane, id, wt);
      if (lane < top_k) {
        ids[t * top_k + lane] = id;
        w[t * top_k + lane] = wt;
        s_ids[t * top_k + lane] = id;
      }
    }
  }
  __syncthreads();
  const int nk = n_tokens * top_k;
  group_block(s_ids, nk, 0, nk, true, n_experts, counts, offsets, perm, inv_perm, dev_error, sh);
}

// Route and group a batch of at most 64 flat entries with one wavefront:
// lane f holds entry f, so the histogram, the scan over experts and the
// stable ranks need no workgroup barrier.
template <int PER>
__global__ __launch_bounds__(kWave) void route_group_wave_kernel(
    const float* __restrict__ logits, int n_tokens, int n_experts, int top_k, float routed_scale,
    RouteOpts opts, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm) {
  __shared__ int s_count[MOE_MAX_EXPERTS];
  __shared__ int s_ids[kWave];
  __shared__ double s_kb[PER * kWave];  // keys for group scoring
  const int lane = threadIdx.x;
  for (int e = lane; e < n_experts; e += kWave) s_count[e] = 0;
  for (int t = 0; t < n_tokens; ++t) {
    int id;
    float wt;
    route_token_opts<PER>(logits + (size_t)t * n_experts, n_experts, top_k, routed_scale, opts,
                          lane, s_kb, id, wt);
    if (lane < top_k) {
      ids[t * top_k + lane] = id;
      w[t * top_k + lane] = wt;
      s_ids[t * top_k + lane] = id;
    }
  }
  __syncthreads();
  const int nk = n_tokens * top_k;
  const int e = lane < nk ? s_ids[lane] : -1;
  if (e >= 0) atomicAdd(&s_count[e], 1);
  __syncthreads();
  // exclusive scan of the counts, PER experts per lane
  int local = 0;
  for (int j = 0; j < PER; ++j) {
    const int x = lane * PER + j;
    local += x < n_experts ? s_count[x] : 0;
  }
  const int incl = wave_incl_scan(local);
  int run = incl - local;
  for (int j = 0; j < PER; ++j) {
    const int x = lane * PER + j;
    if (x < n_experts) {
      const int c = s_count[x];
      counts[x] = c;
      offsets[x] = run;
      s_count[x] = run;  // now the first slot of the expert
      run += c;
    }
  }
  if (lane == kWave - 1) offsets[n_experts] = incl;
  __syncthreads();
  // stable rank: earlier lanes holding the same expert
  const bool valid = e >= 0;
  uint64_t same = __ballot(valid);
  for (int b = 0; (1 << b) < n_experts; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  if (valid) {
    const int p = s_count[e] + __popcll(same & lanemask_lt(lane));
    perm[p] = lane;
    inv_perm[lane] = p;
  } else if (lane < nk) {
    inv_perm[lane] = -1;  // a slot dropped by tail pruning
  }
}

int per_lane(int n_experts) { return (n_experts + kWave - 1) / kWave; }

}  // namespace

hipError_t launch_route(const float* logits, int n_tokens, int n_experts, int top_k,
                        float routed_scale, const RouteOpts& opts, int32_t* ids, float* w,
                        hipStream_t stream) {
  const dim3 grid((n_tokens + 3) / 4), block(256);
  const int per = per_lane(n_experts);
#define MOE_ROUTE(P)                                                                   \
  route_topk_kernel<P><<<grid, block, 0, stream>>>(logits, n_tokens, n_experts, top_k, \
                                                   routed_scale, opts, ids, w)
  if (per <= 1)
    MOE_ROUTE(1);
  else if (per <= 2)
    MOE_ROUTE(2);
  else if (per <= 4)
    MOE_ROUTE(4);
  else if (per <= 8)
    MOE_ROUTE(8);
  else
    MOE_ROUTE(16);
#undef MOE_ROUTE
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

hipError_t launch_group(const int32_t* ids, int n_tokens, int top_k, int n_experts,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        int32_t* dev_error, hipStream_t stream) {
  // workgroups of at least kGroupChunk indices (a multiple of 1024), at most
  // kGroupMaxBlocks of them: each one reads all nk ids once to count them
  const int nk = n_tokens * top_k;
  const int want = min(kGroupMaxBlocks, max(1, (nk + kGroupChunk - 1) / kGroupChunk));
  const int blk = max(kGroupThreads,
                      (nk + want * kGroupThreads - 1) / (want * kGroupThreads) * kGroupThreads);
  const int blocks = max(1, (nk + blk - 1) / blk);
  group_kernel<<<blocks, kGroupThreads, 0, stream>>>(ids, nk, blk, n_experts, counts, offsets,
                                                     perm, inv_perm, dev_error);
  return hipGetLastError();
}

hipError_t launch_route_group(const float* logits, int n_tokens, int n_experts, int top_k,
                              float routed_scale, const RouteOpts& opts, int32_t* ids, float* w,
                              int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, int32_t* dev_error, hipStream_t stream) {
  // one workgroup routes at most four tokens per wavefront; larger batches
  // route on a wavefront per token and group in a second kernel (one
  // workgroup routing 512 tokens took 133 us, the two kernels ~15)
  // the single-workgroup route+group keeps each wavefront's group keys in the
  // grouping's LDS, room for 512 experts per wavefront
  const bool grouped_wide = opts.n_group > 1 && n_experts > 512;
  if (n_tokens > kFusedMaxTokens || (int64_t)n_tokens * top_k > kFusedMaxFlat ||
      (grouped_wide && (int64_t)n_tokens * top_k > kWave)) {
    hipError_t e =
        launch_route(logits, n_tokens, n_experts, top_k, routed_scale, opts, ids, w, stream);
    if (e != hipSuccess) return e;
    return launch_group(ids, n_tokens, top_k, n_experts, counts, offsets, perm, inv_perm,
                        dev_error, stream);
  }
  const int per = per_lane(n_experts);
  if ((int64_t)n_tokens * top_k <= kWave) {
#define MOE_RGW(P)                                                                           \
  route_group_wave_kernel<P><<<1, kWave, 0, stream>>>(logits, n_tokens, n_experts, top_k,    \
                                                      routed_scale, opts, ids, w, counts,    \
                                                      offsets, perm, inv_perm)
    if (per <= 1)
      MOE_RGW(1);
    else if (per <= 2)
      MOE_RGW(2);
    else if (per <= 4)
      MOE_RGW(4);
    else if (per <= 8)
      MOE_RGW(8);
    else
      MOE_RGW(16);
#undef MOE_RGW
    return hipGetLastError();
  }
  const int tpw = (n_tokens + kGroupWaves - 1) / kGroupWaves;
#define MOE_RG(P, T)                                                                          \
  route_group_kernel<P, T><<<1, kGroupThreads, 0, stream>>>(                                 \
      logits, n_tokens, n_experts, top_k, routed_scale, opts, ids, w, counts, offsets, perm, \
      inv_perm, dev_error)
#define MOE_RG_T(P)   \
  if (tpw <= 1)       \
    MOE_RG(P, 1);     \
  else if (tpw <= 2)  \
    MOE_RG(P, 2);     \
  else                \
    MOE_RG(P, 4);
  if (per <= 1) {
    MOE_RG_T(1)
  } else if (per <= 2) {
    MOE_RG_T(2)
  } else if (per <= 4) {
    MOE_RG_T(4)
  } else if (per <= 8) {
    MOE_RG_T(8)
  } else {
    MOE_RG_T(16)
  }
#undef MOE_RG_T
#undef MOE_RG
  return hipGetLastError();
}

}  // namespace moe

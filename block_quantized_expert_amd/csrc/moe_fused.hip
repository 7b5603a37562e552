// Single-token decode of the whole routed MoE FFN in one kernel: learned
// routing, grouping, gate/up with SwiGLU, a grid-wide barrier, the down
// projection and the weighted combine.
//
// "DeepSeek-V4-Flash 284B -- Deep-Dive Mathematical & Kernel Guide":
//   section 1, SQRT_SOFTPLUS top-k gating; section 3.2, combine equation
//   y = e_shared(x) + sum_i w_i e_{k_i}(x) with sum_i w_i = 1.5;
//   section 4, SwiGLU equation h = SiLU(W_gate x) * (W_up x), y = W_down h.
// "DeepSeek V4 target engine (CPU + optional CUDA tier)", introduction:
//   routed experts in MXFP4.
//
// Why one kernel: at one token the layer is a stream of ~94 MB of weights
// read once, and three separate kernels each pay a start-up chain (lookups,
// first loads) and a tail with the memory idle.  Here every workgroup routes
// the token itself (1 KiB of logits), so its weight loads start at once, and
// the down weights are requested before the grid barrier so that their
// transfer overlaps the wait.
//
// One workgroup of 16 wavefronts per compute unit; the grid is exactly the
// number that fit on the GPU at once, so all of them are resident.  Phases:
//  1. routing: wavefront 0 takes the top-k of the logits (k rounds of a
//     wavefront maximum, ties to the lower expert) and copies x into LDS;
//     meanwhile four other wavefronts compute every expert's gate score in fp64,
//     needed only for the weights at the end of gate/up.  The k experts in
//     ascending order are the active segments 0..k-1, the shared expert is
//     segment k.  With one token every segment has exactly one slot, and
//     slot a belongs to segment a.  Workgroup 0 writes the routing outputs
//     (ids, weights, counts, offsets, perm, inv_perm).  Quad 1, when its
//     first item belongs to the shared expert, copies that item's codes into
//     LDS once the logits have arrived, so the memory is busy during the
//     selection.
//  2. gate/up: items (segment, 16 intermediate rows); a quad of four
//     wavefronts takes one item, each wavefront a quarter of the reduction
//     (its codes leave as one burst).  SwiGLU, then w_a * h is kept as a bf16
//     pair hi + lo (w_a = 1 for the shared expert).
//  3. the grid barrier (epoch flags, see arrive / wait_release); the down
//     codes of the workgroup's first row block are requested between its
//     arrival and its wait, so they arrive during the wait.  Every wait is
//     bounded: on timeout the workgroup reports MOE_DEVERR_SYNC, writes NaN
//     into its rows of y and skips the rest, so every wavefront always
//     exits and an incomplete y cannot pass for a result.
//  4. down: a workgroup takes 16 hidden rows over the whole intermediate
//     dimension; wavefront w takes the 128-wide steps w, w + 16, ... for
//     every segment, with its slice of w_a * h staged in its own LDS rows.
//     The 16 partial sums meet in LDS and are added in wavefront order into
//     y, so no partial result leaves the workgroup.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_formats.h"
#include "moe_kernels.h"
#include "moe_route.h"

namespace moe {
namespace {

constexpr int kFThreads = 1024;
constexpr int kFWaves = kFThreads / kWave;     // 16
constexpr int kQuads = kFWaves / 4;            // gate/up items in flight per workgroup
constexpr int kRouteWave = 0;                  // first to start; requests the logits first
constexpr int kFPer = 4;                       // experts per lane in routing (E <= 256)
constexpr int kFSlots = MOE_MAX_TOP_K + 1;      // one token: k routed slots + shared
constexpr int kMaxHidden = 4096;               // x staged whole in LDS
constexpr int kMaxInter = 4096;                // down scales of a row block staged in LDS
constexpr int kDScale = 16 * (kMaxInter / 32);  // their bytes per segment
constexpr int kHRow = 136;                      // bf16 per staged h row (128 + 8)

struct FusedSmem {
  unsigned long long epoch;  // this launch's barrier value (FusedSync::launch + 1)
  int ids[MOE_MAX_TOP_K];   // routed experts in rank order (-1: dropped by tail pruning)
  int act[kFSlots];         // expert of segment a (n_experts: shared), ascending
  int nkept;                // routed segments: top_k, or the experts kept by pruning
  float wa[kFSlots];        // routing options: the weight of segment a
  float wslot[MOE_MAX_TOP_K];  // routing options: the weight of slot (rank) r
  int ok;
  double s[kFPer * kWave];  // sqrt(softplus(logit)) of every expert
  double gkeys[kFPer * kWave];  // routing options: selection keys for group scoring
  f32x4 gu_red[kQuads][3][2][4];  // gate/up sums of wavefronts 1-3 of a quad (token lanes)
  f32x4 dn_red[kFWaves][4][2];    // down sums of every wavefront (hi and lo columns)
  alignas(16) uint8_t dsc[kFSlots][kDScale];  // down scales of the row block, per segment
  union {
    struct {
      __bf16 x[kMaxHidden];
      // a shared-expert item copied from memory during the routing: per
      // wavefront of quad 1, 2S code vectors (gate, up alternating) and
      // 2S/4 scale vectors, each 64 lanes x 16 bytes
      u32x4 pre[4][2 * 8 + 2 * 2][kWave];
    } gu;
    struct {
      __bf16 hi[kFWaves][kFSlots][kHRow];  // wavefront w: w_a * h of its step
      __bf16 lo[kFWaves][kFSlots][kHRow];
    } dn;
  } u;
};

// Synchronisation words live in the caller's workspace and carry the
// launch's epoch (the workspace's launch count plus one, see FusedSync), so
// nothing needs resetting between calls and no word is ever
// read-modify-written: device-wide atomic updates of one address serialise
// at the memory (~0.1 us each).
//
// Every word that passes between workgroups during the call (h and the
// flags) is stored and loaded at device scope, which on this GPU writes
// through and reads past the per-XCD L2 caches.  Publishing therefore needs
// no cache writeback or invalidate (a device-scope fence is one of each, over
// the whole L2 of the XCD, and hundreds of workgroups fencing at once stall
// every load behind them): every wavefront waits until its stores have
// completed (stores_done; __syncthreads alone does not wait for them), the
// workgroup meets at a barrier, and only then is its flag stored.
__device__ __forceinline__ unsigned long long poll(const unsigned long long* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void post(unsigned long long* a, unsigned long long v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void st_dev8(void* a, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(a), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev8(const void* a) {
  return __hip_atomic_load(static_cast<uint64_t*>(const_cast<void*>(a)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier over `grid` resident workgroups, in two halves so that the
// caller can request loads in between: arrive() stores this workgroup's
// arrival flag once its earlier stores have completed; wait_release() has
// wavefront 0 of every workgroup read all the flags (four per lane, requested
// together) until each holds the launch's epoch.  Reading them directly, rather
// than through one workgroup that collects them and posts a release, saves
// two memory round trips, and these are long while the down codes stream.
// wait_release() returns false on timeout (a bounded wait).
__device__ void arrive(const FusedParams& f, const FusedSmem& sm) {
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) post(f.sync->arrive + blockIdx.x, sm.epoch);
}

__device__ bool wait_release(const FusedParams& f, FusedSmem& sm) {
  if (threadIdx.x < kWave) {
    const unsigned long long ep = sm.epoch ^ f.wait_xor;
    const int lane = threadIdx.x;
    uint32_t spins = 0;
    int ok = 1;
    for (;;) {
      bool mine = true;
      for (int b0 = 0; b0 < f.grid; b0 += 4 * kWave) {
        unsigned long long v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = poll(f.sync->arrive + min(b0 + i * kWave + lane, f.grid - 1));
#pragma unroll
        for (int i = 0; i < 4; ++i) mine = mine && v[i] == ep;
      }
      if (__ballot(!mine) == 0) break;
      __builtin_amdgcn_s_sleep(2);
      if (++spins > f.spin_limit) {
        ok = 0;
        break;
      }
    }
    if (lane == 0) sm.ok = ok;
  }
  __syncthreads();
  return sm.ok != 0;
}

// S = hidden / 512: reduction steps of 128 per wavefront quarter in gate/up.
// PK (S a multiple of 4): the layer's packed copy (moe_pack_experts), where a
// wavefront's step of a 16-row block is one contiguous KiB in its lanes'
// order and a lane's scale bytes of four steps one word; the lanes hold the
// same bytes as with the row-major arrays.
template <int S, bool PK>
__global__ __launch_bounds__(kFThreads) void decode_fused_kernel(FusedParams f) {
  static_assert(!PK || S % 4 == 0, "packed scale words cover four steps");
  const FfnParams& p = f.p;
  __shared__ FusedSmem sm;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int quad = wave >> 2, wq = wave & 3;
  const int slot = (quad + 3) & 3;  // quad's place in the gate/up item order
  const int g = lane >> 4, r16 = lane & 15;
  const int k = p.top_k;
  const int G = gridDim.x;
  // routed segments (the kept experts), known once the routing is done
  int kk = k, nseg = k + p.has_shared;

  // gate/up items: the shared expert's row blocks first, then segment a's
  const int rbr = p.inter >> 4;
  const int ns = p.has_shared ? p.shared_inter >> 4 : 0;
  int gu_items = ns + k * rbr;
  const int64_t cb = p.hidden / 2, sb = p.hidden / 32;
  u32x4 qg[S], qu[S];
  uint32_t wg[S], wu[S];
  // request the codes and scales of an item (this wavefront's quarter)
  const int nks = p.hidden >> 7;
  auto issue = [&](int item) {
    const bool shared = item < ns;
    const int a = uniform(shared ? kk : (item - ns) / rbr);
    const int rb = uniform(shared ? item : item - ns - a * rbr);
    const int e = shared ? 0 : uniform(sm.act[a]);
    if constexpr (PK) {
      // row block blk, steps wq S .. wq S + S - 1: S consecutive KiB; the
      // scale words of its S / 4 chunks
      const int64_t blk = (shared ? 0 : (int64_t)e * rbr) + rb;
      const uint8_t* gc = p.pk_c[shared ? 3 : 0] + (blk * nks + wq * S) * 1024 + lane * 16;
      const uint8_t* uc = p.pk_c[shared ? 4 : 1] + (blk * nks + wq * S) * 1024 + lane * 16;
      const uint8_t* gs = p.pk_s[shared ? 3 : 0] + (blk * (nks / 4) + wq * S / 4) * 256 + lane * 4;
      const uint8_t* us = p.pk_s[shared ? 4 : 1] + (blk * (nks / 4) + wq * S / 4) * 256 + lane * 4;
      // every line of the packed copy is read whole, once: past the caches
#pragma unroll
      for (int j = 0; j < S; ++j) {
        qg[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gc + j * 1024));
        qu[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(uc + j * 1024));
      }
#pragma unroll
      for (int v = 0; v < S / 4; ++v) {
        wg[v] = *reinterpret_cast<const uint32_t*>(gs + v * 256);
        wu[v] = *reinterpret_cast<const uint32_t*>(us + v * 256);
      }
      return;
    }
    const int64_t row = (shared ? 0 : (int64_t)e * p.inter) + rb * 16 + r16;
    const uint8_t* gc = (shared ? p.sgate_c : p.gate_c) + row * cb + wq * S * 64 + g * 16;
    const uint8_t* uc = (shared ? p.sup_c : p.up_c) + row * cb + wq * S * 64 + g * 16;
    const uint8_t* gs = (shared ? p.sgate_s : p.gate_s) + row * sb + wq * S * 4;
    const uint8_t* us = (shared ? p.sup_s : p.up_s) + row * sb + wq * S * 4;
#pragma unroll
    for (int j = 0; j < S; ++j) {
      qg[j] = load16(gc + j * 64);
      qu[j] = load16(uc + j * 64);
    }
    if constexpr (S >= 4) {
#pragma unroll
      for (int v = 0; v < S / 4; ++v) {
        const u32x4 a4 = load16(gs + 16 * v), b4 = load16(us + 16 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wg[4 * v + i] = a4[i];
          wu[4 * v + i] = b4[i];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < S; ++j) {
        wg[j] = reinterpret_cast<const uint32_t*>(gs)[j];
        wu[j] = reinterpret_cast<const uint32_t*>(us)[j];
      }
    }
  };

  // copy a shared-expert item's codes and scales (this wavefront's quarter)
  // into LDS: the same bytes issue() would load, lane l's 16 at 16l
  auto issue_lds = [&](int item) {
    if constexpr (PK) {
      // the codes into LDS; the S / 4 scale words straight into registers
      // (fetch_lds waits for them with the copies)
      const uint8_t* gc = p.pk_c[3] + ((int64_t)item * nks + wq * S) * 1024 + lane * 16;
      const uint8_t* uc = p.pk_c[4] + ((int64_t)item * nks + wq * S) * 1024 + lane * 16;
#pragma unroll
      for (int j = 0; j < S; ++j) {
        __builtin_amdgcn_global_load_lds(
            gc + j * 1024, (__attribute__((address_space(3))) void*)(&sm.u.gu.pre[wq][2 * j][0]),
            16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            uc + j * 1024,
            (__attribute__((address_space(3))) void*)(&sm.u.gu.pre[wq][2 * j + 1][0]), 16, 0, 0);
      }
      const uint8_t* gs = p.pk_s[3] + ((int64_t)item * (nks / 4) + wq * S / 4) * 256 + lane * 4;
      const uint8_t* us = p.pk_s[4] + ((int64_t)item * (nks / 4) + wq * S / 4) * 256 + lane * 4;
#pragma unroll
      for (int v = 0; v < S / 4; ++v) {
        wg[v] = *reinterpret_cast<const uint32_t*>(gs + v * 256);
        wu[v] = *reinterpret_cast<const uint32_t*>(us + v * 256);
      }
      return;
    }
    const int64_t row = (int64_t)item * 16 + r16;
    const uint8_t* gc = p.sgate_c + row * cb + wq * S * 64 + g * 16;
    const uint8_t* uc = p.sup_c + row * cb + wq * S * 64 + g * 16;
    const uint8_t* gs = p.sgate_s + row * sb + wq * S * 4;
    const uint8_t* us = p.sup_s + row * sb + wq * S * 4;
    auto dma = [&](const uint8_t* src, int slot) {
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(&sm.u.gu.pre[wq][slot][0]), 16, 0, 0);
    };
#pragma unroll
    for (int j = 0; j < S; ++j) {
      dma(gc + j * 64, 2 * j);
      dma(uc + j * 64, 2 * j + 1);
    }
#pragma unroll
    for (int v = 0; v < S / 4; ++v) {
      dma(gs + 16 * v, 2 * S + 2 * v);
      dma(us + 16 * v, 2 * S + 2 * v + 1);
    }
  };
  auto fetch_lds = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the copies have landed
#pragma unroll
    for (int j = 0; j < S; ++j) {
      qg[j] = sm.u.gu.pre[wq][2 * j][lane];
      qu[j] = sm.u.gu.pre[wq][2 * j + 1][lane];
    }
    if constexpr (PK) return;  // the scale words are in registers
#pragma unroll
    for (int v = 0; v < S / 4; ++v) {
      const u32x4 a4 = sm.u.gu.pre[wq][2 * S + 2 * v][lane];
      const u32x4 b4 = sm.u.gu.pre[wq][2 * S + 2 * v + 1][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wg[4 * v + i] = a4[i];
        wu[4 * v + i] = b4[i];
      }
    }
  };
  // quad 1's first item, when it belongs to the shared expert, needs no
  // routing: its bytes are requested at once, so the memory works during
  // the routing
  const bool early = S >= 4 && quad == 1 && (int)blockIdx.x < ns;

  // the wavefronts that compute the gate scores: four that share no SIMD
  // with the routing wavefront (wavefront w runs on SIMD w % 4) and hold no
  // early item
  const int score_part = wave == 9 ? 0 : wave == 10 ? 1 : wave == 11 ? 2 : wave == 13 ? 3 : -1;

  // ---- 1. routing and grouping; x staged
  if (wave == kFWaves - 1 && lane == 0) {
    // the launch count is read before this workgroup arrives at the barrier
    // and stored back (by workgroup 0) only after every workgroup has
    // arrived, so all of them read the same value
    sm.epoch = ld_dev8(&f.sync->launch) + 1ull;
  }
  if (early) {
    // first wait for a logit of our own, so that these copies queue behind
    // the routing's loads and do not delay them
    const float first = f.logits[lane];
    asm volatile("s_waitcnt vmcnt(0)" ::"v"(first) : "memory");
    issue_lds(blockIdx.x);
  }
  if (f.route_opts) {
    // groups, a selection bias or tail pruning.  Groups and a bias select on
    // the fp64 scores: the four score wavefronts compute all of them into LDS
    // first (one expert per lane), then wavefront 0 selects.  Pruning alone
    // selects on the logits, as the plain path.  Wavefront 14 copies x.
    const bool on_scores = !opts_select_on_logits(f.ropts);  // uniform
    if (wave == 14) {
      for (int i = 0; i < p.hidden / 512; ++i)
        __builtin_amdgcn_global_load_lds(
            static_cast<const __bf16*>(p.x) + i * 512 + lane * 8,
            (__attribute__((address_space(3))) void*)(&sm.u.gu.x[i * 512]), 16, 0, 0);
    }
    // wavefront 0's selection bias, requested before the scores' barrier
    float bv[kFPer];
#pragma unroll
    for (int j = 0; j < kFPer; ++j) bv[j] = 0.0f;
    if (wave == kRouteWave && f.ropts.bias) {
#pragma unroll
      for (int j = 0; j < kFPer; ++j) bv[j] = f.ropts.bias[min(j * kWave + lane, p.n_experts - 1)];
    }
    if (on_scores) {
      if (score_part >= 0) {
        const int e = score_part * kWave + lane;
        if (e < p.n_experts) sm.s[e] = gate_score((double)f.logits[e]);
      }
      __syncthreads();
    }
    if (wave == kRouteWave) {
      int id;
      float wt;
      if (on_scores) {
        double sv[kFPer];
#pragma unroll
        for (int j = 0; j < kFPer; ++j) {
          const int e = min(j * kWave + lane, p.n_experts - 1);
          sv[j] = j * kWave + lane < p.n_experts ? sm.s[e] : 0.0;
        }
        route_select_grouped<kFPer>(sv, bv, p.n_experts, k, f.routed_scale, f.ropts, lane,
                                    sm.gkeys, id, wt);
      } else {
        route_token<kFPer>(f.logits, p.n_experts, k, f.routed_scale, lane, id, wt);
      }
      if (opts_prune(f.ropts, k)) prune_slots(k, f.ropts.keep_max, f.ropts.min_w, lane, id, wt);
      const bool kept = lane < k && id >= 0;
      const int nk = __popcll(__ballot(kept));
      int below = 0;  // kept experts below this one: its segment
      for (int j = 0; j < k; ++j) {
        const int o = read_lane(id, j);
        below += (o >= 0 && o < id) ? 1 : 0;
      }
      if (lane < k) {
        sm.ids[lane] = id;
        sm.wslot[lane] = wt;
      }
      if (kept) {
        sm.act[below] = id;
        sm.wa[below] = wt;
      }
      if (lane == 0) {
        sm.nkept = nk;
        if (p.has_shared) sm.act[nk] = p.n_experts;
      }
      if (blockIdx.x == 0 && lane < k) {
        f.topk_ids[lane] = id;
        f.inv_perm[lane] = kept ? below : -1;
        if (kept) f.perm[below] = lane;
      }
    } else if (wave == 14) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the copies of x have landed
    }
  } else if (wave == kRouteWave) {
    uint32_t key[kFPer];
    load_keys<kFPer>(f.logits, p.n_experts, lane, key);
    // x goes straight from memory into LDS (lane l of copy i writes bytes
    // 16l .. 16l+15 of 1 KiB piece i); requested after the logits, so that
    // the selection does not wait for it (loads complete in order)
    for (int i = 0; i < p.hidden / 512; ++i)
      __builtin_amdgcn_global_load_lds(
          static_cast<const __bf16*>(p.x) + i * 512 + lane * 8,
          (__attribute__((address_space(3))) void*)(&sm.u.gu.x[i * 512]), 16, 0, 0);
    int id;
    uint32_t id_key;
    route_select<kFPer>(key, k, lane, id, id_key);
    (void)id_key;
    // slot of rank i = number of chosen experts below id (ids are distinct)
    int below = 0;
    for (int j = 0; j < k; ++j) below += read_lane(id, j) < id ? 1 : 0;
    if (lane < k) {
      sm.ids[lane] = id;
      sm.act[below] = id;
    }
    if (lane == 0) {
      sm.nkept = k;
      if (p.has_shared) sm.act[k] = p.n_experts;
    }
    if (blockIdx.x == 0 && lane < k) {
      f.topk_ids[lane] = id;
      f.perm[below] = lane;
      f.inv_perm[lane] = below;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the copies of x have landed
  } else if (score_part >= 0) {
    // the gate scores, in fp64, by four otherwise idle wavefronts while the
    // selection runs (only the weights need them, at the end of gate/up)
    const int e = score_part * kWave + lane;
    if (e < p.n_experts) sm.s[e] = gate_score((double)f.logits[e]);
  }
  __syncthreads();
  kk = sm.nkept;
  nseg = kk + p.has_shared;
  gu_items = ns + kk * rbr;
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < p.n_experts; e += kFThreads) {
      int c = 0, off = 0;
      for (int j = 0; j < k; ++j) {
        c += sm.ids[j] == e ? 1 : 0;
        off += (sm.ids[j] >= 0 && sm.ids[j] < e) ? 1 : 0;
      }
      f.counts[e] = c;
      f.offsets[e] = off;
    }
    if (threadIdx.x == 0) f.offsets[p.n_experts] = kk;
  }

  const int ksteps = p.inter >> 7;  // 128-wide steps of the intermediate dimension
  const int n_rb = p.hidden >> 4;
  const int64_t dcb = p.inter / 2, dsb = p.inter / 32;
  // The down scales of this workgroup's first row block: for each segment
  // the 16 rows' scales are one contiguous block (16 * inter / 32 bytes),
  // copied into LDS by wavefront 0 with one instruction per KiB.  Read from
  // there, they cost no request per wavefront and step: one-byte loads per
  // lane doubled the requests of the down-code stream.  The copy lands long
  // before it is read (arrive() waits for wavefront 0's loads).
  if (wave == 0 && (int)blockIdx.x < n_rb) {
    const int64_t bytes = 16 * dsb;
    for (int a = 0; a < nseg; ++a) {
      const int e = uniform(sm.act[a]);
      const bool shared = e == p.n_experts;
      // packed: the row block's scale words, the same number of bytes
      const int64_t blk = (shared ? 0 : (int64_t)e * n_rb) + blockIdx.x;
      const uint8_t* src = PK ? p.pk_s[shared ? 5 : 2] + blk * (ksteps / 4) * 256
                              : (shared ? p.sdown_s : p.down_s) + blk * 16 * dsb;
      for (int i = 0; i * 1024 < bytes; ++i)
        if (i * 1024 + lane * 16 < bytes)
          __builtin_amdgcn_global_load_lds(
              src + i * 1024 + lane * 16,
              (__attribute__((address_space(3))) void*)(&sm.dsc[a][i * 1024]), 16, 0, 0);
    }
  }

  // ---- 2. gate/up: quad q takes items (4 it + slot) G + blockIdx.x, with
  // slot = (q + 3) % 4: quad 1 takes the first items (the shared expert's)
  const int n_it = (gu_items + kQuads * G - 1) / (kQuads * G);  // same for every quad
  for (int it = 0; it < n_it; ++it) {
    const int item = (it * kQuads + slot) * G + blockIdx.x;
    const bool live = item < gu_items;  // uniform per quad
    f32x4 ag = f32x4{0, 0, 0, 0}, au = f32x4{0, 0, 0, 0};
    if (live) {
      if (it == 0 && early)
        fetch_lds();
      else
        issue(item);
#pragma unroll
      for (int j = 0; j < S; ++j) {
        // token column 0 only; the other columns multiply zeros
        bf16x8 b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          b[t] = as_bf16x8(r16 == 0 ? *reinterpret_cast<const u32x4*>(
                                          &sm.u.gu.x[(wq * S + j) * 128 + g * 32 + 8 * t])
                                    : u32x4{0, 0, 0, 0});
        // the step's scale byte of the lane's 32-input block: byte g of the
        // row's word for the step, or byte j % 4 of the packed word
        const float sgv = ue8m0_to_f32(PK ? (wg[j >> 2] >> (8 * (j & 3))) & 0xFF
                                          : (wg[j] >> (8 * g)) & 0xFF);
        const float suv = ue8m0_to_f32(PK ? (wu[j >> 2] >> (8 * (j & 3))) & 0xFF
                                          : (wu[j] >> (8 * g)) & 0xFF);
#pragma unroll
        for (int t = 0; t < 4; ++t) ag = mfma_bf16(fp4x8_to_bf16(qg[j][t], sgv), b[t], ag);
#pragma unroll
        for (int t = 0; t < 4; ++t) au = mfma_bf16(fp4x8_to_bf16(qu[j][t], suv), b[t], au);
      }
      if (wq > 0 && r16 == 0) {
        sm.gu_red[quad][wq - 1][0][g] = ag;
        sm.gu_red[quad][wq - 1][1][g] = au;
      }
    }
    __syncthreads();
    if (live && wq == 0 && r16 == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        ag += sm.gu_red[quad][w][0][g];
        au += sm.gu_red[quad][w][1][g];
      }
      const bool shared = item < ns;
      const int a = shared ? kk : (item - ns) / rbr;
      const int rb = shared ? item : item - ns - a * rbr;
      float wa = 1.0f;
      if (a != kk) {
        if (f.route_opts) {
          wa = sm.wa[a];
        } else {
          double total = 0.0;
          for (int i = 0; i < k; ++i) total += sm.s[sm.ids[i]];
          wa = routed_weight(sm.s[sm.act[a]], total, f.routed_scale);
        }
      }
      bf16x4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = ag[r];
        const float h = wa * (gv / (1.0f + expf(-gv)) * au[r]);
        __bf16 x0, x1;
        split_bf16(h, x0, x1);
        hi[r] = x0;
        lo[r] = x1;
      }
      const int64_t o = (int64_t)a * p.h_stride + rb * 16 + 4 * g;
      st_dev8(p.h_hi + o, __builtin_bit_cast(uint64_t, hi));
      st_dev8(p.h_lo + o, __builtin_bit_cast(uint64_t, lo));
    }
    if (n_it > 1) __syncthreads();  // gu_red is reused
  }

  if (blockIdx.x == 0 && wave == 0 && lane < k) {
    if (f.route_opts) {
      f.topk_w[lane] = sm.wslot[lane];
    } else {
      double total = 0.0;
      for (int i = 0; i < k; ++i) total += sm.s[sm.ids[i]];
      f.topk_w[lane] = routed_weight(sm.s[sm.ids[lane]], total, f.routed_scale);
    }
  }

  // ---- 3. grid barrier; the first row block's down codes requested meanwhile
  u32x4 dq[kFSlots];
  uint32_t ds[kFSlots];
  // (the grid covers every row block, so rb is blockIdx.x: see
  // fused_decode_steps)
  auto load_down = [&](int rb, int ks) {
#pragma unroll
    for (int a = 0; a < kFSlots; ++a) {
      const int aa = a < nseg ? a : 0;
      const int e = uniform(sm.act[aa]);
      const bool shared = e == p.n_experts;
      const int64_t row = (shared ? 0 : (int64_t)e * p.hidden) + rb * 16 + r16;
      const int64_t blk = (shared ? 0 : (int64_t)e * n_rb) + rb;
      const uint8_t* c = PK ? p.pk_c[shared ? 5 : 2] + (blk * ksteps + ks) * 1024 + lane * 16
                            : (shared ? p.sdown_c : p.down_c) + row * dcb + ks * 64 + g * 16;
      if (a < nseg) {
        if constexpr (PK)  // whole lines, read once
          dq[a] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c));
        else
          dq[a] = load16(c);
        // copied into LDS above
        ds[a] = PK ? sm.dsc[a][(ks >> 2) * 256 + lane * 4 + (ks & 3)]
                   : sm.dsc[a][r16 * dsb + ks * 4 + g];
      }
    }
  };
  // wavefront 0 polls the flags: it requests nothing before, so that no poll
  // waits behind a load (a wavefront's loads complete in order)
  const bool pre = (int)blockIdx.x < n_rb && wave > 0 && wave < ksteps;
  arrive(f, sm);
  if (pre) load_down(blockIdx.x, wave);
  const bool released = wait_release(f, sm);
  // the next launch on this workspace takes the next epoch (also after a
  // give-up: its flags must not match what this launch posted)
  if (blockIdx.x == 0 && threadIdx.x == 0) st_dev8(&f.sync->launch, sm.epoch);
  if (!released) {
    // some workgroup never arrived (the grid was not all resident): this
    // workgroup's rows of y are not computed; NaN there makes the failure
    // visible in y itself, whether or not the caller passed dev_error
    if (threadIdx.x == 0 && f.dev_error) atomicOr(f.dev_error, MOE_DEVERR_SYNC);
    for (int rb = blockIdx.x; rb < n_rb; rb += G)
      if (threadIdx.x < 16) p.y[rb * 16 + threadIdx.x] = __builtin_nanf("");
    return;
  }

  // ---- 4. down: row block rb = blockIdx.x, wavefront w takes steps w, w + 16, ...
  for (int rb = blockIdx.x; rb < n_rb; rb += G) {
    // B column 0 carries the hi halves of w_a * h, column 1 the lo halves,
    // so one MFMA takes both; two accumulators (by sub-step parity) keep
    // consecutive MFMAs independent
    f32x4 acc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
    for (int ks = wave; ks < ksteps; ks += kFWaves) {
      if (!(pre && rb == (int)blockIdx.x && ks == wave)) load_down(rb, ks);
      // stage this step of w_a * h for every segment: chunk c = 16a + c16
      // holds the 8 values c16*8 .. +7 of the step
      uint64_t hv[3][4];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int c = lane + i * kWave;
        if (c < nseg * 16) {
          const int64_t o = (int64_t)(c >> 4) * p.h_stride + ks * 128 + (c & 15) * 8;
          hv[i][0] = ld_dev8(p.h_hi + o);
          hv[i][1] = ld_dev8(p.h_hi + o + 4);
          hv[i][2] = ld_dev8(p.h_lo + o);
          hv[i][3] = ld_dev8(p.h_lo + o + 4);
        }
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int c = lane + i * kWave;
        if (c < nseg * 16) {
          __bf16* dh = &sm.u.dn.hi[wave][c >> 4][(c & 15) * 8];
          __bf16* dl = &sm.u.dn.lo[wave][c >> 4][(c & 15) * 8];
          *reinterpret_cast<u32x4*>(dh) = u32x4{(uint32_t)hv[i][0], (uint32_t)(hv[i][0] >> 32),
                                                (uint32_t)hv[i][1], (uint32_t)(hv[i][1] >> 32)};
          *reinterpret_cast<u32x4*>(dl) = u32x4{(uint32_t)hv[i][2], (uint32_t)(hv[i][2] >> 32),
                                                (uint32_t)hv[i][3], (uint32_t)(hv[i][3] >> 32)};
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's rows are written
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int a = 0; a < kFSlots; ++a) {
        if (a < nseg) {  // uniform
          const float sc = ue8m0_to_f32(ds[a]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 wv = fp4x8_to_bf16(dq[a][j], sc);
            const __bf16* src = r16 == 0 ? &sm.u.dn.hi[wave][a][g * 32 + 8 * j]
                                         : &sm.u.dn.lo[wave][a][g * 32 + 8 * j];
            const bf16x8 b = as_bf16x8(r16 < 2 ? *reinterpret_cast<const u32x4*>(src)
                                               : u32x4{0, 0, 0, 0});
            acc[j & 1] = mfma_bf16(wv, b, acc[j & 1]);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // the staged rows are read before the next step
    }
    if (r16 < 2) sm.dn_red[wave][g][r16] = acc[0] + acc[1];
    __syncthreads();
    if (threadIdx.x < 16) {
      const int gg = threadIdx.x >> 2, r = threadIdx.x & 3;
      float sum = 0.0f;
      for (int w = 0; w < kFWaves; ++w) sum += sm.dn_red[w][gg][0][r] + sm.dn_red[w][gg][1][r];
      p.y[rb * 16 + threadIdx.x] = sum;
    }
    __syncthreads();
  }
}

template <typename... Params, typename... Args>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds,
                  hipStream_t stream, hipEvent_t start, hipEvent_t stop, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
  void* argv[] = {const_cast<void*>(static_cast<const void*>(&args))...};
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                                          argv, lds, stream, start, stop, 0);
  return e != hipSuccess ? e : hipGetLastError();
}

// Workgroups of the kernel that fit on the device at once; every one of them
// must be resident for the grid barrier.
template <int S, bool PK>
hipError_t resident_grid(int* grid) {
  static int cached = 0;
  static hipError_t status = hipSuccess;
  if (cached == 0 && status == hipSuccess) {
    int dev = 0, cus = 0, per_cu = 0;
    status = hipGetDevice(&dev);
    if (status == hipSuccess)
      status = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (status == hipSuccess)
      status = hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(decode_fused_kernel<S, PK>), kFThreads, 0);
    if (status == hipSuccess) cached = per_cu * cus;
  }
  *grid = cached;
  return status;
}

template <int S, bool PK>
hipError_t fused_launch(FusedParams f, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  int grid = 0;
  const hipError_t e = resident_grid<S, PK>(&grid);
  if (e != hipSuccess) return e;
  if (grid < 1) return hipErrorInvalidConfiguration;
  if (grid > FusedSync::kMaxGrid) grid = FusedSync::kMaxGrid;  // still all resident
  f.grid = grid;
  return launch(decode_fused_kernel<S, PK>, dim3(grid), dim3(kFThreads), 0, stream, start, stop,
                f);
}

}  // namespace

int fused_decode_steps(const FfnParams& p) {
  if (p.n_tokens != 1 || p.x_f32 || p.w_type != MOE_W_MXFP4) return 0;
  if (p.n_experts > kFPer * kWave || p.top_k > MOE_MAX_TOP_K) return 0;
  if (p.has_shared && (p.sw_type != MOE_W_MXFP4 || p.shared_inter != p.inter)) return 0;
  if (p.inter % 128 != 0 || p.inter > kMaxInter) return 0;
  if (p.hidden % 512 != 0 || p.hidden > kMaxHidden) return 0;
  const int s = p.hidden / 512;
  int grid = 0;
  hipError_t e = hipErrorInvalidValue;
  // the packed copy when the layer has one (it exists only for shapes that
  // are multiples of 512, so S is 4 or 8 here)
  const bool pk = p.packed && s % 4 == 0;
  switch (s) {
    case 1: e = resident_grid<1, false>(&grid); break;
    case 2: e = resident_grid<2, false>(&grid); break;
    case 4: e = pk ? resident_grid<4, true>(&grid) : resident_grid<4, false>(&grid); break;
    case 8: e = pk ? resident_grid<8, true>(&grid) : resident_grid<8, false>(&grid); break;
    default: return 0;
  }
  // every workgroup takes at most one row block of the down projection (a
  // failed query means no device: then nothing launches anyway)
  if (e == hipSuccess && min(grid, FusedSync::kMaxGrid) < p.hidden / 16) return 0;
  return s;
}

hipError_t launch_decode_fused(const FusedParams& f, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop) {
  const bool pk = f.p.packed;
  switch (fused_decode_steps(f.p)) {
    case 1: return fused_launch<1, false>(f, stream, start, stop);
    case 2: return fused_launch<2, false>(f, stream, start, stop);
    case 4: return pk ? fused_launch<4, true>(f, stream, start, stop)
                      : fused_launch<4, false>(f, stream, start, stop);
    case 8: return pk ? fused_launch<8, true>(f, stream, start, stop)
                      : fused_launch<8, false>(f, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe

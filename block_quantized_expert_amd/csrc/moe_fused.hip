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
// Phases of every workgroup (the grid is exactly the number of workgroups
// that fit on the GPU at once, so all of them are resident):
//  1. routing: wavefront 0 takes the top-k of the logits (radix select,
//     ties to the lower expert); the k experts in ascending order are the
//     active segments 0..k-1, the shared expert is segment k.  With one token
//     every segment has exactly one slot, and slot a belongs to segment a.
//     Workgroup 0 writes the routing outputs (ids, weights, counts, offsets,
//     perm, inv_perm).
//  2. gate/up: items (segment, 16 intermediate rows), grid-strided; the four
//     wavefronts each take a quarter of the reduction (its codes leave as one
//     burst), x is staged in LDS once per workgroup; SwiGLU; h as bf16 hi/lo.
//  3. the grid barrier (epoch flags, see arrive / wait_release); the down
//     codes of the workgroup's first down item are requested between its
//     arrival and its wait, so they arrive during the wait.  Every wait is
//     bounded: on timeout the kernel reports MOE_DEVERR_SYNC and skips the
//     rest, so every wavefront always exits.
//  4. down: items (16 hidden rows, one 512-wide part q of the intermediate
//     dimension), grid-strided; wavefront w takes step 4q + w for every
//     segment, with w_a * h staged in its own LDS rows; the four partial sums
//     meet in LDS and go to partial[q], and the part posts its flag; part 0
//     waits for the others and adds partial[0..nq-1] in that order into y.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_formats.h"
#include "moe_kernels.h"
#include "moe_route.h"

namespace moe {
namespace {

constexpr int kFThreads = 256;
constexpr int kFWaves = kFThreads / kWave;
constexpr int kFPer = 4;                       // experts per lane in routing (E <= 256)
constexpr int kFSlots = MOE_MAX_TOP_K + 1;      // one token: k routed slots + shared
constexpr int kHRow = 136;                      // bf16 per staged h row (128 + 8)
constexpr uint32_t kSpinLimit = 1u << 20;       // polls of a flag (about a second)
constexpr int kGroups = FusedSync::kGroups;
constexpr int kMaxParts = FusedSync::kMaxParts;

struct FusedSmem {
  int ids[MOE_MAX_TOP_K];   // routed experts in rank order
  float w[MOE_MAX_TOP_K];
  int act[kFSlots];         // expert of segment a (n_experts: shared), ascending
  float wseg[kFSlots];      // routing weight of segment a's slot (1: shared)
  int ok;
  union {
    struct {
      __bf16 x[kFWaves][8 * 128 + 8];  // wavefront w: its quarter of x
      f32x4 red[kFWaves - 1][2][kWave];
    } gu;
    struct {
      __bf16 hi[kFWaves][kFSlots][kHRow];  // wavefront w: w_a * h of its step
      __bf16 lo[kFWaves][kFSlots][kHRow];
      f32x4 red[kFWaves - 1][kWave];
    } dn;
  } u;
};

// Synchronisation words live in the caller's workspace and carry the call's
// epoch (a 64-bit value the host never repeats), so nothing needs resetting
// between calls and no word is ever read-modify-written: device-wide atomic
// updates of one address serialise at the memory (~0.1 us each), and a
// thousand of them would cost a whole decode step.
//
// Every word that passes between workgroups during the call (h, the partial
// sums, the flags) is stored and loaded at device scope, which on this GPU
// writes through and reads past the per-XCD L2 caches.  Publishing therefore
// needs no cache writeback or invalidate (a device-scope fence is one of
// each, over the whole L2 of the XCD, and a thousand workgroups fencing at
// once stall every load behind them): every wavefront waits until its stores
// have completed (stores_done; __syncthreads alone does not wait for them),
// the workgroup meets at a barrier, and only then is its flag stored.
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
__device__ __forceinline__ u32x4 ld_dev16(const void* a) {
  const uint64_t v0 = ld_dev8(a), v1 = ld_dev8(static_cast<const char*>(a) + 8);
  return u32x4{(uint32_t)v0, (uint32_t)(v0 >> 32), (uint32_t)v1, (uint32_t)(v1 >> 32)};
}
__device__ __forceinline__ float ld_dev_f32(const float* a) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(a)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Grid barrier over `grid` resident workgroups, in two halves so that the
// caller can request loads in between: arrive() stores this workgroup's
// arrival flag once its earlier stores have completed; wait() has workgroup 0
// wait for every flag and then post the epoch into kGroups release words on
// separate cache lines, while workgroup b waits on word b % kGroups.  wait()
// returns false on timeout (a bounded wait).
__device__ void arrive(const FusedParams& f) {
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) post(f.sync->arrive + blockIdx.x, f.epoch);
}

__device__ bool wait_release(const FusedParams& f, FusedSmem& sm) {
  const unsigned long long ep = f.epoch;
  if (blockIdx.x == 0 && threadIdx.x < kWave) {
    // lane l watches flags l, l + 64, ...; a flag once seen is not read again
    uint32_t spins = 0;
    uint32_t seen = 0;
    int ok = 1;
    for (;;) {
      int i = 0;
      for (int b = threadIdx.x; b < f.grid; b += kWave, ++i)
        if (!((seen >> i) & 1u) && poll(f.sync->arrive + b) == ep) seen |= 1u << i;
      const uint32_t want = f.grid > threadIdx.x ? (2u << ((f.grid - 1 - threadIdx.x) / kWave)) - 1u : 0u;
      if (__ballot(seen != want) == 0) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        ok = 0;
        break;
      }
    }
    if (ok && threadIdx.x < kGroups) post(&f.sync->release[threadIdx.x].v, ep);
    if (threadIdx.x == 0) sm.ok = ok;
  } else if (threadIdx.x == 0) {
    const unsigned long long* r = &f.sync->release[blockIdx.x % kGroups].v;
    uint32_t spins = 0;
    int ok = 1;
    while (poll(r) != ep) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        ok = 0;
        break;
      }
    }
    sm.ok = ok;
  }
  __syncthreads();
  return sm.ok != 0;
}

template <int S>
__global__ __launch_bounds__(kFThreads) void decode_fused_kernel(FusedParams f) {
  const FfnParams& p = f.p;
  __shared__ FusedSmem sm;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 4, r16 = lane & 15;
  const int k = p.top_k;
  const int nseg = k + p.has_shared;

  // ---- 1. routing and grouping
  if (wave == 0) {
    int id;
    float wt;
    route_token<kFPer>(f.logits, p.n_experts, k, f.routed_scale, lane, id, wt);
    // slot of rank i = number of chosen experts below id (ids are distinct)
    int below = 0;
    for (int j = 0; j < k; ++j) below += read_lane(id, j) < id ? 1 : 0;
    if (lane < k) {
      sm.ids[lane] = id;
      sm.w[lane] = wt;
      sm.act[below] = id;
      sm.wseg[below] = wt;
    }
    if (lane == 0 && p.has_shared) {
      sm.act[k] = p.n_experts;
      sm.wseg[k] = 1.0f;
    }
    if (blockIdx.x == 0 && lane < k) {
      f.topk_ids[lane] = id;
      f.topk_w[lane] = wt;
      f.perm[below] = lane;
      f.inv_perm[lane] = below;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < p.n_experts; e += kFThreads) {
      int c = 0, off = 0;
      for (int j = 0; j < k; ++j) {
        c += sm.ids[j] == e ? 1 : 0;
        off += sm.ids[j] < e ? 1 : 0;
      }
      f.counts[e] = c;
      f.offsets[e] = off;
    }
    if (threadIdx.x == 0) f.offsets[p.n_experts] = k;
  }

  // ---- 2. gate/up: x staged once per workgroup, each wavefront its quarter
  for (int c = lane; c < 16 * S; c += kWave)
    *reinterpret_cast<u32x4*>(&sm.u.gu.x[wave][c * 8]) =
        load16(static_cast<const __bf16*>(p.x) + wave * S * 128 + c * 8);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's rows are written
  __builtin_amdgcn_wave_barrier();

  const int rbr = p.inter >> 4;
  const int gu_items = k * rbr + (p.has_shared ? p.shared_inter >> 4 : 0);
  const int64_t cb = p.hidden / 2, sb = p.hidden / 32;
  for (int item = blockIdx.x; item < gu_items; item += gridDim.x) {
    const int a = uniform(item < k * rbr ? item / rbr : k);
    const int rb = uniform(item < k * rbr ? item - a * rbr : item - k * rbr);
    const int e = uniform(sm.act[a]);
    const bool shared = e == p.n_experts;
    const int rows = shared ? p.shared_inter : p.inter;
    const int64_t row = (shared ? 0 : (int64_t)e * rows) + rb * 16 + r16;
    const uint8_t* gc = (shared ? p.sgate_c : p.gate_c) + row * cb + wave * S * 64 + g * 16;
    const uint8_t* uc = (shared ? p.sup_c : p.up_c) + row * cb + wave * S * 64 + g * 16;
    const uint8_t* gs = (shared ? p.sgate_s : p.gate_s) + row * sb + wave * S * 4;
    const uint8_t* us = (shared ? p.sup_s : p.up_s) + row * sb + wave * S * 4;
    u32x4 qg[S], qu[S];
#pragma unroll
    for (int j = 0; j < S; ++j) {
      qg[j] = load16(gc + j * 64);
      qu[j] = load16(uc + j * 64);
    }
    uint32_t wg[S], wu[S];
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
    f32x4 ag = f32x4{0, 0, 0, 0}, au = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < S; ++j) {
      // token column 0 only; the other columns multiply zeros
      bf16x8 b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[t] = as_bf16x8(r16 == 0 ? *reinterpret_cast<const u32x4*>(
                                        &sm.u.gu.x[wave][j * 128 + g * 32 + 8 * t])
                                  : u32x4{0, 0, 0, 0});
      const float sgv = ue8m0_to_f32((wg[j] >> (8 * g)) & 0xFF);
      const float suv = ue8m0_to_f32((wu[j] >> (8 * g)) & 0xFF);
#pragma unroll
      for (int t = 0; t < 4; ++t) ag = mfma_bf16(fp4x8_to_bf16(qg[j][t], sgv), b[t], ag);
#pragma unroll
      for (int t = 0; t < 4; ++t) au = mfma_bf16(fp4x8_to_bf16(qu[j][t], suv), b[t], au);
    }
    if (wave > 0) {
      sm.u.gu.red[wave - 1][0][lane] = ag;
      sm.u.gu.red[wave - 1][1][lane] = au;
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kFWaves - 1; ++w) {
        ag += sm.u.gu.red[w][0][lane];
        au += sm.u.gu.red[w][1][lane];
      }
      if (r16 == 0) {
        bf16x4 hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = ag[r];
          const float h = gv / (1.0f + expf(-gv)) * au[r];
          __bf16 x0, x1;
          split_bf16(h, x0, x1);
          hi[r] = x0;
          lo[r] = x1;
        }
        const int64_t o = (int64_t)a * p.h_stride + rb * 16 + 4 * g;
        st_dev8(p.h_hi + o, __builtin_bit_cast(uint64_t, hi));
        st_dev8(p.h_lo + o, __builtin_bit_cast(uint64_t, lo));
      }
    }
    __syncthreads();
  }

  // ---- 3. the first down item's codes, then the grid barrier
  const int nq = p.inter / 512;  // 512-wide parts of the intermediate dimension
  const int dn_items = (p.hidden >> 4) * nq;
  const int64_t dcb = p.inter / 2, dsb = p.inter / 32;
  u32x4 dq[kFSlots];
  uint32_t ds[kFSlots];
  auto load_down = [&](int item) {
    const int rb = item / nq, q = item - (item / nq) * nq;
    const int ks = 4 * q + wave;
#pragma unroll
    for (int a = 0; a < kFSlots; ++a) {
      const int aa = a < nseg ? a : 0;
      const int e = uniform(sm.act[aa]);
      const bool shared = e == p.n_experts;
      const int64_t row = (shared ? 0 : (int64_t)e * p.hidden) + rb * 16 + r16;
      const uint8_t* c = (shared ? p.sdown_c : p.down_c) + row * dcb + ks * 64 + g * 16;
      const uint8_t* s = (shared ? p.sdown_s : p.down_s) + row * dsb + ks * 4 + g;
      if (a < nseg) {
        dq[a] = load16(c);
        ds[a] = *s;
      }
    }
  };
  arrive(f);
  if (blockIdx.x < dn_items) load_down(blockIdx.x);
  if (!wait_release(f, sm)) {
    if (threadIdx.x == 0 && f.dev_error) atomicOr(f.dev_error, MOE_DEVERR_SYNC);
    return;
  }

  // ---- 4. down: item (16 rows, part q), wavefront w takes step 4q + w
  for (int item = blockIdx.x; item < dn_items; item += gridDim.x) {
    if (item != (int)blockIdx.x) load_down(item);
    const int rb = item / nq, q = item - (item / nq) * nq;
    const int ks = 4 * q + wave;
    // stage w_a * (h_hi + h_lo) of this step for every segment, split again
    for (int c = lane; c < nseg * 16; c += kWave) {
      const int a = c >> 4, c16 = c & 15;
      const int64_t o = (int64_t)a * p.h_stride + ks * 128 + c16 * 8;
      const bf16x8 hh = as_bf16x8(ld_dev16(p.h_hi + o));
      const bf16x8 hl = as_bf16x8(ld_dev16(p.h_lo + o));
      const float wa = sm.wseg[a];
      bf16x8 oh, ol;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = wa * (static_cast<float>(hh[j]) + static_cast<float>(hl[j]));
        __bf16 x0, x1;
        split_bf16(v, x0, x1);
        oh[j] = x0;
        ol[j] = x1;
      }
      *reinterpret_cast<u32x4*>(&sm.u.dn.hi[wave][a][c16 * 8]) = __builtin_bit_cast(u32x4, oh);
      *reinterpret_cast<u32x4*>(&sm.u.dn.lo[wave][a][c16 * 8]) = __builtin_bit_cast(u32x4, ol);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    f32x4 acc_h = f32x4{0, 0, 0, 0}, acc_l = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int a = 0; a < kFSlots; ++a) {
      if (a < nseg) {  // uniform
        const float sc = ue8m0_to_f32(ds[a]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 wv = fp4x8_to_bf16(dq[a][j], sc);
          const bf16x8 bh = as_bf16x8(r16 == 0 ? *reinterpret_cast<const u32x4*>(
                                                     &sm.u.dn.hi[wave][a][g * 32 + 8 * j])
                                               : u32x4{0, 0, 0, 0});
          const bf16x8 bl = as_bf16x8(r16 == 0 ? *reinterpret_cast<const u32x4*>(
                                                     &sm.u.dn.lo[wave][a][g * 32 + 8 * j])
                                               : u32x4{0, 0, 0, 0});
          acc_h = mfma_bf16(wv, bh, acc_h);
          acc_l = mfma_bf16(wv, bl, acc_l);
        }
      }
    }
    f32x4 acc = acc_h + acc_l;
    if (wave > 0) sm.u.dn.red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kFWaves - 1; ++w) acc += sm.u.dn.red[w][lane];
      if (r16 == 0) {
        float* o = f.partial + (int64_t)q * p.hidden + rb * 16 + 4 * g;
        st_dev8(o, ((uint64_t)__float_as_uint(acc[1]) << 32) | __float_as_uint(acc[0]));
        st_dev8(o + 2, ((uint64_t)__float_as_uint(acc[3]) << 32) | __float_as_uint(acc[2]));
      }
    }
    // part 0 of the row block waits for the other parts and adds them up in
    // order (all workgroups are resident and no part waits on anything after
    // the grid barrier, so the wait ends)
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) post(f.sync->part + (int64_t)rb * kMaxParts + q, f.epoch);
    if (q == 0) {
      if (threadIdx.x == 0) {
        int ok = 1;
        uint32_t spins = 0;
        for (int qq = 1; qq < nq && ok; ++qq) {
          while (poll(f.sync->part + (int64_t)rb * kMaxParts + qq) != f.epoch) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
              ok = 0;
              break;
            }
          }
        }
        sm.ok = ok;
      }
      __syncthreads();
      if (!sm.ok) {
        if (threadIdx.x == 0 && f.dev_error) atomicOr(f.dev_error, MOE_DEVERR_SYNC);
      } else if (threadIdx.x < 16) {
        float sum = 0.0f;
        for (int qq = 0; qq < nq; ++qq)
          sum += ld_dev_f32(f.partial + (int64_t)qq * p.hidden + rb * 16 + threadIdx.x);
        p.y[rb * 16 + threadIdx.x] = sum;
      }
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
template <int S>
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
          &per_cu, reinterpret_cast<const void*>(decode_fused_kernel<S>), kFThreads, 0);
    if (status == hipSuccess) cached = per_cu * cus;
  }
  *grid = cached;
  return status;
}

template <int S>
hipError_t fused_launch(FusedParams f, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  int grid = 0;
  const hipError_t e = resident_grid<S>(&grid);
  if (e != hipSuccess) return e;
  if (grid < 1) return hipErrorInvalidConfiguration;
  if (grid > FusedSync::kMaxGrid) grid = FusedSync::kMaxGrid;  // still all resident
  f.grid = grid;
  return launch(decode_fused_kernel<S>, dim3(grid), dim3(kFThreads), 0, stream, start, stop, f);
}

}  // namespace

int fused_decode_steps(const FfnParams& p) {
  if (p.n_tokens != 1 || p.x_f32 || p.w_type != MOE_W_MXFP4) return 0;
  if (p.n_experts > kFPer * kWave || p.top_k > MOE_MAX_TOP_K) return 0;
  if (p.has_shared && (p.sw_type != MOE_W_MXFP4 || p.shared_inter != p.inter)) return 0;
  if (p.inter % 512 != 0 || p.hidden % 512 != 0) return 0;
  if (p.inter / 512 > kMaxParts || p.hidden / 16 > FusedSync::kMaxRowBlocks) return 0;
  const int s = p.hidden / 512;
  return (s == 1 || s == 2 || s == 4 || s == 8) ? s : 0;
}

hipError_t launch_decode_fused(const FusedParams& f, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop) {
  switch (fused_decode_steps(f.p)) {
    case 1: return fused_launch<1>(f, stream, start, stop);
    case 2: return fused_launch<2>(f, stream, start, stop);
    case 4: return fused_launch<4>(f, stream, start, stop);
    case 8: return fused_launch<8>(f, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe

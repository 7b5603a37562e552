// Expert FFN on the matrix cores: gate/up with on-the-fly block decode and
// the SwiGLU epilogue, then the down projection with the routing weight and
// the combine.
//
// "DeepSeek-V4-Flash 284B -- Deep-Dive Mathematical & Kernel Guide":
//   section 4, SwiGLU equation: h = SiLU(W_gate x) * (W_up x), y = W_down h,
//     h_j = g_j / (1 + exp(-g_j)) * u_j;
//   section 3.2, combine equation: y = e_shared(x) + sum_i w_i e_{k_i}(x).
// "DeepSeek V4 target engine (CPU + optional CUDA tier)", introduction:
//   routed experts in MXFP4, dense (shared) weights in fp8-e4m3 + UE8M0.
//
// Work decomposition.  A segment is one routed expert (grouped slots
// offsets[e] .. offsets[e+1]) or the shared expert (slots N*k .. N*k+N-1,
// token t at slot N*k + t).  A segment is cut into token tiles of TN = 16*NBT
// slots and blocks of 16 output rows; one work item is (segment, tile, row
// block).  Every workgroup rebuilds the item prefix from the device-side
// counts (no host synchronisation) and walks the items with a grid stride.
//
// Inside an item the four wavefronts split the reduction dimension in steps
// of 128: in step ks lane l owns row (l % 16) and the 32 consecutive
// reduction indices ks*128 + 32*(l/16) .. +31 -- one MXFP4 block, i.e. 16
// code bytes and one scale byte (fp8: 32 bytes, one scale per step).  Those
// 32 decoded weights feed four 16x16x32 MFMAs (sub-step j takes indices
// +8j .. +8j+7); the activation (or h) operand is loaded with the same index
// map, so the products pair up.  A wavefront issues the code loads of up to
// CH steps before decoding any of them, so each one keeps several KiB of
// weights in flight.  The partial sums of the four wavefronts meet in LDS.
//
// Combine.  The down kernel writes each slot's weighted output to the
// workspace; the last workgroup to finish a 16-row block (an agent-scope
// counter per block) sums that block for every token in a fixed order --
// shared first, then slots 0..k-1 -- so y is deterministic and no separate
// combine launch is needed.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSeg = MOE_MAX_EXPERTS + 1;
constexpr int kMaxGrid = 256 * 8;  // 256 CUs, up to 8 resident workgroups each

// ------------------------------------------------------------ work items

struct Item {
  int seg;
  int slot0;  // first slot of the tile
  int m;      // slots in the tile (1..TN)
  int row0;   // first output row of the block
};

__device__ __forceinline__ int seg_items(const FfnParams& p, int s, int tn, bool down) {
  const bool shared = s == p.n_experts;
  const int m = shared ? p.n_tokens : p.counts[s];
  const int rows = down ? p.hidden : (shared ? p.shared_inter : p.inter);
  return (m + tn - 1) / tn * (rows >> 4);
}

// s_pref[s] = items in segments before s; s_pref[nseg] = total.
__device__ int build_item_prefix(const FfnParams& p, int tn, bool down, int* s_pref,
                                 int* s_tmp) {
  const int nseg = p.n_experts + p.has_shared;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (nseg + kThreads - 1) / kThreads;
  const int s0 = tid * per;
  const int s1 = min(s0 + per, nseg);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += seg_items(p, s, tn, down);
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) s_tmp[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_tmp[w];
  int run = before + incl - local;
  for (int s = s0; s < s1; ++s) {
    s_pref[s] = run;
    run += seg_items(p, s, tn, down);
  }
  if (tid == kThreads - 1) s_pref[nseg] = before + incl;
  __syncthreads();
  return s_pref[nseg];
}

__device__ __forceinline__ Item find_item(const FfnParams& p, const int* s_pref, int item,
                                          int tn, bool down) {
  int lo = 0, hi = p.n_experts + p.has_shared;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= item)
      lo = mid;
    else
      hi = mid;
  }
  const bool shared = lo == p.n_experts;
  const int rows = down ? p.hidden : (shared ? p.shared_inter : p.inter);
  const int rbn = rows >> 4;
  const int local = item - s_pref[lo];
  const int tile = local / rbn;
  const int rb = local - tile * rbn;
  const int m_all = shared ? p.n_tokens : p.counts[lo];
  const int start = shared ? p.n_tokens * p.top_k : p.offsets[lo];
  Item it;
  it.seg = lo;
  it.slot0 = start + tile * tn;
  it.m = min(tn, m_all - tile * tn);
  it.row0 = rb * 16;
  return it;
}

// ------------------------------------------------------- weight formats

// Per reduction step a lane holds Q 16-byte code vectors and one scale.
template <int WT>
struct Fmt;

template <>
struct Fmt<MOE_W_MXFP4> {
  static constexpr int Q = 1;
  static constexpr int CH = 8;  // steps preloaded per chunk
  __device__ static int64_t row_bytes(int cols) { return cols / 2; }
  __device__ static int64_t scale_row_bytes(int cols) { return cols / 32; }
  __device__ static int code_off(int ks, int g) { return ks * 64 + g * 16; }
  __device__ static int scale_off(int ks, int g) { return ks * 4 + g; }
  __device__ static void decode(const u32x4 (&q)[Q], uint32_t u, bf16x8 (&a)[4]) {
    const float s = ue8m0_to_f32(u);
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = fp4x8_to_bf16(q[0][j], s);
  }
};

template <>
struct Fmt<MOE_W_FP8E4M3_B128> {
  static constexpr int Q = 2;
  static constexpr int CH = 4;
  __device__ static int64_t row_bytes(int cols) { return cols; }
  __device__ static int64_t scale_row_bytes(int cols) { return cols / 128; }
  __device__ static int code_off(int ks, int g) { return ks * 128 + g * 32; }
  __device__ static int scale_off(int ks, int) { return ks; }
  __device__ static void decode(const u32x4 (&q)[Q], uint32_t u, bf16x8 (&a)[4]) {
    const float s = ue8m0_to_f32(u);
    a[0] = fp8x8_to_bf16(q[0][0], q[0][1], s);
    a[1] = fp8x8_to_bf16(q[0][2], q[0][3], s);
    a[2] = fp8x8_to_bf16(q[1][0], q[1][1], s);
    a[3] = fp8x8_to_bf16(q[1][2], q[1][3], s);
  }
};

template <int WT>
__device__ __forceinline__ void load_codes(const uint8_t* crow, const uint8_t* srow, int ks,
                                           int g, u32x4 (&q)[Fmt<WT>::Q], uint32_t& u) {
  const uint8_t* c = crow + Fmt<WT>::code_off(ks, g);
#pragma unroll
  for (int i = 0; i < Fmt<WT>::Q; ++i) q[i] = load16(c + 16 * i);
  u = srow[Fmt<WT>::scale_off(ks, g)];
}

// ------------------------------------------------------- B operands

// 32 consecutive bf16 values -> four B fragments (zeros for a null row).
__device__ __forceinline__ void load_bf16_32(const __bf16* src, bf16x8 (&b)[4]) {
  if (src) {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(load16(src + 8 * j));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(u32x4{0, 0, 0, 0});
  }
}

// 32 consecutive fp32 values -> high and low bf16 B fragments.
__device__ __forceinline__ void load_f32_32(const float* src, bf16x8 (&hi)[4], bf16x8 (&lo)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 v = src ? *reinterpret_cast<const f32x4*>(src + 8 * j + 4 * h) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        __bf16 a, b;
        split_bf16(v[r], a, b);
        hi[j][4 * h + r] = a;
        lo[j][4 * h + r] = b;
      }
    }
  }
}

// number of reduction steps ks = wave + 4j below nks
__device__ __forceinline__ int wave_steps(int nks, int wave) {
  return nks > wave ? (nks - wave + kWaves - 1) / kWaves : 0;
}

// ------------------------------------------------------- gate/up

template <int NBT, bool XF32, int WT>
__device__ __forceinline__ void gate_up_item(const FfnParams& p, const Item& it, bool shared,
                                             int wave, int g, int r16, f32x4 (&ag)[NBT],
                                             f32x4 (&au)[NBT]) {
  using F = Fmt<WT>;
  constexpr int CH = F::CH;
  const int rows = shared ? p.shared_inter : p.inter;
  const int64_t cb = F::row_bytes(p.hidden);
  const int64_t sb = F::scale_row_bytes(p.hidden);
  const int64_t row = (shared ? 0 : (int64_t)it.seg * rows) + it.row0 + r16;
  const uint8_t* gcr = (shared ? p.sgate_c : p.gate_c) + row * cb;
  const uint8_t* gsr = (shared ? p.sgate_s : p.gate_s) + row * sb;
  const uint8_t* ucr = (shared ? p.sup_c : p.up_c) + row * cb;
  const uint8_t* usr = (shared ? p.sup_s : p.up_s) + row * sb;

  // activation row of each of this lane's token columns
  const int64_t shared_base = (int64_t)p.n_tokens * p.top_k;
  const char* xr[NBT];
#pragma unroll
  for (int tb = 0; tb < NBT; ++tb) {
    const int n = tb * 16 + r16;
    xr[tb] = nullptr;
    if (n < it.m) {
      const int64_t slot = it.slot0 + n;
      const int64_t tok = shared ? slot - shared_base : p.perm[slot] / p.top_k;
      xr[tb] = static_cast<const char*>(p.x) + tok * p.hidden * (XF32 ? 4 : 2);
    }
  }
  const int nbt = (it.m + 15) >> 4;
  const int S = wave_steps(p.hidden / 128, wave);

  for (int j0 = 0; j0 < S; j0 += CH) {
    const int rem = min(CH, S - j0);
    u32x4 qg[CH][F::Q], qu[CH][F::Q];
    uint32_t sg[CH], su[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < rem) {
        const int ks = wave + kWaves * (j0 + i);
        load_codes<WT>(gcr, gsr, ks, g, qg[i], sg[i]);
        load_codes<WT>(ucr, usr, ks, g, qu[i], su[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < rem) {
        const int kofs = (wave + kWaves * (j0 + i)) * 128 + g * 32;
        bf16x8 wg[4], wu[4];
        F::decode(qg[i], sg[i], wg);
        F::decode(qu[i], su[i], wu);
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
          if (tb >= nbt) break;
          if constexpr (XF32) {
            bf16x8 bh[4], bl[4];
            load_f32_32(xr[tb] ? reinterpret_cast<const float*>(xr[tb]) + kofs : nullptr, bh,
                        bl);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              ag[tb] = mfma_bf16(wg[j], bh[j], ag[tb]);
              ag[tb] = mfma_bf16(wg[j], bl[j], ag[tb]);
              au[tb] = mfma_bf16(wu[j], bh[j], au[tb]);
              au[tb] = mfma_bf16(wu[j], bl[j], au[tb]);
            }
          } else {
            bf16x8 b[4];
            load_bf16_32(xr[tb] ? reinterpret_cast<const __bf16*>(xr[tb]) + kofs : nullptr, b);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              ag[tb] = mfma_bf16(wg[j], b[j], ag[tb]);
              au[tb] = mfma_bf16(wu[j], b[j], au[tb]);
            }
          }
        }
      }
    }
  }
}

template <int NBT, bool XF32>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(FfnParams p) {
  constexpr int TN = 16 * NBT;
  __shared__ int s_pref[kMaxSeg + 1];
  __shared__ int s_tmp[kWaves];
  __shared__ f32x4 s_red[kWaves - 1][2 * NBT][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;

  // the down kernel's per-row-block counters start from zero every call
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < p.hidden / 16; i += kThreads) p.rb_count[i] = 0;

  const int total = build_item_prefix(p, TN, false, s_pref, s_tmp);
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const Item it = find_item(p, s_pref, item, TN, false);
    const bool shared = it.seg == p.n_experts;
    f32x4 ag[NBT], au[NBT];
#pragma unroll
    for (int tb = 0; tb < NBT; ++tb) {
      ag[tb] = f32x4{0, 0, 0, 0};
      au[tb] = f32x4{0, 0, 0, 0};
    }
    if ((shared ? p.sw_type : p.w_type) == MOE_W_MXFP4)
      gate_up_item<NBT, XF32, MOE_W_MXFP4>(p, it, shared, wave, g, r16, ag, au);
    else
      gate_up_item<NBT, XF32, MOE_W_FP8E4M3_B128>(p, it, shared, wave, g, r16, ag, au);

    if (wave > 0) {
#pragma unroll
      for (int tb = 0; tb < NBT; ++tb) {
        s_red[wave - 1][2 * tb][lane] = ag[tb];
        s_red[wave - 1][2 * tb + 1][lane] = au[tb];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kWaves - 1; ++w) {
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
          ag[tb] += s_red[w][2 * tb][lane];
          au[tb] += s_red[w][2 * tb + 1][lane];
        }
      }
#pragma unroll
      for (int tb = 0; tb < NBT; ++tb) {
        const int n = tb * 16 + r16;
        if (n < it.m) {
          const int64_t slot = it.slot0 + n;
          bf16x4 hi, lo;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gv = ag[tb][r];
            const float h = gv / (1.0f + expf(-gv)) * au[tb][r];
            __bf16 a, b;
            split_bf16(h, a, b);
            hi[r] = a;
            lo[r] = b;
          }
          const int64_t o = slot * p.h_stride + it.row0 + 4 * g;
          *reinterpret_cast<bf16x4*>(p.h_hi + o) = hi;
          *reinterpret_cast<bf16x4*>(p.h_lo + o) = lo;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- down + combine

template <int NBT, int WT>
__device__ __forceinline__ void down_item(const FfnParams& p, const Item& it, bool shared,
                                          int wave, int g, int r16, f32x4 (&acc)[NBT]) {
  using F = Fmt<WT>;
  constexpr int CH = F::CH;
  const int kdim = shared ? p.shared_inter : p.inter;
  const int64_t cb = F::row_bytes(kdim);
  const int64_t sb = F::scale_row_bytes(kdim);
  const int64_t row = (shared ? 0 : (int64_t)it.seg * p.hidden) + it.row0 + r16;
  const uint8_t* dcr = (shared ? p.sdown_c : p.down_c) + row * cb;
  const uint8_t* dsr = (shared ? p.sdown_s : p.down_s) + row * sb;

  const __bf16* hh[NBT];
  const __bf16* hl[NBT];
#pragma unroll
  for (int tb = 0; tb < NBT; ++tb) {
    const int n = tb * 16 + r16;
    hh[tb] = nullptr;
    hl[tb] = nullptr;
    if (n < it.m) {
      const int64_t o = (int64_t)(it.slot0 + n) * p.h_stride;
      hh[tb] = p.h_hi + o;
      hl[tb] = p.h_lo + o;
    }
  }
  const int nbt = (it.m + 15) >> 4;
  const int S = wave_steps(kdim / 128, wave);

  for (int j0 = 0; j0 < S; j0 += CH) {
    const int rem = min(CH, S - j0);
    u32x4 q[CH][F::Q];
    uint32_t su[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (i < rem) load_codes<WT>(dcr, dsr, wave + kWaves * (j0 + i), g, q[i], su[i]);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < rem) {
        const int kofs = (wave + kWaves * (j0 + i)) * 128 + g * 32;
        bf16x8 a[4];
        F::decode(q[i], su[i], a);
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
          if (tb >= nbt) break;
          bf16x8 bh[4], bl[4];
          load_bf16_32(hh[tb] ? hh[tb] + kofs : nullptr, bh);
          load_bf16_32(hl[tb] ? hl[tb] + kofs : nullptr, bl);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[tb] = mfma_bf16(a[j], bh[j], acc[tb]);
            acc[tb] = mfma_bf16(a[j], bl[j], acc[tb]);
          }
        }
      }
    }
  }
}

// y rows [row0, row0+16) of every token from the per-slot outputs, in the
// fixed order shared, slot 0, ..., slot k-1.
__device__ void combine_rows(const FfnParams& p, int row0) {
  const int64_t nk = (int64_t)p.n_tokens * p.top_k;
  for (int idx = threadIdx.x; idx < p.n_tokens * 4; idx += kThreads) {
    const int t = idx >> 2;
    const int64_t q = row0 + 4 * (idx & 3);
    f32x4 acc = f32x4{0, 0, 0, 0};
    if (p.has_shared) acc = *reinterpret_cast<const f32x4*>(p.obuf + (nk + t) * p.hidden + q);
    for (int j = 0; j < p.top_k; ++j) {
      const int pp = p.inv_perm[(int64_t)t * p.top_k + j];
      if (pp >= 0) acc += *reinterpret_cast<const f32x4*>(p.obuf + (int64_t)pp * p.hidden + q);
    }
    *reinterpret_cast<f32x4*>(p.y + (int64_t)t * p.hidden + q) = acc;
  }
}

template <int NBT>
__global__ __launch_bounds__(kThreads) void down_kernel(FfnParams p) {
  constexpr int TN = 16 * NBT;
  __shared__ int s_pref[kMaxSeg + 1];
  __shared__ int s_tmp[kWaves];
  __shared__ int s_last;
  __shared__ f32x4 s_red[kWaves - 1][NBT][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int total = build_item_prefix(p, TN, true, s_pref, s_tmp);
  const int per_block = total / (p.hidden >> 4);  // items that feed one row block

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const Item it = find_item(p, s_pref, item, TN, true);
    const bool shared = it.seg == p.n_experts;
    f32x4 acc[NBT];
#pragma unroll
    for (int tb = 0; tb < NBT; ++tb) acc[tb] = f32x4{0, 0, 0, 0};
    if ((shared ? p.sw_type : p.w_type) == MOE_W_MXFP4)
      down_item<NBT, MOE_W_MXFP4>(p, it, shared, wave, g, r16, acc);
    else
      down_item<NBT, MOE_W_FP8E4M3_B128>(p, it, shared, wave, g, r16, acc);

    if (wave > 0) {
#pragma unroll
      for (int tb = 0; tb < NBT; ++tb) s_red[wave - 1][tb][lane] = acc[tb];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < kWaves - 1; ++w) {
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) acc[tb] += s_red[w][tb][lane];
      }
#pragma unroll
      for (int tb = 0; tb < NBT; ++tb) {
        const int n = tb * 16 + r16;
        if (n < it.m) {
          const int64_t slot = it.slot0 + n;
          const float wt = shared ? 1.0f : p.topk_w[p.perm[slot]];
          *reinterpret_cast<f32x4*>(p.obuf + slot * p.hidden + it.row0 + 4 * g) = acc[tb] * wt;
        }
      }
    }
    // publish this item's outputs, then count it against its row block
    __threadfence();
    __syncthreads();
    const int rb = it.row0 >> 4;
    if (threadIdx.x == 0) s_last = atomicAdd(&p.rb_count[rb], 1) == per_block - 1;
    __syncthreads();
    if (s_last) {
      __threadfence();  // see every other item's outputs
      combine_rows(p, it.row0);
      if (threadIdx.x == 0) p.rb_count[rb] = 0;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- launches

int pick_nbt(int n_tokens) {
  if (n_tokens <= 16) return 1;
  if (n_tokens <= 32) return 2;
  if (n_tokens <= 48) return 3;
  return 4;
}

// Upper bound on the token tiles: sum_e ceil(m_e/TN) <= N*k/TN + min(E, N*k).
int64_t routed_tiles_bound(const FfnParams& p, int tn) {
  const int64_t nk = (int64_t)p.n_tokens * p.top_k;
  return nk / tn + (nk < p.n_experts ? nk : p.n_experts);
}

int grid_for(int64_t items) {
  if (items < 1) return 1;
  return (int)(items < kMaxGrid ? items : kMaxGrid);
}

template <int NBT>
hipError_t gate_up_nbt(const FfnParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  constexpr int TN = 16 * NBT;
  const int64_t shared_tiles = p.has_shared ? (p.n_tokens + TN - 1) / TN : 0;
  const int64_t items = routed_tiles_bound(p, TN) * (p.inter / 16) +
                        shared_tiles * (p.shared_inter / 16);
  const dim3 grid(grid_for(items)), block(kThreads);
  if (p.x_f32)
    hipExtLaunchKernelGGL(gate_up_kernel<NBT, true>, grid, block, 0, stream, start, stop, 0, p);
  else
    hipExtLaunchKernelGGL(gate_up_kernel<NBT, false>, grid, block, 0, stream, start, stop, 0, p);
  return hipGetLastError();
}

template <int NBT>
hipError_t down_nbt(const FfnParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  constexpr int TN = 16 * NBT;
  const int64_t shared_tiles = p.has_shared ? (p.n_tokens + TN - 1) / TN : 0;
  const int64_t items = (routed_tiles_bound(p, TN) + shared_tiles) * (p.hidden / 16);
  hipExtLaunchKernelGGL(down_kernel<NBT>, dim3(grid_for(items)), dim3(kThreads), 0, stream,
                        start, stop, 0, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_gate_up(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                              hipEvent_t stop) {
  switch (pick_nbt(p.n_tokens)) {
    case 1: return gate_up_nbt<1>(p, stream, start, stop);
    case 2: return gate_up_nbt<2>(p, stream, start, stop);
    case 3: return gate_up_nbt<3>(p, stream, start, stop);
    default: return gate_up_nbt<4>(p, stream, start, stop);
  }
}

hipError_t launch_ffn_down(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
  switch (pick_nbt(p.n_tokens)) {
    case 1: return down_nbt<1>(p, stream, start, stop);
    case 2: return down_nbt<2>(p, stream, start, stop);
    case 3: return down_nbt<3>(p, stream, start, stop);
    default: return down_nbt<4>(p, stream, start, stop);
  }
}

}  // namespace moe

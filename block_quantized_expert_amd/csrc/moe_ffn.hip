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
// Small batches (decode) stage the tile's activation rows in LDS once per
// item, and run the down projection and the combine as one pass in which a
// workgroup owns 16 output rows for every token and walks all active
// experts: the routing weight is folded into the staged h, so each token's
// sum builds up in one accumulator in a fixed order (deterministic, no
// per-slot outputs).  Larger batches write weighted per-slot outputs and
// sum them in a separate combine kernel, shared first then slots 0..k-1.
//
// Which gate/up runs: bf16 activations of up to 16 tokens with MXFP4 experts
// take gate_up_decode_kernel; fp32 activations take gate_up_kernel; every
// other batch goes to the grouped GEMMs (moe_gemm.hip), which store h as
// three E4M3 parts for their own down projection.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_formats.h"
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSeg = MOE_MAX_EXPERTS + 1;
constexpr int kMaxGrid = 256 * 8;  // 256 CUs, up to 8 resident workgroups each
constexpr int kLdsBudget = 140 * 1024;  // dynamic LDS a kernel may ask for

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
  it.seg = uniform(lo);
  it.slot0 = uniform(start + tile * tn);
  it.m = uniform(min(tn, m_all - tile * tn));
  it.row0 = uniform(rb * 16);
  return it;
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

// The same from the LDS copy of the activations: `row` is a byte offset into
// s_x (negative: zeros), `k` the first reduction index.
__device__ __forceinline__ void load_bf16_32_lds(const char* s_x, int row, int k,
                                                 bf16x8 (&b)[4]) {
  if (row >= 0) {
    const char* src = s_x + row + k * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(src + 16 * j));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = as_bf16x8(u32x4{0, 0, 0, 0});
  }
}

__device__ __forceinline__ void load_f32_32_lds(const char* s_x, int row, int k,
                                                bf16x8 (&hi)[4], bf16x8 (&lo)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 v = row >= 0 ? *reinterpret_cast<const f32x4*>(s_x + row + (k + 8 * j + 4 * h) * 4)
                         : f32x4{0, 0, 0, 0};
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

// Activation rows of an item's token columns: in global memory, or staged
// in LDS (row stride x_stride bytes) when XLDS.
struct XRows {
  const char* row[4];
};

template <int NBT, bool XF32, bool XLDS, int WT>
__device__ __forceinline__ void gate_up_item(const FfnParams& p, const Item& it, bool shared,
                                             int wave, int g, int r16, char* s_x, int x_stride,
                                             f32x4 (&ag)[NBT], f32x4 (&au)[NBT]) {
  using F = Fmt<WT>;
  constexpr int CH = F::CH;
  constexpr int XB = XF32 ? 4 : 2;  // activation bytes
  const int rows = shared ? p.shared_inter : p.inter;
  const int64_t cb = F::row_bytes(p.hidden);
  const int64_t sb = F::scale_row_bytes(p.hidden);
  const int64_t row = (shared ? 0 : (int64_t)it.seg * rows) + it.row0 + r16;
  const uint8_t* gcr = (shared ? p.sgate_c : p.gate_c) + row * cb;
  const uint8_t* gsr = (shared ? p.sgate_s : p.gate_s) + row * sb;
  const uint8_t* ucr = (shared ? p.sup_c : p.up_c) + row * cb;
  const uint8_t* usr = (shared ? p.sup_s : p.up_s) + row * sb;
  const int64_t shared_base = (int64_t)p.n_tokens * p.top_k;
  const int S = uniform(wave_steps(p.hidden / 128, wave));
  const int nbt = (it.m + 15) >> 4;

  // chunk 0's codes are requested before the activations are staged; a
  // chunk's loads are unconditional (steps past the end repeat the last
  // one) so they leave in one burst
  u32x4 qg[CH][F::Q], qu[CH][F::Q];
  uint32_t sg[CH], su[CH];
  auto load_chunk = [&](int j0) {
    const int last = S - 1;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ks = wave + kWaves * min(j0 + i, last);
      load_codes<WT>(gcr, gsr, ks, g, qg[i], sg[i]);
      load_codes<WT>(ucr, usr, ks, g, qu[i], su[i]);
    }
  };
  if (S > 0) load_chunk(0);

  // token columns: a global activation row, or a byte offset into the LDS
  // copy of the tile (-1 for an empty column)
  const char* xr[NBT];
  int xo[NBT];
  if constexpr (XLDS) {
    const int per_row = p.hidden * XB / 16;
    const int chunks = it.m * per_row;
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
      const int n = c / per_row;
      const int off = (c - n * per_row) * 16;
      const int64_t slot = it.slot0 + n;
      const int64_t tok = shared ? slot - shared_base : p.perm[slot] / p.top_k;
      *reinterpret_cast<u32x4*>(s_x + n * x_stride + off) =
          load16(static_cast<const char*>(p.x) + tok * p.hidden * XB + off);
    }
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < NBT; ++tb) {
      const int n = tb * 16 + r16;
      xo[tb] = n < it.m ? n * x_stride : -1;
      xr[tb] = nullptr;
    }
  } else {
#pragma unroll
    for (int tb = 0; tb < NBT; ++tb) {
      const int n = tb * 16 + r16;
      xr[tb] = nullptr;
      xo[tb] = -1;
      if (n < it.m) {
        const int64_t slot = it.slot0 + n;
        const int64_t tok = shared ? slot - shared_base : p.perm[slot] / p.top_k;
        xr[tb] = static_cast<const char*>(p.x) + tok * p.hidden * XB;
      }
    }
  }

  for (int j0 = 0; j0 < S; j0 += CH) {
    const int rem = min(CH, S - j0);
    if (j0 > 0) load_chunk(j0);
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
            if constexpr (XLDS)
              load_f32_32_lds(s_x, xo[tb], kofs, bh, bl);
            else
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
            if constexpr (XLDS)
              load_bf16_32_lds(s_x, xo[tb], kofs, b);
            else
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

template <int NBT, bool XF32, bool XLDS>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(FfnParams p, int x_stride) {
  constexpr int TN = 16 * NBT;
  extern __shared__ __align__(16) char s_x[];
  __shared__ int s_pref[kMaxSeg + 1];
  __shared__ int s_tmp[kWaves];
  __shared__ f32x4 s_red[kWaves - 1][2 * NBT][kWave];
  // the grouped down's queue counters start this call at 0
  if (blockIdx.x == 0 && threadIdx.x < kQueueWords) p.qctr[threadIdx.x] = 0u;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 4, r16 = lane & 15;

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
      gate_up_item<NBT, XF32, XLDS, MOE_W_MXFP4>(p, it, shared, wave, g, r16, s_x, x_stride,
                                                 ag, au);
    else
      gate_up_item<NBT, XF32, XLDS, MOE_W_FP8E4M3_B128>(p, it, shared, wave, g, r16, s_x,
                                                        x_stride, ag, au);

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
      if (p.lazy_tau > 0.0f && !shared) {
        // the slots' largest |SiLU(g)| over this block's rows
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
          const float mx = silu_col_max(silu_abs_max4(ag[tb]));
          if (g == 0 && tb * 16 + r16 < it.m)
            atomicMax(p.gmax + it.slot0 + tb * 16 + r16, __float_as_uint(mx));
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

// ------------------------------------------------------- gate/up, decode

constexpr int kDecodeMaxTokens = 16;  // one MFMA column block
constexpr int kMaxChunks = MOE_MAX_EXPERTS / kWave;

// Index of the a-th routed expert that has a token, or -1.  Every
// wavefront works it out on its own (no barrier); the count loads are
// issued before any of them is used.
__device__ __forceinline__ int nth_active_expert(const FfnParams& p, int a, int lane) {
  const int nch = (p.n_experts + kWave - 1) / kWave;
  int cnt[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int x = c * kWave + lane;
    cnt[c] = (c < nch && x < p.n_experts) ? p.counts[x] : 0;
  }
  int seen = 0, e = -1;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const uint64_t on = __ballot(cnt[c] > 0);
    const int pc = __popcll(on);
    if (e < 0 && a < seen + pc) {
      const uint64_t below = (1ull << lane) - 1ull;
      const bool me = cnt[c] > 0 && __popcll(on & below) == a - seen;
      e = c * kWave + __builtin_ctzll(__ballot(me));
    }
    seen += pc;
  }
  return uniform(e);
}

// Gate/up for a decode batch (at most 16 tokens, bf16 activations, MXFP4
// gate and up, hidden = 512*S).  Block b < a_bound*inter/16 is row block
// b % (inter/16) of the (b / (inter/16))-th routed expert that has tokens
// (blocks past the last such expert leave at once); the rest are the shared
// expert's row blocks.  Wavefront w owns reduction steps w*S .. w*S+S-1, so
// its 2*S code vectors and its scale bytes (4*S contiguous bytes of each
// row) leave as one burst, and it stages only its own quarter of the
// activations in LDS.  The four partial sums meet in LDS for the SwiGLU.
//
// MODE 0 runs gate and up together.  The gate-first lazy skip ("[RFC /
// Benchmarks] Fitting 284B DeepSeek-V4-Flash in 57.61 GiB RAM", section 5)
// splits the routed blocks over two launches: MODE 1 (routed blocks only)
// computes g, keeps it in gbuf and merges each slot's largest |SiLU(g)| into
// gmax; MODE 2 first reads the tile's slots from gmax and leaves at once,
// before requesting any weight, when every one is below lazy_tau (so a
// skipped expert's up rows are never read), else computes u and writes
// h = SiLU(g) u, with h = 0 for the slots below the threshold; the shared
// expert's blocks run gate and up in MODE 2.
template <int S, int MODE>
__global__ __launch_bounds__(kThreads) void gate_up_decode_kernel(FfnParams p, int a_bound,
                                                                  int m_max) {
  constexpr int kRow = S * 128 + 8;  // bf16 per staged token row (+8: other banks)
  extern __shared__ __align__(16) char s_dyn[];
  __shared__ f32x4 s_red[kWaves - 1][2][kWave];
  // the grouped down's queue counters start this call at 0
  if (blockIdx.x == 0 && threadIdx.x < kQueueWords) p.qctr[threadIdx.x] = 0u;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 4, r16 = lane & 15;
  const int rb_r = p.inter >> 4;
  const int routed_blocks = a_bound * rb_r;
  const int blk = blockIdx.x;
  int e, rb;
  if (blk < routed_blocks) {
    const int a = blk / rb_r;
    rb = blk - a * rb_r;
    e = nth_active_expert(p, a, lane);
    if (e < 0) return;  // the same on every wavefront: the block leaves whole
  } else {
    if (MODE == 1) return;  // not launched: MODE 1 has the routed blocks only
    e = p.n_experts;
    rb = blk - routed_blocks;
  }
  const bool shared = e == p.n_experts;
  // tokens of the tile; distinct ids per token keep m <= N (<= m_max), the
  // clamp keeps repeated ids (outside the ABI's preconditions) inside the
  // staged rows
  const int m = uniform(min(shared ? p.n_tokens : p.counts[e], m_max));
  const int slot0 = uniform(shared ? p.n_tokens * p.top_k : p.offsets[e]);
  bool col_live = r16 < m;  // MODE 2: the column's slot passes the threshold
  if (MODE == 2 && !shared) {
    const float gm = __uint_as_float(p.gmax[slot0 + min(r16, m - 1)]);
    col_live = col_live && gm >= p.lazy_tau;
    if (__ballot(col_live) == 0) return;  // the same in every wavefront
  }
  const bool do_gate = MODE != 2 || shared;  // uniform
  const bool do_up = MODE != 1;
  const int rows = shared ? p.shared_inter : p.inter;
  const int64_t cb = p.hidden / 2, sb = p.hidden / 32;
  const int64_t row = (shared ? 0 : (int64_t)e * rows) + rb * 16 + r16;
  const uint8_t* gc = (shared ? p.sgate_c : p.gate_c) + row * cb + wave * S * 64 + g * 16;
  const uint8_t* uc = (shared ? p.sup_c : p.up_c) + row * cb + wave * S * 64 + g * 16;
  const uint8_t* gs = (shared ? p.sgate_s : p.gate_s) + row * sb + wave * S * 4;
  const uint8_t* us = (shared ? p.sup_s : p.up_s) + row * sb + wave * S * 4;

  // one burst: codes, then the 4*S scale bytes of each row as whole words
  u32x4 qg[S], qu[S];
  uint32_t wg[S], wu[S];
  if (do_gate) {
#pragma unroll
    for (int j = 0; j < S; ++j) qg[j] = load16(gc + j * 64);
  }
  if (do_up) {
#pragma unroll
    for (int j = 0; j < S; ++j) qu[j] = load16(uc + j * 64);
  }
  if constexpr (S >= 4) {
#pragma unroll
    for (int v = 0; v < S / 4; ++v) {
      if (do_gate) {
        const u32x4 a4 = load16(gs + 16 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) wg[4 * v + i] = a4[i];
      }
      if (do_up) {
        const u32x4 b4 = load16(us + 16 * v);
#pragma unroll
        for (int i = 0; i < 4; ++i) wu[4 * v + i] = b4[i];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      if (do_gate) wg[j] = reinterpret_cast<const uint32_t*>(gs)[j];
      if (do_up) wu[j] = reinterpret_cast<const uint32_t*>(us)[j];
    }
  }

  // this wavefront's quarter of the tile's activations
  __bf16* s_xq = reinterpret_cast<__bf16*>(s_dyn) + (size_t)wave * m_max * kRow;
  for (int c = lane; c < m * 16 * S; c += kWave) {
    const int n = c / (16 * S);
    const int off = c - n * 16 * S;  // 16-byte chunk inside the quarter
    const int64_t tok = shared ? n : p.perm[slot0 + n] / p.top_k;
    *reinterpret_cast<u32x4*>(s_xq + n * kRow + off * 8) =
        load16(static_cast<const __bf16*>(p.x) + tok * p.hidden + wave * S * 128 + off * 8);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS rows are written
  __builtin_amdgcn_wave_barrier();

  f32x4 ag = f32x4{0, 0, 0, 0}, au = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < S; ++j) {
    bf16x8 b[4];
    if (r16 < m) {
      const __bf16* src = s_xq + r16 * kRow + j * 128 + g * 32;
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(src + 8 * t));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
    if (do_gate) {
      const float sgv = ue8m0_to_f32((wg[j] >> (8 * g)) & 0xFF);
#pragma unroll
      for (int t = 0; t < 4; ++t) ag = mfma_bf16(fp4x8_to_bf16(qg[j][t], sgv), b[t], ag);
    }
    if (do_up) {
      const float suv = ue8m0_to_f32((wu[j] >> (8 * g)) & 0xFF);
#pragma unroll
      for (int t = 0; t < 4; ++t) au = mfma_bf16(fp4x8_to_bf16(qu[j][t], suv), b[t], au);
    }
  }

  if (wave > 0) {
    s_red[wave - 1][0][lane] = ag;
    s_red[wave - 1][1][lane] = au;
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) {
      ag += s_red[w][0][lane];
      au += s_red[w][1][lane];
    }
    if (MODE == 1) {
      // g of rows rb*16 + 4g .. +3 for the column's slot, and the slot's
      // largest |SiLU(g)| over the block's 16 rows
      const float mx = silu_col_max(silu_abs_max4(ag));
      if (r16 < m) {
        *reinterpret_cast<f32x4*>(p.gbuf + (int64_t)(slot0 + r16) * p.inter + rb * 16 + 4 * g) =
            ag;
        if (g == 0) atomicMax(p.gmax + slot0 + r16, __float_as_uint(mx));
      }
    } else if (r16 < m) {
      if (MODE == 2 && !shared)
        ag = *reinterpret_cast<const f32x4*>(p.gbuf + (int64_t)(slot0 + r16) * p.inter +
                                             rb * 16 + 4 * g);
      bf16x4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = ag[r];
        const float h = col_live ? gv / (1.0f + expf(-gv)) * au[r] : 0.0f;
        __bf16 a, b;
        split_bf16(h, a, b);
        hi[r] = a;
        lo[r] = b;
      }
      const int64_t o = (int64_t)(slot0 + r16) * p.h_stride + rb * 16 + 4 * g;
      *reinterpret_cast<bf16x4*>(p.h_hi + o) = hi;
      *reinterpret_cast<bf16x4*>(p.h_lo + o) = lo;
    }
  }
}

// ------------------------------------------------------- combine

// y[t] = o_shared[t] + sum_i w[t*k + i] * o[inv_perm[t*k + i]], in that
// fixed order, leaving out slots dropped by tail pruning or by the lazy
// skip; four features (three words of 24-bit floats per slot) per thread.
// UNIFORM (hidden a multiple of 256): a wavefront's 256 features lie in one
// token, whose slots and weights are then read once per wavefront through
// the scalar cache instead of by every lane.  K = top_k: the token's slot
// indices and weights, then all its output loads, are issued with no branch
// between them (a dropped slot loads slot 0's outputs and is not added).
template <bool UNIFORM, int K>
__global__ __launch_bounds__(256) void combine_kernel(FfnParams p) {
  const int h4 = p.hidden / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.n_tokens * h4) return;
  const int64_t t = UNIFORM ? (int64_t)__builtin_amdgcn_readfirstlane((int)(i / h4)) : i / h4;
  const int64_t q = (i - t * h4) * 4;
  // slot s's four features at word (s * hidden + q) / 4 * 3
  auto slot_out = [&](int64_t s) { return load_f24x4(p.obuf + (s * p.hidden + q) / 4 * 3); };
  int pp[K];
  float wj[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    pp[j] = p.inv_perm[t * K + j];
    wj[j] = p.topk_w[t * K + j];
  }
  if (p.lazy_tau != 0.0f) {
    // a slot the lazy skip drops contributes nothing
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (pp[j] >= 0 && __uint_as_float(p.gmax[pp[j]]) < p.lazy_tau) pp[j] = -1;
  }
  f32x4 o[K];
#pragma unroll
  for (int j = 0; j < K; ++j) o[j] = slot_out(pp[j] >= 0 ? pp[j] : 0);
  // the sum in the fixed order: shared, then slot 0 .. top_k-1
  f32x4 acc = f32x4{0, 0, 0, 0};
  if (p.has_shared) acc = slot_out((int64_t)p.n_tokens * K + t);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const f32x4 a = acc + wj[j] * o[j];
    acc = pp[j] >= 0 ? a : acc;
  }
  *reinterpret_cast<f32x4*>(p.y + t * p.hidden + q) = acc;
}


// ------------------------------------------------------- down + combine, small batch

constexpr int kSmallWaves = 8;
constexpr int kSmallThreads = kSmallWaves * kWave;
constexpr int kSmallMaxTokens = 16;  // one MFMA column per token
constexpr int kSmallMaxSlots = 128;
constexpr int kSmallMaxActive = kSmallMaxSlots + 1;
constexpr int kStageRow = 136;  // bf16 per staged row: 128 + 8 so rows start on other banks

// One workgroup per 16 output rows.  Units (active expert a, step s of the
// current chunk) are dealt to the eight wavefronts; a unit decodes the 16
// rows x 128 reduction indices of expert a's down matrix and multiplies
// them with the staged w*h of every token (column n = token n, zero where
// the token did not pick the expert).
//
// Latency order: the routing inputs arrive in one round trip (the slot and
// weight of every flat entry through inv_perm and topk_w, the counts and
// first slots of every expert); then the chunk's first h values and all of
// a wavefront's weight codes leave as one burst, so the h staging overlaps
// the weight transfer; the B fragments of unit b+1 are read from LDS while
// unit b multiplies.
template <int WT, int SWT>
__global__ __launch_bounds__(kSmallThreads) void down_combine_small_kernel(FfnParams p,
                                                                            int spc) {
  constexpr bool kMerged = WT == SWT;  // the shared expert's units join the bursts
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_act[kSmallMaxActive];   // expert id (n_experts: shared)
  __shared__ int s_off[kSmallMaxActive];   // first slot of the active expert
  __shared__ int16_t s_col[kSmallMaxActive][kSmallMaxTokens];  // slot of token n or -1
  __shared__ float s_w[kSmallMaxSlots];
  __shared__ int s_nact, s_nroute;
  __shared__ f32x4 s_red[kSmallWaves - 1][kWave];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 4, r16 = lane & 15;
  const int row0 = blockIdx.x * 16;
  const int nk = p.n_tokens * p.top_k;  // >= 1 on this path
  const int n_slots = nk + (p.has_shared ? p.n_tokens : 0);

  const int nks = max(p.inter, p.has_shared ? p.shared_inter : 0) / 128;
  // staging of one group of 8 reduction indices of one slot of a chunk
  auto group_at = [&](int gi, int& s, int& slot, int& q8) {
    q8 = gi & 15;
    const int rest = gi >> 4;
    slot = rest % n_slots;
    s = rest / n_slots;
  };
  constexpr int kPre = 4;  // h groups per thread requested ahead
  u32x4 ph[kPre], pl[kPre];
  // every staged row lies inside the workspace (slot < n_slots, index <
  // h_stride); rows of slots that no token owns are staged but never read
  auto prefetch_h = [&](int ks0, int groups) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      int s, slot, q8;
      group_at(min(tid + i * kSmallThreads, groups - 1), s, slot, q8);
      const int64_t o = (int64_t)slot * p.h_stride + (ks0 + s) * 128 + q8 * 8;
      ph[i] = load16(p.h_hi + o);
      pl[i] = load16(p.h_lo + o);
    }
  };
  // the first chunk's h and the routing inputs in one round trip, before
  // the weight traffic of the whole chip starts
  prefetch_h(0, min(spc, nks) * n_slots * 16);
  const int fi = min(tid, nk - 1);
  const int my_slot = p.inv_perm[fi];
  const float my_w = p.topk_w[fi];
  // lazy skip: slots whose gate stayed below the threshold are left out, and
  // an expert none of whose slots passes is not active (its down rows are
  // never read)
  const bool lazy = p.lazy_tau > 0.0f;
  const bool my_live =
      my_slot >= 0 && (!lazy || __uint_as_float(p.gmax[my_slot]) >= p.lazy_tau);
  if (wave == 0) {
    const int nch = uniform((p.n_experts + kWave - 1) / kWave);
    int cnt[kMaxChunks], off[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      cnt[c] = 0;
      off[c] = 0;
      if (c < nch) {
        const int x = min(c * kWave + lane, p.n_experts - 1);
        cnt[c] = p.counts[x];
        off[c] = p.offsets[x];
      }
    }
    int nact = 0;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      bool on = c < nch && c * kWave + lane < p.n_experts && cnt[c] > 0;
      if (lazy && on) {
        bool any = false;
        for (int j = 0; j < cnt[c]; ++j)
          any = any || __uint_as_float(p.gmax[off[c] + j]) >= p.lazy_tau;
        on = any;
      }
      const uint64_t m = __ballot(on);
      if (on) {
        const int a = nact + __popcll(m & ((1ull << lane) - 1ull));
        s_act[a] = c * kWave + lane;
        s_off[a] = off[c];
      }
      nact += __popcll(m);
    }
    if (lane == 0) {
      s_nroute = nact;
      if (p.has_shared) {
        s_act[nact] = p.n_experts;
        s_off[nact] = nk;
      }
      s_nact = nact + (p.has_shared ? 1 : 0);
    }
  }
  for (int i = tid; i < kSmallMaxActive * kSmallMaxTokens; i += kSmallThreads)
    (&s_col[0][0])[i] = -1;
  for (int i = tid; i < kSmallMaxSlots; i += kSmallThreads) s_w[i] = 0.0f;
  if (tid < kStageRow * 2 / 16) {
    char* z = smem + (size_t)2 * spc * n_slots * kStageRow * 2;
    *reinterpret_cast<u32x4*>(z + tid * 16) = u32x4{0, 0, 0, 0};
  }
  __syncthreads();
  const int A = s_nact, AR = s_nroute;
  if (tid < nk && my_live) {
    int lo = 0, hi = AR;  // active expert owning the slot
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= my_slot)
        lo = mid;
      else
        hi = mid;
    }
    s_col[lo][tid / p.top_k] = (int16_t)my_slot;
    s_w[my_slot] = my_w;
  }
  for (int q = nk + tid; q < n_slots; q += kSmallThreads) {
    s_col[A - 1][q - nk] = (int16_t)q;
    s_w[q] = 1.0f;
  }
  __syncthreads();

  __bf16* s_bh = reinterpret_cast<__bf16*>(smem);
  __bf16* s_bl = s_bh + (size_t)spc * n_slots * kStageRow;
  const __bf16* s_z = s_bl + (size_t)spc * n_slots * kStageRow;  // zero row
  f32x4 acc_h = f32x4{0, 0, 0, 0}, acc_l = f32x4{0, 0, 0, 0};

  // units u = s * A + a of a chunk are dealt round-robin to the wavefronts,
  // kSmallBatch at a time: the codes of a whole batch are requested before
  // any of them is decoded
  constexpr int kSmallBatch = 2 * Fmt<WT>::CH;  // 16 MXFP4 or 8 fp8 units
  u32x4 q[kSmallBatch][Fmt<WT>::Q];
  uint32_t su[kSmallBatch];
  int ua[kSmallBatch], us[kSmallBatch], uslot[kSmallBatch];
  // a unit that does not exist (past the end, a step beyond the expert's
  // width, the shared expert when its format differs) loads routed expert
  // 0's first step, which always exists, and is skipped by compute_batch;
  // the loads of a batch stay one burst
  const int Ad = max(A, 1);  // A == 0 only with no units at all
  const int64_t cb_r = Fmt<WT>::row_bytes(p.inter), sb_r = Fmt<WT>::scale_row_bytes(p.inter);
  const int64_t cb_s = Fmt<WT>::row_bytes(p.shared_inter);
  const int64_t sb_s = Fmt<WT>::scale_row_bytes(p.shared_inter);
  // byte offsets from down_c / down_s: one routed expert, this row block of
  // routed expert 0, this row block of the shared matrix
  const uint64_t estride_c = (uint64_t)(p.hidden * cb_r), estride_s = (uint64_t)(p.hidden * sb_r);
  const uint64_t cbase_r = (uint64_t)(row0 * cb_r), sbase_r = (uint64_t)(row0 * sb_r);
  const uint64_t cbase_s = (uint64_t)p.sdown_c - (uint64_t)p.down_c + (uint64_t)(row0 * cb_s);
  const uint64_t sbase_s = (uint64_t)p.sdown_s - (uint64_t)p.down_s + (uint64_t)(row0 * sb_s);
  const int kmax_r = p.inter / 128, kmax_s = kMerged ? p.shared_inter / 128 : 0;
  const int64_t lane_cr = r16 * cb_r + Fmt<WT>::code_off(0, g);
  const int64_t lane_cs = r16 * cb_s + Fmt<WT>::code_off(0, g);
  const int64_t lane_sr = r16 * sb_r + Fmt<WT>::scale_off(0, g);
  const int64_t lane_ss = r16 * sb_s + Fmt<WT>::scale_off(0, g);
  auto load_batch = [&](int ks0, int units, int u0) {
    // pass 1: the LDS lookups of every unit of the batch (expert, slot of
    // the lane's token), stepping (s, a) along u = u0 + 8b without divisions
    int be[kSmallBatch], bslot[kSmallBatch], ba[kSmallBatch];
    int s = uniform(u0 / Ad), a = uniform(u0 - s * Ad);
#pragma unroll
    for (int b = 0; b < kSmallBatch; ++b) {
      const bool in = u0 + b * kSmallWaves < units;
      ba[b] = a;
      us[b] = s;
      be[b] = s_act[in ? a : 0];
      bslot[b] = s_col[in ? a : 0][r16];
      a += kSmallWaves;
      while (a >= Ad) {
        a -= Ad;
        ++s;
      }
    }
    // pass 2: one burst of code and scale loads.  An address is a wave-
    // uniform part (matrix, expert, row block, step) plus the lane's part
    // (row r16, quarter g); the shared matrix is reached by adding the
    // distance between the two allocations, so no pointer is reloaded
#pragma unroll
    for (int b = 0; b < kSmallBatch; ++b) {
      const int e = uniform(be[b]);
      const int sh = e == p.n_experts;
      const int ks = ks0 + us[b];
      const int real = (u0 + b * kSmallWaves < units) & (ks < (sh ? kmax_s : kmax_r));
      const int use_sh = real & sh;
      const uint32_t e_eff = (real & !sh) ? (uint32_t)e : 0u;
      const uint32_t ks_eff = real ? (uint32_t)ks : 0u;
      const uint64_t cu = (uint64_t)e_eff * estride_c + (use_sh ? cbase_s : cbase_r) +
                          (uint64_t)(ks_eff * (uint32_t)Fmt<WT>::code_off(1, 0));
      const uint64_t su_ = (uint64_t)e_eff * estride_s + (use_sh ? sbase_s : sbase_r) +
                           (uint64_t)(ks_eff * (uint32_t)Fmt<WT>::scale_off(1, 0));
      const uint8_t* c = p.down_c + cu + (use_sh ? lane_cs : lane_cr);
      const uint8_t* sc = p.down_s + su_ + (use_sh ? lane_ss : lane_sr);
#pragma unroll
      for (int i = 0; i < Fmt<WT>::Q; ++i) q[b][i] = load16(c + 16 * i);
      su[b] = *sc;
      ua[b] = real ? ba[b] : -1;
      uslot[b] = real ? bslot[b] : -1;
    }
  };
  // B fragments of unit b: the staged w*h of the lane's token, or the zero
  // row when the token did not pick the unit's expert.  Lanes of absent
  // tokens (r16 >= n_tokens) read nothing and keep the zeros set once per
  // batch, so no fragment is cleared per unit.
  auto read_b = [&](int b, u32x4 (&bh)[4], u32x4 (&bl)[4]) {
    if (r16 < p.n_tokens) {
      const int slot = uslot[b];
      const size_t o = ((size_t)us[b] * n_slots + slot) * kStageRow + g * 32;
      const __bf16* srch = slot >= 0 ? s_bh + o : s_z + g * 32;
      const __bf16* srcl = slot >= 0 ? s_bl + o : s_z + g * 32;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bh[j] = *reinterpret_cast<const u32x4*>(srch + 8 * j);
        bl[j] = *reinterpret_cast<const u32x4*>(srcl + 8 * j);
      }
    }
  };
  auto compute_batch = [&]() {
    u32x4 bh[2][4], bl[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) bh[i][j] = bl[i][j] = u32x4{0, 0, 0, 0};
    read_b(0, bh[0], bl[0]);
#pragma unroll
    for (int b = 0; b < kSmallBatch; ++b) {
      if (b + 1 < kSmallBatch) read_b(b + 1, bh[(b + 1) & 1], bl[(b + 1) & 1]);
      if (ua[b] < 0) continue;  // uniform over the wavefront
      bf16x8 a[4];
      Fmt<WT>::decode(q[b], su[b], a);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc_h = mfma_bf16(a[j], as_bf16x8(bh[b & 1][j]), acc_h);
        acc_l = mfma_bf16(a[j], as_bf16x8(bl[b & 1][j]), acc_l);
      }
    }
  };
  // staging: w * (h_hi + h_lo), split again into hi + lo
  auto stage = [&](int s, int slot, int q8, u32x4 rh, u32x4 rl) {
    const bf16x8 hi = as_bf16x8(rh), lo = as_bf16x8(rl);
    const float wt = s_w[slot];
    bf16x8 oh, ol;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = wt * (static_cast<float>(hi[j]) + static_cast<float>(lo[j]));
      __bf16 x, y;
      split_bf16(v, x, y);
      oh[j] = x;
      ol[j] = y;
    }
    const size_t o = ((size_t)s * n_slots + slot) * kStageRow + q8 * 8;
    *reinterpret_cast<u32x4*>(s_bh + o) = __builtin_bit_cast(u32x4, oh);
    *reinterpret_cast<u32x4*>(s_bl + o) = __builtin_bit_cast(u32x4, ol);
  };
  for (int ks0 = 0; ks0 < nks; ks0 += spc) {
    const int steps = min(spc, nks - ks0);
    const int units = steps * A;
    const int groups = steps * n_slots * 16;
    if (ks0 > 0) prefetch_h(ks0, groups);
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int gi = tid + i * kSmallThreads;
      if (gi < groups) {
        int s, slot, q8;
        group_at(gi, s, slot, q8);
        stage(s, slot, q8, ph[i], pl[i]);
      }
    }
    for (int gi = tid + kPre * kSmallThreads; gi < groups; gi += kSmallThreads) {
      int s, slot, q8;
      group_at(gi, s, slot, q8);
      const int64_t o = (int64_t)slot * p.h_stride + (ks0 + s) * 128 + q8 * 8;
      stage(s, slot, q8, load16(p.h_hi + o), load16(p.h_lo + o));
    }
    __syncthreads();
    load_batch(ks0, units, wave);
    compute_batch();
    for (int u0 = wave + kSmallWaves * kSmallBatch; u0 < units;
         u0 += kSmallWaves * kSmallBatch) {
      load_batch(ks0, units, u0);
      compute_batch();
    }
    // the shared expert in another format: its own loop
    if (!kMerged && p.has_shared) {
      const int a = A - 1;
      for (int s = wave; s < steps; s += kSmallWaves) {
        const int ks = ks0 + s;
        if (ks * 128 >= p.shared_inter) continue;
        const int64_t cb = Fmt<SWT>::row_bytes(p.shared_inter);
        const int64_t sb = Fmt<SWT>::scale_row_bytes(p.shared_inter);
        const int64_t row = row0 + r16;
        u32x4 qs[Fmt<SWT>::Q];
        uint32_t ss;
        load_codes<SWT>(p.sdown_c + row * cb, p.sdown_s + row * sb, ks, g, qs, ss);
        bf16x8 w4[4];
        Fmt<SWT>::decode(qs, ss, w4);
        const int slot = s_col[a][r16];
        const size_t o = ((size_t)s * n_slots + (slot >= 0 ? slot : 0)) * kStageRow + g * 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 z = u32x4{0, 0, 0, 0};
          const bf16x8 bh =
              as_bf16x8(slot >= 0 ? *reinterpret_cast<const u32x4*>(s_bh + o + 8 * j) : z);
          const bf16x8 bl =
              as_bf16x8(slot >= 0 ? *reinterpret_cast<const u32x4*>(s_bl + o + 8 * j) : z);
          acc_h = mfma_bf16(w4[j], bh, acc_h);
          acc_l = mfma_bf16(w4[j], bl, acc_l);
        }
      }
    }
    __syncthreads();
  }

  // the eight partial sums, added in wavefront order
  f32x4 acc = acc_h + acc_l;
  if (wave > 0) s_red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kSmallWaves - 1; ++w) acc += s_red[w][lane];
    if (r16 < p.n_tokens)
      *reinterpret_cast<f32x4*>(p.y + (int64_t)r16 * p.hidden + row0 + 4 * g) = acc;
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

// hipExtLaunchKernel with its status returned; start/stop (may be null)
// record the kernel's own start and end.
template <typename... Params, typename... Args>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds,
                  hipStream_t stream, hipEvent_t start, hipEvent_t stop, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
  void* argv[] = {const_cast<void*>(static_cast<const void*>(&args))...};
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                                          argv, lds, stream, start, stop, 0);
  return e != hipSuccess ? e : hipGetLastError();
}

// Kernels that ask for more than 64 KiB of dynamic LDS say so once.
template <typename K>
hipError_t allow_lds(K kernel) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
}

// fp32 activations: bf16 ones take the grouped GEMM or the decode kernel,
// so only the XF32 instantiations are launched.
template <int NBT>
hipError_t gate_up_launch(const FfnParams& p, dim3 grid, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
  if constexpr (NBT == 1) {
    // a one-block tile's activation rows fit in LDS: stage them once per item
    const int x_stride = p.hidden * 4 + 16;
    const int rows = p.n_tokens < 16 ? p.n_tokens : 16;
    const size_t lds = (size_t)rows * x_stride;
    if (lds <= (size_t)kLdsBudget) {
      static const hipError_t attr = allow_lds(gate_up_kernel<1, true, true>);
      if (attr != hipSuccess) return attr;
      return launch(gate_up_kernel<1, true, true>, grid, dim3(kThreads), lds, stream, start,
                    stop, p, x_stride);
    }
  }
  return launch(gate_up_kernel<NBT, true, false>, grid, dim3(kThreads), 0, stream, start, stop,
                p, 0);
}

template <int NBT>
hipError_t gate_up_nbt(const FfnParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  constexpr int TN = 16 * NBT;
  const int64_t shared_tiles = p.has_shared ? (p.n_tokens + TN - 1) / TN : 0;
  const int64_t items = routed_tiles_bound(p, TN) * (p.inter / 16) +
                        shared_tiles * (p.shared_inter / 16);
  return gate_up_launch<NBT>(p, dim3(grid_for(items)), stream, start, stop);
}

// Slots of a small batch; 0 when the batch takes the per-slot path.
int small_slots(const FfnParams& p) {
  const int slots = p.n_tokens * p.top_k + (p.has_shared ? p.n_tokens : 0);
  if (p.n_tokens > kSmallMaxTokens || slots > kSmallMaxSlots) return 0;
  return slots;
}

template <int WT, int SWT>
hipError_t down_small_launch(const FfnParams& p, int slots, hipStream_t stream, hipEvent_t start,
                             hipEvent_t stop) {
  const int nks = (p.inter > p.shared_inter ? p.inter : p.shared_inter) / 128;
  const int per_step = slots * kStageRow * 2 * 2;  // hi + lo bf16
  const int zero_row = kStageRow * 2;
  int spc = (kLdsBudget - zero_row) / per_step;
  spc = spc < 1 ? 1 : (spc > nks ? nks : spc);
  static const hipError_t attr = allow_lds(down_combine_small_kernel<WT, SWT>);
  if (attr != hipSuccess) return attr;
  return launch(down_combine_small_kernel<WT, SWT>, dim3(p.hidden / 16), dim3(kSmallThreads),
                (size_t)spc * per_step + zero_row, stream, start, stop, p, spc);
}

template <int S>
hipError_t gate_up_decode_launch(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                                 hipEvent_t stop) {
  const int64_t nk = (int64_t)p.n_tokens * p.top_k;
  const int a_bound = (int)(nk < p.n_experts ? nk : p.n_experts);
  const int routed = a_bound * (p.inter / 16);
  const int blocks = routed + (p.has_shared ? p.shared_inter / 16 : 0);
  // every tile holds at most min(N, 16) tokens
  const int m_max = p.n_tokens < kDecodeMaxTokens ? p.n_tokens : kDecodeMaxTokens;
  const size_t lds = (size_t)kWaves * m_max * (S * 128 + 8) * 2;
  if (p.lazy_tau == 0.0f) {
    static const hipError_t attr = allow_lds(gate_up_decode_kernel<S, 0>);
    if (attr != hipSuccess) return attr;
    return launch(gate_up_decode_kernel<S, 0>, dim3(blocks), dim3(kThreads), lds, stream, start,
                  stop, p, a_bound, m_max);
  }
  // gate first: the routed gate rows, then the up rows of the experts some
  // token keeps, and the shared expert
  static const hipError_t attr1 = allow_lds(gate_up_decode_kernel<S, 1>);
  static const hipError_t attr2 = allow_lds(gate_up_decode_kernel<S, 2>);
  if (attr1 != hipSuccess) return attr1;
  if (attr2 != hipSuccess) return attr2;
  hipError_t e = launch(gate_up_decode_kernel<S, 1>, dim3(routed > 0 ? routed : 1),
                        dim3(kThreads), lds, stream, start, nullptr, p, a_bound, m_max);
  if (e != hipSuccess) return e;
  return launch(gate_up_decode_kernel<S, 2>, dim3(blocks), dim3(kThreads), lds, stream, nullptr,
                stop, p, a_bound, m_max);
}

// Zeroes n 32-bit words (the lazy skip's per-slot gate maxima).
__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) v[i] = 0u;
}

// The decode kernel covers small batches of bf16 activations with MXFP4
// gate/up matrices and hidden = 512, 1024, 2048 or 4096; 0 when it does not.
int decode_steps(const FfnParams& p) {
  if (p.n_tokens > kDecodeMaxTokens || p.x_f32 || p.w_type != MOE_W_MXFP4) return 0;
  if (p.has_shared && p.sw_type != MOE_W_MXFP4) return 0;
  const int s = p.hidden / 512;
  if (p.hidden % 512 != 0 || (s != 1 && s != 2 && s != 4 && s != 8)) return 0;
  return s;
}

}  // namespace

bool gate_up_writes_h3(const FfnParams& p) { return !p.x_f32 && decode_steps(p) == 0; }

hipError_t launch_ffn_gate_up(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                              hipEvent_t stop) {
  if (p.lazy_tau > 0.0f) {
    const int64_t nk = (int64_t)p.n_tokens * p.top_k;
    const hipError_t e = launch(zero_u32_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0,
                                stream, nullptr, nullptr, p.gmax, nk);
    if (e != hipSuccess) return e;
  }
  switch (decode_steps(p)) {
    case 1: return gate_up_decode_launch<1>(p, stream, start, stop);
    case 2: return gate_up_decode_launch<2>(p, stream, start, stop);
    case 4: return gate_up_decode_launch<4>(p, stream, start, stop);
    case 8: return gate_up_decode_launch<8>(p, stream, start, stop);
    default: break;
  }
  if (!p.x_f32) return launch_gemm_gate_up(p, stream, start, stop);
  switch (pick_nbt(p.n_tokens)) {
    case 1: return gate_up_nbt<1>(p, stream, start, stop);
    case 2: return gate_up_nbt<2>(p, stream, start, stop);
    case 3: return gate_up_nbt<3>(p, stream, start, stop);
    default: return gate_up_nbt<4>(p, stream, start, stop);
  }
}

template <bool UNIFORM>
hipError_t combine_launch(const FfnParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.n_tokens * (p.hidden / 4);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  switch (p.top_k) {
    case 1: return launch(combine_kernel<UNIFORM, 1>, grid, block, 0, stream, nullptr, nullptr, p);
    case 2: return launch(combine_kernel<UNIFORM, 2>, grid, block, 0, stream, nullptr, nullptr, p);
    case 3: return launch(combine_kernel<UNIFORM, 3>, grid, block, 0, stream, nullptr, nullptr, p);
    case 4: return launch(combine_kernel<UNIFORM, 4>, grid, block, 0, stream, nullptr, nullptr, p);
    case 5: return launch(combine_kernel<UNIFORM, 5>, grid, block, 0, stream, nullptr, nullptr, p);
    case 6: return launch(combine_kernel<UNIFORM, 6>, grid, block, 0, stream, nullptr, nullptr, p);
    case 7: return launch(combine_kernel<UNIFORM, 7>, grid, block, 0, stream, nullptr, nullptr, p);
    default: return launch(combine_kernel<UNIFORM, 8>, grid, block, 0, stream, nullptr, nullptr, p);
  }
}

hipError_t launch_ffn_down(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
  // the small-batch down reads the bf16 pair; h in E4M3 parts goes to the
  // grouped-GEMM down whatever the batch size
  const int slots = gate_up_writes_h3(p) ? 0 : small_slots(p);
  if (slots > 0) {
    const bool r4 = p.w_type == MOE_W_MXFP4;
    const bool s4 = !p.has_shared || p.sw_type == MOE_W_MXFP4;
    if (r4 && s4) return down_small_launch<MOE_W_MXFP4, MOE_W_MXFP4>(p, slots, stream, start, stop);
    if (r4) return down_small_launch<MOE_W_MXFP4, MOE_W_FP8E4M3_B128>(p, slots, stream, start, stop);
    if (s4) return down_small_launch<MOE_W_FP8E4M3_B128, MOE_W_MXFP4>(p, slots, stream, start, stop);
    return down_small_launch<MOE_W_FP8E4M3_B128, MOE_W_FP8E4M3_B128>(p, slots, stream, start,
                                                                      stop);
  }
  // weighted per-slot outputs, then each token's sum in a fixed order
  hipError_t e = launch_gemm_down(p, stream, start, stop);
  if (e != hipSuccess) return e;
  return p.hidden % 256 == 0 ? combine_launch<true>(p, stream) : combine_launch<false>(p, stream);
}

}  // namespace moe

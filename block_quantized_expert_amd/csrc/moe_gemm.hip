// Expert FFN for batches in which experts see many tokens (prefill): grouped
// matrix products on the matrix cores with the weights decoded in registers.
//
// "DeepSeek-V4-Flash 284B -- Deep-Dive Mathematical & Kernel Guide":
//   section 4, SwiGLU equation h = SiLU(W_gate x) * (W_up x), y = W_down h;
//   section 3.2, combine equation y = e_shared(x) + sum_i w_i e_{k_i}(x);
//   section 2 (table B, prefill): MUL_MAT_ID batches the tokens of each
//   expert so that its weights stream once per batch.
// "DeepSeek V4 target engine (CPU + optional CUDA tier)", introduction and
//   GPU coverage: routed experts in MXFP4, dense weights fp8-e4m3 + UE8M0;
//   expert-grouped GEMM on the GPU.
//
// A work item is (segment, row tile, token tile of up to TT slots).  A
// segment is a routed expert (slots offsets[e] .. offsets[e+1]) or the shared
// expert (slot N*k + t is token t).  Items of one row tile are consecutive, so
// the workgroups that multiply the same weights with different token tiles
// run at the same time and share them through the caches.  The grid is
// persistent; every workgroup rebuilds the item prefix from the device-side
// counts (no host synchronisation).
//
// Inside an item each wavefront owns whole output rows over the full
// reduction: no partial sums cross wavefronts.  The reduction runs in steps
// of 128.  The token operand of a step (quantized activation rows gathered
// through perm, or the h rows of the slots) is staged in LDS, double
// buffered; the weight codes of step ks+1 and its token operand are in
// flight while step ks multiplies.
//
// Gate/up (bf16 x): quant_x_kernel first writes x as two E4M3 parts with
// UE8M0 block scales that reproduce the bf16 value.  The weights enter the
// scaled 16x16x128 instruction as stored (E2M1 or E4M3 codes with their
// UE8M0 bytes), so nothing is decoded in registers: two instructions per
// tile and step, one per part.  A workgroup owns 128 intermediate rows and
// up to 112 (MXFP4) or 64 (fp8) tokens; wavefront w owns rows 32w .. 32w+31
// of the gate and of the up matrix (four 16-row blocks), so one token
// fragment read from LDS feeds four instructions and one weight fragment
// feeds up to seven token blocks.  The epilogue applies SwiGLU and writes h
// as three E4M3 parts with their scale bytes (split_e4m3x3).
//
// Down: a workgroup owns 256 hidden rows and up to 64 tokens; wavefront w
// owns rows 64w .. 64w+63 (four blocks).  gemm_down3_kernel multiplies the
// stored weight codes with the three E4M3 parts of h on the scaled
// instruction; gemm_down_kernel serves h as a bf16 hi/lo pair (written by
// the gate/up of fp32 x and by the small-batch decode gate/up): it decodes
// the weights to bf16 and multiplies them with h_hi and h_lo.  Both
// epilogues scale each token column by its routing weight (1 for the
// shared expert) and write the per-slot output; a separate pass sums the
// slots of every token in a fixed order.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_formats.h"
#include "moe_kernels.h"

namespace moe {
namespace {

// Two workgroups of four wavefronts per CU (two wavefronts per SIMD, 256
// registers each).  One workgroup of eight (kGWaves = 8: a token tile staged
// once per CU for 256 gate/up or 512 down rows) measured no faster on the
// 4096-token batch and 5-13 % slower on 32 and 512 tokens: a CU then has no
// second workgroup whose steps cover an item's prologue and epilogue.
constexpr int kGWaves = 4;
constexpr int kGPerCU = 8 / kGWaves;  // workgroups per CU
constexpr int kGThreads = kGWaves * kWave;
constexpr int kGuRows = 32 * kGWaves;  // intermediate rows per gate/up item
constexpr int kDnRows = 64 * kGWaves;  // hidden rows per down item
constexpr int kSegMax = MOE_MAX_EXPERTS + 1;
// dynamic LDS of either kernel; with the static item prefix (4 KiB) the
// workgroups of a CU must fit its 160 KiB
constexpr int kGemmLds = kGWaves == 8 ? 106 * 1024 : 74 * 1024;
// scale blocks in LDS: after two token tiles of up to five blocks (gate/up,
// kGuRows rows x H/32 bytes per matrix, H <= 4096) or two h_hi/h_lo pairs
// of up to three blocks (down, kDnRows rows x I/32 bytes, I <= 2048)
constexpr int kGuScaleOff = 2 * 16 * 5 * 256;
constexpr int kDnScaleOff = 2 * 2 * 16 * 3 * 256;
// gate/up: the scale bytes of two token tiles (8 per row and step, up to 128
// rows), after the weight scales and after two full token tiles
constexpr int kTokScaleBytes = 128 * 8;
constexpr int kTokScaleOff = kGuScaleOff + 2 * kGuRows * (4096 / 32);
static_assert(kTokScaleOff >= 2 * 128 * 256, "gate/up token tiles");
static_assert(kTokScaleOff + 2 * kTokScaleBytes <= kGemmLds, "gate/up LDS");
// gate/up with scale chunks (no LDS weight scales): the token scale bytes of
// four steps (32 per row, up to 128 rows), two of them, after the largest
// token tiles (112 rows x 2 buffers)
constexpr int kTokChunkOff = 2 * 112 * 256;
static_assert(kTokChunkOff + 2 * 128 * 32 <= kGemmLds, "gate/up LDS");
// gate/up epilogue for E2M3 parts: each wavefront's h values staged as
// [112 tokens][36 floats] (32 rows, the stride padded so that a row of 16
// tokens falls on distinct banks)
constexpr int kH6Row = 36;
constexpr int kH6Wave = 112 * kH6Row * 4;
static_assert(kGWaves * kH6Wave <= kGemmLds, "gate/up LDS");
// dynamic LDS + the static item prefix and scan words of a workgroup (plus
// alignment): kGPerCU workgroups in the 160 KiB of a CU
static_assert(kGemmLds + (kSegMax + 1 + kGWaves) * 4 + 64 <= 160 * 1024 / kGPerCU,
              "workgroups per CU");
static_assert(kDnScaleOff + kDnRows * (2048 / 32) <= kGemmLds, "down LDS");

struct GItem {
  int seg;
  int slot0;  // first slot of the token tile
  int m;      // slots in the tile
  int row0;   // first output row of the row tile
};

__device__ __forceinline__ int seg_rows(const FfnParams& p, int s, bool down) {
  return down ? p.hidden : (s == p.n_experts ? p.shared_inter : p.inter);
}

__device__ __forceinline__ int seg_count(const FfnParams& p, int s) {
  return s == p.n_experts ? p.n_tokens : p.counts[s];
}

template <int TT, int RT, bool DOWN>
__device__ __forceinline__ int seg_items(const FfnParams& p, int s) {
  const int rows = seg_rows(p, s, DOWN);
  return (seg_count(p, s) + TT - 1) / TT * ((rows + RT - 1) / RT);
}

// s_pref[s] = items of the segments before s; returns the total.
// Segments seg_lo .. seg_hi-1 take part; s_pref is indexed from seg_lo.
template <int TT, int RT, bool DOWN>
__device__ int item_prefix(const FfnParams& p, int seg_lo, int seg_hi, int* s_pref, int* s_tmp) {
  const int nseg = seg_hi - seg_lo;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (nseg + kGThreads - 1) / kGThreads;
  const int s0 = tid * per, s1 = min(s0 + per, nseg);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += seg_items<TT, RT, DOWN>(p, seg_lo + s);
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
    run += seg_items<TT, RT, DOWN>(p, seg_lo + s);
  }
  if (tid == kGThreads - 1) s_pref[nseg] = before + incl;
  __syncthreads();
  return s_pref[nseg];
}

template <int TT, int RT, bool DOWN>
__device__ __forceinline__ GItem find_item(const FfnParams& p, int seg_lo, int seg_hi,
                                           const int* s_pref, int item) {
  int lo = 0, hi = seg_hi - seg_lo;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= item)
      lo = mid;
    else
      hi = mid;
  }
  const int local = item - s_pref[lo];
  lo += seg_lo;
  const bool shared = lo == p.n_experts;
  const int m_all = seg_count(p, lo);
  const int ntt = (m_all + TT - 1) / TT;
  const int rt = local / ntt;
  const int tile = local - rt * ntt;
  const int start = shared ? p.n_tokens * p.top_k : p.offsets[lo];
  GItem it;
  it.seg = uniform(lo);
  it.slot0 = uniform(start + tile * TT);
  it.m = uniform(min(TT, m_all - tile * TT));
  it.row0 = uniform(rt * RT);
  return it;
}

// Token-operand staging: a tile of TT rows x 256 bytes per reduction step
// (128 bf16, or the 128 hi and 128 lo E4M3 bytes of 128 inputs), copied
// straight from global memory into LDS (no register round trip).  One wavefront copy instruction fills four rows: lane l lands
// at byte 16 l of the block.  In round i wavefront w fills rows
// R i + 4w .. +3 (R = 4 * wavefronts), lane l row R i + 4w + (l >> 4),
// 16-byte position l & 15.  Positions are swizzled, chunk c of row n sits at
// position c ^ (n & 15), so the sixteen rows that one fragment read touches
// hit sixteen different bank groups; each lane therefore fetches the chunk
// that belongs at its position.  Only rows below 16 * nbt are copied; rows
// past the tile repeat a valid row: they only feed token columns that the
// epilogue drops.
template <int TT, bool O32 = false>
struct Stage {
  static constexpr int kRound = 4 * kGWaves;             // rows per round
  static constexpr int kPer = (TT + kRound - 1) / kRound;  // copy rounds
  int row[kPer];                                          // source row per round
  int chunk;                                              // source chunk of this lane

  __device__ static int row_of(int i, int wave, int lane) {
    return kRound * i + 4 * wave + (lane >> 4);
  }
  __device__ void init(int lane) { chunk = (lane & 15) ^ ((4 * wave_id() + (lane >> 4)) & 15); }
  // rows of `stride` bytes, 256 bytes per step; O32: every offset into the
  // buffer is below 2^31 (one address register per row instead of two)
  __device__ void copy(const void* base, int64_t stride, int ks, char* buf, int nbt) const {
    const int64_t c = ks * 256 + chunk * 16;
    const int w = wave_id();
    char* dst = buf + (4 * w) * 256;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (kRound * i + 4 * w < 16 * nbt)
        __builtin_amdgcn_global_load_lds(
            static_cast<const char*>(base) +
                (O32 ? (int64_t)(uint32_t)(row[i] * (uint32_t)stride + (uint32_t)c)
                     : (int64_t)row[i] * stride + c),
            (__attribute__((address_space(3))) void*)(dst + i * kRound * 256), 16, 0, 0);
  }
};

// Token fragment of token block tb, sub-step j: row n = 16 tb + r16, chunk
// 4g + j, at its swizzled position.
__device__ __forceinline__ bf16x8 token_frag(const char* buf, int tb, int j, int g, int r16) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + (tb * 16 + r16) * 256 +
                                                     (((4 * g + j) ^ r16) << 4)));
}

// Wait until at most n vector memory operations of this wavefront are
// outstanding (n < 64: vmcnt bits 3:0 and 15:14), leaving the other
// counters alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// End of a reduction step: this wavefront's copies into LDS have landed
// (at most N later loads, the weights of a later step, still in flight) and
// its LDS reads of the step are complete (lgkmcnt 0), then the workgroup
// barrier; after it the next copies may overwrite the step's buffer.  The
// compiler may place the barrier above the step's MFMAs (they touch no
// memory), so the read wait cannot be left to their operand waits.  A plain
// barrier, not __syncthreads(): its release fence would also wait for the
// later weight loads.
template <int N>
__device__ __forceinline__ void step_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
  __builtin_amdgcn_s_barrier();
}

// Item schedule of one launch.  Workgroups are dealt to the eight XCDs
// round-robin (workgroup b runs on XCD b % 8), and each XCD has its own L2.
// The item order is cut into eight contiguous chunks, one per XCD: the row
// tiles of one expert (which share its token rows) and the token tiles of
// one row tile (which share its weights) then meet in the same L2.
//  - static: workgroup b takes items b / 8, b / 8 + grid / 8, ... of chunk
//    b % 8;
//  - dynamic: each chunk has a counter in the workspace; a workgroup takes
//    tickets from its own XCD's counter while that chunk lasts, then from
//    the other chunks in turn, so workgroups that run out of their own items
//    take over the rest instead of idling.  Every workgroup takes exactly one
//    ticket past the end of every chunk, so the holder of the last one
//    (chunk items + grid - 1) resets that counter to 0 for the next launch;
//    the gate/up pass of each call also zeroes them (a fresh workspace).
//    The next ticket is asked for once the current item's reduction is
//    done, so the atomic's latency hides under its epilogue.
// Tickets on one counter serialise (about 0.1 us each), so the dynamic
// schedule pays only for long items of uneven length: on a hash-routed
// batch of 4096 tokens (about 96 per expert) it took the routed gate/up
// from 873 to 829 us and the down from 775 to 640 us (a static schedule
// left the busiest workgroup 1.14 and 1.25 times the mean work); on 32 and
// 512 tokens (one-token items by the thousand) it was 10-20 % slower.
struct ItemQueue {
  uint32_t* ctr;  // [8]
  int total;
  bool dynamic;
};

// Schedule state kept in LDS by thread 0 between items, so that none of it
// is held in registers across an item.
struct QueueLds {
  int item;    // the workgroup's next item, -1 when it has none left
  int chunks;  // dynamic: chunks exhausted so far, the current one is
               // (blockIdx.x + chunks) & 7; static: the workgroup's index
               // into the dealt order
};

// Thread 0, dynamic schedule: turns ticket tk of the current chunk into the
// next item, moving on to the following chunks (one more ticket each) while
// the ticket is past the end of its chunk; the last ticket past a chunk's
// end resets its counter.
__device__ __noinline__ void queue_advance(const ItemQueue& qu, QueueLds* s, int tk) {
  const int per = (qu.total + 7) >> 3;
  int c = s->chunks;
  for (;;) {
    const int q = (blockIdx.x + c) & 7;
    const int nq = max(0, min(per, qu.total - q * per));
    if (tk < nq) {
      s->item = q * per + tk;
      break;
    }
    if (tk == nq + (int)gridDim.x - 1) atomicExch(qu.ctr + q, 0u);
    if (++c == 8) {
      s->item = -1;
      break;
    }
    tk = (int)atomicAdd(qu.ctr + ((blockIdx.x + c) & 7), 1u);
  }
  s->chunks = c;
}

// Thread 0, static schedule: the next item of the dealt order from index i
// (i, i + grid, ...: chunk i % 8, position i / 8), skipping the padding of
// short chunks.
__device__ __forceinline__ void static_advance(const ItemQueue& qu, QueueLds* s, int i) {
  const int per = (qu.total + 7) >> 3;
  for (; i < 8 * per; i += gridDim.x) {
    const int item = (i & 7) * per + (i >> 3);
    if (item < qu.total) {
      s->item = item;
      s->chunks = i;
      return;
    }
  }
  s->item = -1;
}

// body(item, take): take() asks for the next ticket (dynamic: thread 0;
// called once per item, after its reduction, so the atomic overlaps the
// epilogue; static: nothing).
template <typename Body>
__device__ __forceinline__ void run_queue(const ItemQueue& qu, QueueLds* s, Body&& body) {
  if (threadIdx.x == 0) {
    if (qu.dynamic) {
      s->chunks = 0;
      queue_advance(qu, s, (int)atomicAdd(qu.ctr + (blockIdx.x & 7), 1u));
    } else {
      static_advance(qu, s, blockIdx.x);
    }
  }
  __syncthreads();
  for (int item = s->item; item >= 0; item = s->item) {
    int tk = 0;
    body(item, [&]() {
      if (qu.dynamic && threadIdx.x == 0)
        tk = (int)atomicAdd(qu.ctr + ((blockIdx.x + s->chunks) & 7), 1u);
    });
    __syncthreads();  // every thread has read s->item; the LDS tiles are free
    if (threadIdx.x == 0) {
      if (qu.dynamic)
        queue_advance(qu, s, tk);
      else
        static_advance(qu, s, s->chunks + gridDim.x);
    }
    __syncthreads();
  }
}

// Calls f(std::integral_constant<int, n>) for the runtime n in 1..MAX.
template <int N>
struct IntC {
  static constexpr int value = N;
};
template <int MAX, typename Fn>
__device__ __forceinline__ void dispatch_nbt(int n, Fn&& f) {
  if constexpr (MAX >= 1) {
    if (n == MAX) {
      f(IntC<MAX>{});
      return;
    }
    dispatch_nbt<MAX - 1>(n, f);
  }
}

// Calls f(IntC<k>) for k = K0 .. K1-1 in order, as straight-line code.
template <int K0, int K1, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (K0 < K1) {
    f(IntC<K0>{});
    static_for<K0 + 1, K1>(f);
  }
}

// ------------------------------------------------------------- gate/up

// The activations enter the matrix cores as E4M3 with one UE8M0 scale per 32
// inputs, in two parts that reproduce the bf16 value exactly.  For the 32
// inputs of a block let e be the exponent of the largest magnitude; with
// f = x / 2^(e-7) (|f| < 256), hi = f rounded to E4M3 (4 significant bits)
// and lo = (f - hi) * 16, which is exact in E4M3 as well: f carries at most 8
// significant bits, its bits below hi's span at most 4 more, and
// |lo| <= 16 * |f| / 8 < 448.  Inputs below 2^-13 of the block's largest
// magnitude leave the E4M3 normal range and keep fewer bits (an absolute
// error under 2^(e-17)).  hi is scaled by 2^(e-7), lo by 2^(e-11).
//
// Layout: xq [token][hidden/128][256 bytes] = per 128 inputs the 128 hi bytes
// then the 128 lo bytes, in input order; xs [token][hidden/32][2 bytes] = the
// hi and lo scale bytes of each block.  One thread per block.
__global__ __launch_bounds__(256) void quant_x_kernel(FfnParams p) {
  // the grouped GEMMs' queue counters start this call at 0 (they reset
  // themselves at the end of each launch; this covers a fresh workspace)
  if (blockIdx.x == 0 && threadIdx.x < kQueueWords) p.qctr[threadIdx.x] = 0u;
  const int nb = p.hidden / 32;
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= (int64_t)p.n_tokens * nb) return;
  const int64_t t = blk / nb;
  const int j = (int)(blk - t * nb);
  const __bf16* src = static_cast<const __bf16*>(p.x) + t * p.hidden + 32 * j;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = load16(src + 8 * i);
  uint32_t mag = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) mag = max(mag, max(v[i][c] & 0x7FFFu, (v[i][c] >> 16) & 0x7FFFu));
  // bf16 keeps fp32's exponent field: bits 14:7 of the magnitude.  The hi
  // scale byte is that biased exponent minus 7, kept at least 4 so that the
  // lo scale byte (minus 4 more) stays a valid UE8M0 value.
  const int sb = min(max((int)(mag >> 7) - 7, 4), 254);
  const float inv = __uint_as_float((uint32_t)(254 - sb) << 23);  // 2^(127 - sb)
  uint32_t hw[8], lw[8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; c += 2) {
      // four inputs: the bf16 pairs of words c and c+1
      float f[4];
      f[0] = __uint_as_float(v[i][c] << 16) * inv;
      f[1] = __uint_as_float(v[i][c] & 0xFFFF0000u) * inv;
      f[2] = __uint_as_float(v[i][c + 1] << 16) * inv;
      f[3] = __uint_as_float(v[i][c + 1] & 0xFFFF0000u) * inv;
      int h = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      h = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], h, true);
      const auto d0 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
      const auto d1 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
      int l = __builtin_amdgcn_cvt_pk_fp8_f32((f[0] - d0[0]) * 16.0f, (f[1] - d0[1]) * 16.0f, 0,
                                              false);
      l = __builtin_amdgcn_cvt_pk_fp8_f32((f[2] - d1[0]) * 16.0f, (f[3] - d1[1]) * 16.0f, l, true);
      hw[2 * i + c / 2] = (uint32_t)h;
      lw[2 * i + c / 2] = (uint32_t)l;
    }
  uint8_t* dst = p.xq + t * 2 * (int64_t)p.hidden + (j >> 2) * 256 + (j & 3) * 32;
  *reinterpret_cast<u32x4*>(dst) = u32x4{hw[0], hw[1], hw[2], hw[3]};
  *reinterpret_cast<u32x4*>(dst + 16) = u32x4{hw[4], hw[5], hw[6], hw[7]};
  *reinterpret_cast<u32x4*>(dst + 128) = u32x4{lw[0], lw[1], lw[2], lw[3]};
  *reinterpret_cast<u32x4*>(dst + 144) = u32x4{lw[4], lw[5], lw[6], lw[7]};
  reinterpret_cast<uint16_t*>(p.xs)[blk] = (uint16_t)(sb | ((sb - 4) << 8));
}

// The weight operand of one 16x16x128 tile from the lane's code bytes: MXFP4,
// the lane's 32-input block (16 bytes); fp8, the bytes of inputs 16g .. +15
// and 64 + 16g .. +15 (q[0], q[1]).
template <int WT>
__device__ __forceinline__ i32x8 weight_operand(const u32x4 (&q)[Fmt<WT>::Q]) {
  if constexpr (WT == MOE_W_MXFP4)
    return i32x8{(int)q[0][0], (int)q[0][1], (int)q[0][2], (int)q[0][3], 0, 0, 0, 0};
  else
    return i32x8{(int)q[0][0], (int)q[0][1], (int)q[0][2], (int)q[0][3],
                 (int)q[1][0], (int)q[1][1], (int)q[1][2], (int)q[1][3]};
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// LDS-typed views (32-bit addresses) of the shared-memory tiles.
using lds_cptr = const __attribute__((address_space(3))) char*;
typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef const __attribute__((address_space(3))) uint16_t lds_u16;
typedef const __attribute__((address_space(3))) uint32_t lds_u32;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ lds_cptr to_lds(const char* p) {
  return (lds_cptr)p;  // an address-space cast: the tiles live in LDS
}

// Hides a value's origin from the optimiser (an empty register constraint,
// no instruction), so that constant offsets added to it afterwards stay
// immediates instead of being folded into hoisted per-offset registers.
template <typename T>
__device__ __forceinline__ void opaque(T& v) {
  asm volatile("" : "+v"(v));
}

__device__ __forceinline__ i32x8 join8(u32x4 a, u32x4 b) {
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2],
               (int)b[3]};
}

// Eight values v (two groups of four) of one 32-input block whose largest
// magnitude is mag, as three E4M3 parts: with e the exponent of mag and
// f = v / 2^(e-7), part 1 = f rounded to E4M3, part 2 = (f - part 1) * 16
// rounded, part 3 = (that - part 2) * 16 rounded; v = (p1 + p2/16 + p3/256)
// * 2^(e-7) up to 2^-12 of |v| (each rounding keeps 4 significant bits of a
// remainder no larger than f).  part[q][grp] packs the group's four bytes
// of part q; the return value holds the three parts' UE8M0 scale bytes
// (e-7, e-11, e-15 biased, kept at least 8, 4, 0) in bytes 0..2.
__device__ __forceinline__ uint32_t split_e4m3x3(const float (&v)[2][4], float mag,
                                                uint32_t (&part)[3][2]) {
  const int sb = min(max((int)((__float_as_uint(mag) >> 23) & 0xFF) - 7, 8), 254);
  const float inv = __uint_as_float((uint32_t)(254 - sb) << 23);  // 2^(127 - sb)
#pragma unroll
  for (int grp = 0; grp < 2; ++grp) {
    float f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = v[grp][r] * inv;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w, true);
      part[q][grp] = (uint32_t)w;
      if (q < 2) {
        const auto d0 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
        const auto d1 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
        f[0] = (f[0] - d0[0]) * 16.0f;
        f[1] = (f[1] - d0[1]) * 16.0f;
        f[2] = (f[2] - d1[0]) * 16.0f;
        f[3] = (f[3] - d1[1]) * 16.0f;
      }
    }
  }
  return (uint32_t)sb | ((uint32_t)(sb - 4) << 8) | ((uint32_t)(sb - 8) << 16);
}

// NBT = token blocks of the tile (ceil(m / 16)), a compile-time constant so
// that a step's operand reads and MFMAs form one branch-free block.
// LAZY: the gate-first lazy skip is on (its gate maxima are merged into
// gmax); a separate instantiation, so the plain kernels keep their registers.
template <int WT, int TT, int NBT, bool SC, bool O32, bool LAZY, bool PK, bool H6,
          typename Take>
__device__ __forceinline__ void gate_up_item(const FfnParams& p, const GItem& it, char* smem,
                                             int wave, int lane, Take&& take) {
  using F = Fmt<WT>;
  constexpr int Q = F::Q;
  constexpr int TB = NBT;
  constexpr int FA = WT == MOE_W_MXFP4 ? 4 : 0;  // operand format of the weights
  // Scale bytes (SC: MXFP4, H a multiple of 512 and at most 4096):
  //  - up to five token blocks: the item's scales sit in LDS (kSC, below);
  //  - six and seven: 16-byte chunks of four steps in registers (kCh,
  //    below): a byte load per row and step would add as many memory
  //    requests as the weight codes themselves;
  //  - otherwise: one byte per row and step, loaded with the step's codes.
  // fp8 (SC: H a multiple of 512): the row's one byte per step, four steps
  // in one 4-byte load (kCh).
  // PK (with SC): the packed copy, codes Q KiB per step and row block, a
  // lane's scale bytes of four steps one word (as the chunks below, without
  // the byte gathering)
  constexpr bool kPK = PK && SC;
  // H6 (packed MXFP4 batches with many tokens per expert): the down runs
  // on E2M3 parts of h (h6)
  constexpr bool kH6 = kPK && H6 && WT == MOE_W_MXFP4;
  constexpr bool kSC = SC && WT == MOE_W_MXFP4 && NBT <= 5 && !kPK;
  constexpr bool kCh = SC && (WT == MOE_W_MXFP4 ? NBT >= 6 || kPK : true);
  constexpr int kLoads = (kSC || kCh) ? 4 * Q : 4 * (Q + 1);  // vector loads of one step's weights
  const int g = lane >> 4, r16 = lane & 15;
  const bool shared = it.seg == p.n_experts;
  const int rows = shared ? p.shared_inter : p.inter;
  const int64_t cb = F::row_bytes(p.hidden), sb = F::scale_row_bytes(p.hidden);
  const int nks = p.hidden / 128;
  constexpr int nbt = NBT;
  const int nk = p.n_tokens * p.top_k;

  // the lane's rows: gate/up (mat) x two 16-row blocks (rb); row block 1
  // lies 16 rows after row block 0.  A wavefront past the matrix end (the
  // last row tile of a matrix whose rows are not a multiple of kGuRows)
  // reads row block 0 of the tile and stores nothing.
  const int wrow = it.row0 + 32 * wave;
  const bool live = wrow < rows;
  const int64_t lrow = (shared ? 0 : (int64_t)it.seg * rows) + (live ? wrow : it.row0) + r16;
  // the lane's scale bytes (its code bytes of a step: MXFP4 16 at 16g; fp8
  // 16 at 16g and 16 at 64 + 16g, addressed from the wavefront base below)
  const int64_t ls = lrow * sb + F::scale_off(0, g);
  const uint8_t* cbase[2] = {shared ? p.sgate_c : p.gate_c, shared ? p.sup_c : p.up_c};
  const uint8_t* sbase[2] = {shared ? p.sgate_s : p.gate_s, shared ? p.sup_s : p.up_s};
  // the wavefront's first row as a uniform base, the lane's rows as a 32-bit
  // offset (32 rows of at most H bytes), so a load needs one address register
  const int64_t wrow_g = (shared ? 0 : (int64_t)it.seg * rows) + (live ? wrow : it.row0);
  const uint8_t* cwave[2] = {cbase[0] + wrow_g * cb, cbase[1] + wrow_g * cb};
  const uint32_t lco = (uint32_t)(r16 * cb) + 16 * g;
  // packed: the wavefront's first row block (rows wrow_g .. +31 are blocks
  // wrow_g / 16 and the next) in both matrices
  const uint8_t* pkc[2] = {nullptr, nullptr};
  const uint8_t* pks[2] = {nullptr, nullptr};
  if constexpr (kPK) {
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
      pkc[mat] = p.pk_c[(shared ? 3 : 0) + mat] + (wrow_g / 16) * nks * 1024 * Q;
      pks[mat] = p.pk_s[(shared ? 3 : 0) + mat] + (wrow_g / 16) * (nks / 4) * 256;
    }
  }

  // Token rows of this lane's copies (rows past the tile repeat row 0): the
  // 256-byte step rows of xq through Stage, and one 4-byte half of a row's
  // 8 scale bytes per step (wavefront w copies rows 32w .. 32w+31, a lane
  // pair per row).
  using St = Stage<TT, O32>;
  St st;
  st.init(lane);
  int srow;
  {
    // all perm loads first (clamped into perm; the shared expert needs none)
    int pv[St::kPer];
#pragma unroll
    for (int i = 0; i < St::kPer; ++i) {
      const int n = St::row_of(i, wave, lane);
      pv[i] = p.perm[min(it.slot0 + (n < it.m ? n : 0), nk - 1)];
    }
    const int ns = 32 * wave + (lane >> 1);
    const int slot_s = it.slot0 + (ns < it.m ? ns : 0);
    const int pvs = p.perm[min(slot_s, nk - 1)];
#pragma unroll
    for (int i = 0; i < St::kPer; ++i) {
      const int n = St::row_of(i, wave, lane);
      const int slot = it.slot0 + (n < it.m ? n : 0);
      st.row[i] = shared ? slot - nk : pv[i] / p.top_k;
    }
    srow = shared ? slot_s - nk : pvs / p.top_k;
  }
  // the lane's bytes of its token-scale row: with O32 one 32-bit offset
  // from the uniform base (no 64-bit lane address to keep across items)
  using XsOff = std::conditional_t<O32, uint32_t, int64_t>;
  const XsOff xs_row = (XsOff)srow * (XsOff)(p.hidden / 16);
  const uint8_t* xsl = p.xs + (xs_row + 4 * (lane & 1));

  // weight codes: the current step and the next
  u32x4 q0[2][2][Q], q1[2][2][Q];
  uint32_t u0[2][2], u1[2][2];
  auto load_w = [&](int ks, u32x4 (&q)[2][2][Q], uint32_t (&u)[2][2]) {
    const int k = min(ks, nks - 1);  // past the end: reload the last step
    if constexpr (kPK) {
      // MXFP4 packed lines (routed experts, and a shared expert of the same
      // format) are read whole, once per token tile: past the caches, which
      // then keep the activation rows and scale words.  Packed fp8 codes
      // are only ever a shared expert's, read by every token tile of the
      // batch: cached.
#pragma unroll
      for (int mat = 0; mat < 2; ++mat)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < Q; ++i) {
            const u32x4* a = reinterpret_cast<const u32x4*>(
                pkc[mat] + (uint32_t)(((rb * nks + k) * Q + i) * 1024 + lane * 16));
            if constexpr (WT == MOE_W_MXFP4)
              q[mat][rb][i] = __builtin_nontemporal_load(a);
            else
              q[mat][rb][i] = load16(a);
          }
      return;
    }
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int i = 0; i < Q; ++i)
          q[mat][rb][i] = load16(cwave[mat] + (lco + (uint32_t)(16 * rb * cb + F::code_off(k, 0) + 64 * i)));
        if (!kSC && !kCh) u[mat][rb] = sbase[mat][ls + 16 * rb * sb + F::scale_off(k, 0)];
      }
  };
  // scale chunks (kCh): the 16 scale bytes of steps 4c .. 4c+3 of a row in
  // one load shared by the row's four lanes, once per four steps; the lane
  // keeps its own byte of each of the four steps in sp.  (Their lines can
  // leave the L2 between two loads, so this costs re-fetches that the LDS
  // copy avoids; it is the fallback where that copy does not fit.)
  u32x4 scw[2][2];
  uint32_t sp[2][2], spn[2][2];
  const int64_t srow_w = ls - F::scale_off(0, g);
  auto load_sc = [&](int c) {
    const int cc = min(c, nks / 4 - 1);
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if constexpr (kPK)
          spn[mat][rb] = *reinterpret_cast<const uint32_t*>(
              pks[mat] + (uint32_t)((rb * (nks / 4) + cc) * 256 + lane * 4));
        else if constexpr (WT == MOE_W_MXFP4)
          scw[mat][rb] = load16(sbase[mat] + srow_w + 16 * rb * sb + 16 * cc);
        else
          scw[mat][rb][0] =
              *reinterpret_cast<const uint32_t*>(sbase[mat] + srow_w + 16 * rb * sb + 4 * cc);
      }
  };
  auto take_sc = [&]() {
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if constexpr (kPK) {
          sp[mat][rb] = spn[mat][rb];
        } else if constexpr (WT == MOE_W_MXFP4) {
          uint32_t v = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t) v |= ((scw[mat][rb][t] >> (8 * g)) & 0xFFu) << (8 * t);
          sp[mat][rb] = v;
        } else {
          sp[mat][rb] = scw[mat][rb][0];
        }
      }
  };
  // scales (kSC): the item's kGuRows rows of each matrix are consecutive, so
  // their scale bytes are one contiguous block (kGuRows * H/32 bytes), copied
  // into LDS at the start of the item (1 KiB per copy instruction) and read
  // from there at every step.  Loaded from memory per step (one byte per
  // row) they doubled the weight stream's requests; loaded per four steps
  // (16 bytes) the lines left the L2 between loads and were fetched up to
  // eight times each.
  constexpr int kTokB = kSC ? 16 * NBT * 256 : TT * 256;  // bytes of one token tile
  char* const sscale = smem + kGuScaleOff;                // [mat][kGuRows][sb]
  auto copy_scales = [&]() {
    const int64_t bytes = (int64_t)kGuRows * sb;  // per matrix
    const int64_t row0 = (shared ? 0 : (int64_t)it.seg * rows) + it.row0;
#pragma unroll
    for (int mat = 0; mat < 2; ++mat) {
      const uint8_t* src = sbase[mat] + row0 * sb;
      for (int64_t o = (int64_t)wave * 1024; o < bytes; o += kGWaves * 1024)
        if (o + lane * 16 < bytes)
          __builtin_amdgcn_global_load_lds(
              src + o + lane * 16,
              (__attribute__((address_space(3))) void*)(sscale + mat * bytes + o), 16, 0, 0);
    }
  };
  auto scale_byte = [&](int mat, int rb, int ks) -> uint32_t {
    return *reinterpret_cast<const uint8_t*>(
        sscale + (mat * kGuRows + 32 * wave + 16 * rb + r16) * sb + ks * 4 + g);
  };

  f32x4 acc[2][2][TB];
#pragma unroll
  for (int mat = 0; mat < 2; ++mat)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[mat][rb][tb] = f32x4{0, 0, 0, 0};

  // token tile b at smem + b * kTokB, its scales at kTokScaleOff + b * 1 KiB
  // (offsets from smem keep LDS addressing)
  auto buf = [&](int b) { return smem + (b & 1) * kTokB; };
  // token scale bytes of step ks: per step (8 bytes a row), or with the
  // weight-scale chunks (kCh) per four steps (32 bytes a row, one request
  // per row instead of four), in buffer (ks / 4) & 1, row stride 32
  auto tsb = [&](int b) { return smem + kTokScaleOff + (b & 1) * kTokScaleBytes; };
  auto tsc = [&](int ks) -> const char* {
    return kCh ? smem + kTokChunkOff + ((ks >> 2) & 1) * (128 * 32) + (ks & 3) * 8 : tsb(ks);
  };
  constexpr int kTsStride = kCh ? 32 : 8;
  auto copy_tsc = [&](int c) {  // kCh: chunk c (steps 4c .. 4c+3), lane pairs of rows 32w ..
    const int cc = min(c, nks / 4 - 1);
    if (32 * wave < 16 * nbt)
      __builtin_amdgcn_global_load_lds(
          p.xs + (xs_row + (XsOff)(cc * 32 + 16 * (lane & 1))),
          (__attribute__((address_space(3))) void*)(smem + kTokChunkOff + (c & 1) * (128 * 32) +
                                                    1024 * wave),
          16, 0, 0);
  };
  // step ks's activations (rows, and per step their scale bytes) into buffer ks & 1
  auto copy_tok = [&](int ks) {
    st.copy(p.xq, 2 * (int64_t)p.hidden, ks, buf(ks), nbt);
    if (!kCh && 32 * wave < 16 * nbt)
      __builtin_amdgcn_global_load_lds(
          xsl + ks * 8, (__attribute__((address_space(3))) void*)(tsb(ks) + 256 * wave), 4, 0, 0);
  };
  // one reduction step: step ks's weights qq (and their scale bytes uu, when
  // not chunked) times the token tile in LDS, hi and lo parts
  auto step_mma = [&](int ks, const u32x4 (&qq)[2][2][Q], const uint32_t (&uu)[2][2]) {
    const char* cur = buf(ks);
    const char* cts = tsc(ks);
    uint32_t sa[2][2];
    i32x8 a[2][2];
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        sa[mat][rb] = kSC ? scale_byte(mat, rb, ks) : kCh ? sp[mat][rb] >> (8 * (ks & 3)) : uu[mat][rb];
        a[mat][rb] = weight_operand<WT>(qq[mat][rb]);
      }
    // operand u = 2 tb + part (part 0: hi bytes, chunks g and 4+g; part 1:
    // lo bytes, chunks 8+g and 12+g) is read while operand u-1 multiplies,
    // so two 8-register operands are live at a time
    // The lane's four chunk addresses in token block 0 and its scale bytes'
    // address, once per step; block tb lies tb * 4096 (scales tb * 16 *
    // kTsStride) bytes further, which the LDS reads take as their immediate
    // offset.  (Written as one expression per read, the compiler hoists a
    // separate loop-invariant register per token block and part.)
    lds_cptr pc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pc[c] = to_lds(cur) + r16 * 256 + (((4 * c + g) ^ r16) << 4);
      opaque(pc[c]);
    }
    lds_cptr ps = to_lds(cts) + r16 * kTsStride + 2 * g;
    opaque(ps);
    // operand u is read kAhead operands before it multiplies (a ring of
    // kAhead + 1 eight-register operands), so the LDS latency is covered by
    // 4 * kAhead instructions
    constexpr int kAhead = 1;
    i32x8 bop[kAhead + 1];
    uint32_t sbt[2];
    auto read_op = [&](int u) {
      const int tb = u >> 1, part = u & 1;
      bop[u % (kAhead + 1)] =
          join8(*reinterpret_cast<const lds_u32x4*>(pc[2 * part] + tb * 4096),
                *reinterpret_cast<const lds_u32x4*>(pc[2 * part + 1] + tb * 4096));
      if (part == 0)
        sbt[tb & 1] = *reinterpret_cast<const lds_u16*>(ps + tb * 16 * kTsStride);
    };
#pragma unroll
    for (int u = 0; u < kAhead && u < 2 * TB; ++u) read_op(u);
#pragma unroll
    for (int u = 0; u < 2 * TB; ++u) {
      if (u + kAhead < 2 * TB) read_op(u + kAhead);
      const int tb = u >> 1;
      const i32x8& b = bop[u % (kAhead + 1)];
#pragma unroll
      for (int mat = 0; mat < 2; ++mat)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          if ((u & 1) == 0)
            acc[mat][rb][tb] = mfma_scaled<FA, 0, 0>(a[mat][rb], b, acc[mat][rb][tb],
                                                     sa[mat][rb], sbt[tb & 1]);
          else
            acc[mat][rb][tb] = mfma_scaled<FA, 0, 1>(a[mat][rb], b, acc[mat][rb][tb],
                                                     sa[mat][rb], sbt[tb & 1]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (kSC) copy_scales();
  if (kCh) {
    load_sc(0);
    copy_tsc(0);
  }
  load_w(0, q0, u0);
  copy_tok(0);
  wait_vm<0>();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    // every fourth step (kCh): this chunk's scales out of the load
    // registers, then the next chunk's requested (before the step's other
    // loads, so that the end-of-step wait below still counts only the
    // weights after the copy)
    if (kCh && (ks & 3) == 0) {
      take_sc();
      load_sc((ks >> 2) + 1);
      copy_tsc((ks >> 2) + 1);  // its buffer held chunk c-1, done before this step
    }
    // step ks+1's activations, then its weights (one step ahead: the step
    // ends by moving them into q0, so a deeper register ring would only
    // wait for its loads at the same place)
    if (ks + 1 < nks) copy_tok(ks + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ks + 1, q1, u1);
    __builtin_amdgcn_sched_barrier(0);
    step_mma(ks, q0, u0);
    step_barrier<kLoads>();  // the copies have landed (the weights in flight)
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int i = 0; i < Q; ++i) q0[mat][rb][i] = q1[mat][rb][i];
        u0[mat][rb] = u1[mat][rb];
      }
  }
  wait_vm<0>();  // the reloads past the end
  take();        // the next item's ticket, in flight during the epilogue

  // SwiGLU, then h as three E4M3 parts (split_e4m3x3) under the scale of
  // the wavefront's 32 rows, which are one 32-input block of the down
  // projection: the lane holds rows 4g .. 4g+3 of row block rb for token
  // column r16, and the four lanes of a token meet in two shuffles.
  const int64_t hs = p.h_stride;
  if (LAZY && !shared) {
    // gate-first lazy skip: each slot's largest |SiLU(g)| over the
    // wavefront's 32 rows, merged into gmax (the combine leaves out the
    // slots below the threshold)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const float mx =
          silu_col_max(fmaxf(silu_abs_max4(acc[0][0][tb]), silu_abs_max4(acc[0][1][tb])));
      const int n = tb * 16 + r16;
      if (live && g == 0 && n < it.m) atomicMax(p.gmax + it.slot0 + n, __float_as_uint(mx));
    }
  }
  if constexpr (kH6) {
    // h as three E2M3 parts for the 32x32x64 down (packed MXFP4 layers):
    // the wavefront's 32 rows of a token are one block of the down's
    // reduction, so each lane first gathers a token's 32 values (through
    // LDS, the token tiles being free once every wavefront is past its last
    // step) and then converts them with the block conversion instructions:
    // part q under the scale 2^(e_q - 2) of the largest magnitude 2^e_q of
    // what the parts before left (2^(e_q - 1) when that would exceed 7.5),
    // so each part uses the whole E2M3 range.
    __syncthreads();
    float* const stage = reinterpret_cast<float*>(smem + wave * kH6Wave);  // [TT][kH6Row]
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = acc[0][rb][tb][r];
          hv[r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[1][rb][tb][r];
        }
        *reinterpret_cast<f32x4*>(stage + (tb * 16 + r16) * kH6Row + rb * 16 + 4 * g) = hv;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wavefront's LDS writes are done (lgkmcnt 0)
    __builtin_amdgcn_wave_barrier();
    const int kb = it.row0 / 32 + wave;  // the down's 32-value block of these rows
    if (live) {
      for (int t = lane; t < it.m; t += kWave) {
        float f[32];
        const float* src = stage + t * kH6Row;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + 4 * i);
#pragma unroll
          for (int j = 0; j < 4; ++j) f[4 * i + j] = v4[j];
        }
        const int64_t slot = it.slot0 + t;
        uint2* dst = reinterpret_cast<uint2*>(p.h6 + ((int64_t)kb * p.n_slots + slot) * 72);
        uint32_t sw = 0;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          float mag = 0.0f;
#pragma unroll
          for (int i = 0; i < 32; ++i) mag = fmaxf(mag, fabsf(f[i]));
          // biased exponent of the scale: e - 2, or e - 1 above 7.5 * 2^(e-2)
          int sb = (int)((__float_as_uint(mag) >> 23) & 0xFF) - 2;
          if (mag > 7.5f * __uint_as_float((uint32_t)max(sb, 1) << 23)) sb += 1;
          sb = min(max(sb, 1), 254);
          const float sc = __uint_as_float((uint32_t)sb << 23);
          // the conversion interleaves its two sources: value 2j from the
          // first, 2j+1 from the second
          f32x16 ev, od;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            ev[j] = f[2 * j];
            od[j] = f[2 * j + 1];
          }
          const u32x6 w = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, sc);
          const f32x32 back = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(w, sc);
#pragma unroll
          for (int i = 0; i < 32; ++i) f[i] -= back[i];
#pragma unroll
          for (int i = 0; i < 3; ++i) dst[3 * q + i] = uint2{w[2 * i], w[2 * i + 1]};
          sw |= (uint32_t)sb << (8 * q);
        }
        p.h6s[(int64_t)kb * p.n_slots + slot] = sw;
      }
    }
    return;
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    float v[2][4];
    float mag = 0.0f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = acc[0][rb][tb][r];
        // SiLU with the hardware exponential and reciprocal (a few ulp,
        // far below the 2^-12 that the three-part split keeps): the
        // range-reduced expf and the IEEE division cost about 20
        // instructions per element, most of this epilogue
        v[rb][r] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[1][rb][tb][r];
        mag = fmaxf(mag, fabsf(v[rb][r]));
      }
    mag = fmaxf(mag, __shfl_xor(mag, 16));
    mag = fmaxf(mag, __shfl_xor(mag, 32));
    uint32_t part[3][2];
    const uint32_t sbytes = split_e4m3x3(v, mag, part);
    const int n = tb * 16 + r16;
    if (live && n < it.m) {
      const int hrow = it.row0 + 32 * wave;  // h3 keeps 128-row blocks of three parts
      uint8_t* dst = p.h3 + (int64_t)(it.slot0 + n) * 3 * hs + (hrow >> 7) * 384 + (hrow & 127) + 4 * g;
#pragma unroll
      for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) *reinterpret_cast<uint32_t*>(dst + q * 128 + 16 * rb) = part[q][rb];
      if (g == 0)
        *reinterpret_cast<uint32_t*>(p.h3s + (int64_t)(it.slot0 + n) * (hs / 32) * 4 +
                                     (it.row0 / 32 + wave) * 4) = sbytes;
    }
  }
}

template <int WT, int TT, bool SC, bool O32, bool LAZY, bool PK, bool H6>
__global__ __launch_bounds__(kGThreads, kGPerCU) void gemm_gate_up_kernel(FfnParams p, int seg_lo,
                                                                     int seg_hi,
                                                                     uint32_t* qctr) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_pref[kSegMax + 1];
  __shared__ int s_tmp[kGThreads / kWave];
  __shared__ QueueLds s_q;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int total = item_prefix<TT, kGuRows, false>(p, seg_lo, seg_hi, s_pref, s_tmp);
  run_queue(ItemQueue{qctr, total, qctr != nullptr}, &s_q, [&](int item, auto&& take) {
    const GItem it = find_item<TT, kGuRows, false>(p, seg_lo, seg_hi, s_pref, item);
    dispatch_nbt<TT / 16>((it.m + 15) >> 4, [&](auto nb) {
      gate_up_item<WT, TT, decltype(nb)::value, SC, O32, LAZY, PK, H6>(p, it, smem, wave, lane,
                                                                    take);
    });
  });
}

// The packed MXFP4 routed experts (writing h6) and a packed fp8 shared
// expert in one launch: items below the routed total are routed 112-token
// items, the rest the shared expert's 64-token items.  The shared items make
// up the last chunks of the queue: the workgroups that start there run them
// first, the rest take them when their own chunks run dry, so no launch
// boundary idles the chip between the two.
template <bool LAZY>
__global__ __launch_bounds__(kGThreads, kGPerCU) void gemm_gate_up_mix_kernel(FfnParams p,
                                                                         uint32_t* qctr) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_pref[kSegMax + 1];
  __shared__ int s_tmp[kGThreads / kWave];
  __shared__ QueueLds s_q;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int E = p.n_experts;
  const int routed = item_prefix<112, kGuRows, false>(p, 0, E, s_pref, s_tmp);
  const int ntt = (p.n_tokens + 63) / 64, nrt = (p.shared_inter + kGuRows - 1) / kGuRows;
  const int total = routed + ntt * nrt;
  run_queue(ItemQueue{qctr, total, qctr != nullptr}, &s_q, [&](int item, auto&& take) {
    if (item >= routed) {
      // groups of eight token tiles, row tiles outer within a group: the
      // items in flight on one XCD share their tokens and weight rows in L2
      const int local = item - routed, g = local / (8 * nrt), in = local - g * 8 * nrt;
      const int gn = min(8, ntt - 8 * g), rt = in / gn, tile = 8 * g + (in - rt * gn);
      GItem it;
      it.seg = E;
      it.slot0 = uniform(p.n_tokens * p.top_k + tile * 64);
      it.m = uniform(min(64, p.n_tokens - tile * 64));
      it.row0 = uniform(rt * kGuRows);
      dispatch_nbt<4>((it.m + 15) >> 4, [&](auto nb) {
        gate_up_item<MOE_W_FP8E4M3_B128, 64, decltype(nb)::value, true, true, LAZY, true, false>(
            p, it, smem, wave, lane, take);
      });
      return;
    }
    const GItem it = find_item<112, kGuRows, false>(p, 0, E, s_pref, item);
    dispatch_nbt<7>((it.m + 15) >> 4, [&](auto nb) {
      gate_up_item<MOE_W_MXFP4, 112, decltype(nb)::value, true, true, LAZY, true, true>(
          p, it, smem, wave, lane, take);
    });
  });
}

// ------------------------------------------------------------- down

template <int WT, int TT, int NBT, bool SC, typename Take>
__device__ __forceinline__ void down_item(const FfnParams& p, const GItem& it, char* smem,
                                          int wave, int lane, Take&& take) {
  using F = Fmt<WT>;
  constexpr int Q = F::Q;
  constexpr int TB = NBT;
  constexpr int RB = kDnRows / (16 * kGWaves);  // row blocks per wavefront
  // scale bytes as in gate/up (SC: I a multiple of 512, and at most 2048
  // for MXFP4): MXFP4 in LDS for up to three token blocks (kSC), in 16-byte
  // chunks for four; fp8 four steps' bytes of a row in one 4-byte load
  constexpr bool kSC = SC && WT == MOE_W_MXFP4 && NBT <= 3;
  constexpr bool kCh = SC && (WT == MOE_W_MXFP4 ? NBT == 4 : true);
  constexpr int kLoads = (kSC || kCh) ? RB * Q : RB * (Q + 1);
  const int g = lane >> 4, r16 = lane & 15;
  const bool shared = it.seg == p.n_experts;
  const int kdim = shared ? p.shared_inter : p.inter;
  const int64_t cb = F::row_bytes(kdim), sb = F::scale_row_bytes(kdim);
  const int nks = kdim / 128;
  constexpr int nbt = NBT;
  // row blocks of this wavefront inside the matrix (the last tile may be short)
  const int wrow0 = it.row0 + 64 * wave;
  const int nrb = uniform(max(0, min(RB, (p.hidden - wrow0) / 16)));

  // the lane's row in block 0.  Blocks past the matrix end (only in a short
  // last row tile) reuse block 0's operands and are multiplied like the
  // others, but not stored: a test around each MFMA would make every one a
  // branch target with a full LDS wait in front of it.
  const int64_t r0 = wrow0 + r16 < p.hidden ? wrow0 + r16 : r16;
  const int64_t lrow = (shared ? 0 : (int64_t)it.seg * p.hidden) + r0;
  const int64_t lc = lrow * cb + F::code_off(0, g), ls = lrow * sb + F::scale_off(0, g);
  const uint8_t* cbase = shared ? p.sdown_c : p.down_c;
  const uint8_t* sbase = shared ? p.sdown_s : p.down_s;

  // h rows (slots) copied by this lane; rows past the tile repeat row 0
  Stage<TT> st;
  st.init(lane);
#pragma unroll
  for (int i = 0; i < Stage<TT>::kPer; ++i) {
    const int n = Stage<TT>::row_of(i, wave, lane);
    st.row[i] = it.slot0 + (n < it.m ? n : 0);
  }

  // weight codes of the current step and the next
  u32x4 q0[RB][Q], q1[RB][Q];
  uint32_t u0[RB], u1[RB];
  auto load_w = [&](int ks, u32x4 (&q)[RB][Q], uint32_t (&u)[RB]) {
    const int k = min(ks, nks - 1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rr = rb < nrb ? rb : 0;
#pragma unroll
      for (int i = 0; i < Q; ++i)
        q[rb][i] = load16(cbase + lc + 16 * rr * cb + F::code_off(k, 0) + 16 * i);
      if (!kSC && !kCh) u[rb] = sbase[ls + 16 * rr * sb + F::scale_off(k, 0)];
    }
  };
  u32x4 scw[RB];
  uint32_t sp[RB];
  const int64_t srow = ls - F::scale_off(0, g);
  auto load_sc = [&](int c) {
    const int cc = min(c, nks / 4 - 1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rr = rb < nrb ? rb : 0;
      if constexpr (WT == MOE_W_MXFP4)
        scw[rb] = load16(sbase + srow + 16 * rr * sb + 16 * cc);
      else
        scw[rb][0] = *reinterpret_cast<const uint32_t*>(sbase + srow + 16 * rr * sb + 4 * cc);
    }
  };
  auto take_sc = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (WT == MOE_W_MXFP4) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) v |= ((scw[rb][t] >> (8 * g)) & 0xFFu) << (8 * t);
        sp[rb] = v;
      } else {
        sp[rb] = scw[rb][0];
      }
    }
  };
  // scales (kSC), as in gate/up: the item's rows (up to kDnRows, fewer in the
  // last tile of the matrix) as one contiguous block in LDS
  constexpr int kTokB = kSC ? 16 * NBT * 256 : TT * 256;  // bytes of one h tile
  char* const sscale = smem + kDnScaleOff;                // [kDnRows][sb]
  auto copy_scales = [&]() {
    const int64_t bytes = (int64_t)min(kDnRows, p.hidden - it.row0) * sb;
    const uint8_t* src = sbase + ((shared ? 0 : (int64_t)it.seg * p.hidden) + it.row0) * sb;
    for (int64_t o = (int64_t)wave * 1024; o < bytes; o += kGWaves * 1024)
      if (o + lane * 16 < bytes)
        __builtin_amdgcn_global_load_lds(
            src + o + lane * 16, (__attribute__((address_space(3))) void*)(sscale + o), 16, 0,
            0);
  };
  auto scale_byte = [&](int rb, int ks) -> uint32_t {
    const int rr = rb < nrb ? rb : 0;
    return *reinterpret_cast<const uint8_t*>(sscale + (64 * wave + 16 * rr + r16) * sb + ks * 4 +
                                             g);
  };

  f32x4 acc[RB][TB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[rb][tb] = f32x4{0, 0, 0, 0};

  // h_hi of step parity b at smem + 2b * kTokB, h_lo right after it
  auto bh = [&](int b) { return smem + (b & 1) * (2 * kTokB); };
  auto bl = [&](int b) { return smem + (b & 1) * (2 * kTokB) + kTokB; };
  if (kSC) copy_scales();
  if (kCh) load_sc(0);
  load_w(0, q0, u0);
  st.copy(p.h_hi, 2 * p.h_stride, 0, bh(0), nbt);
  st.copy(p.h_lo, 2 * p.h_stride, 0, bl(0), nbt);
  wait_vm<0>();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    if (kCh && (ks & 3) == 0) {
      take_sc();
      load_sc((ks >> 2) + 1);
    }
    if (ks + 1 < nks) {
      st.copy(p.h_hi, 2 * p.h_stride, ks + 1, bh(ks + 1), nbt);
      st.copy(p.h_lo, 2 * p.h_stride, ks + 1, bl(ks + 1), nbt);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next step's weights (one step ahead: the step ends by moving them
    // into q0, so a deeper register ring would only wait for its loads there)
    load_w(ks + 1, q1, u1);
    __builtin_amdgcn_sched_barrier(0);
    const char* curh = bh(ks);
    const char* curl = bl(ks);
    float sc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      sc[rb] = ue8m0_to_f32(kSC ? scale_byte(rb, ks) : kCh ? (sp[rb] >> (8 * (ks & 3))) & 0xFFu
                                                            : u0[rb]);
    bf16x8 a[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) a[0][rb] = F::decode_j(q0[rb], sc[rb], 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j + 1 < 4) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) a[(j + 1) & 1][rb] = F::decode_j(q0[rb], sc[rb], j + 1);
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const bf16x8 fh = token_frag(curh, tb, j, g, r16);
        const bf16x8 fl = token_frag(curl, tb, j, g, r16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[rb][tb] = mfma_bf16(a[j & 1][rb], fh, acc[rb][tb]);
          acc[rb][tb] = mfma_bf16(a[j & 1][rb], fl, acc[rb][tb]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    step_barrier<kLoads>();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < Q; ++i) q0[rb][i] = q1[rb][i];
      u0[rb] = u1[rb];
    }
  }
  wait_vm<0>();
  take();  // the next item's ticket, in flight during the epilogue

  // the per-slot outputs, unweighted: the combine applies the routing
  // weights (so no item waits for them to arrive before its first step)
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int n = tb * 16 + r16;
    if (tb < nbt && n < it.m) {
      const int64_t slot = it.slot0 + n;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb < nrb)
          store_f24x4(p.obuf + (slot * p.hidden + wrow0 + 16 * rb + 4 * g) / 4 * 3, acc[rb][tb]);
      }
    }
  }
}

template <int WT, int TT, bool SC>
__global__ __launch_bounds__(kGThreads, kGPerCU) void gemm_down_kernel(FfnParams p, int seg_lo,
                                                                  int seg_hi, uint32_t* qctr) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_pref[kSegMax + 1];
  __shared__ int s_tmp[kGThreads / kWave];
  __shared__ QueueLds s_q;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int total = item_prefix<TT, kDnRows, true>(p, seg_lo, seg_hi, s_pref, s_tmp);
  run_queue(ItemQueue{qctr, total, qctr != nullptr}, &s_q, [&](int item, auto&& take) {
    const GItem it = find_item<TT, kDnRows, true>(p, seg_lo, seg_hi, s_pref, item);
    dispatch_nbt<TT / 16>((it.m + 15) >> 4, [&](auto nb) {
      down_item<WT, TT, decltype(nb)::value, SC>(p, it, smem, wave, lane, take);
    });
  });
}

// ------------------------------------------------------ down on E4M3 parts
//
// The grouped-GEMM path with bf16 x stores h as three E4M3 parts per
// element (split_e4m3x3).  The down projection feeds them to the scaled
// instruction as its B operand with the weight codes and scale bytes as
// stored: three 16x16x128 instructions per tile and step, where the bf16
// pair took eight 16x16x32 ones and a decode.  An h tile is three planes of
// 16 NBT rows x 128 bytes per step (one per part) and 16 scale bytes per
// row.  LDS per workgroup: two tiles, then (up to three token blocks) the
// item's weight scales, then the tiles' scale bytes.  Up to 64 tokens per
// tile: 96 would fit (so that an expert with up to 96 tokens streams its
// down weights once) but measured 8 % slower on hash4096 and 15 % slower on
// prefill512.
constexpr int kD3Tok = 64;
constexpr int kD3Full = 2 * 3 * kD3Tok * 128 + 2 * kD3Tok * 16;             // full tiles
constexpr int kD3Sc = 2 * 3 * 48 * 128 + kDnRows * (2048 / 32) + 2 * 48 * 16;  // 3 blocks + scales
constexpr int kD3Lds = kD3Full > kD3Sc ? kD3Full : kD3Sc;
static_assert(kD3Lds <= kGemmLds, "down LDS");

// An h plane in LDS has rows of 128 bytes: chunk c of row n sits at
// position c ^ ((n >> 1) & 7), so the 16 rows that one operand read touches
// (two rows share a 256-byte bank line) hit distinct banks.

template <int WT, int NBT, bool SC, bool PK, typename Take>
__device__ __forceinline__ void down3_item(const FfnParams& p, const GItem& it, char* smem,
                                           int wave, int lane, Take&& take) {
  using F = Fmt<WT>;
  constexpr int Q = F::Q;
  constexpr int TB = NBT;
  constexpr int kPlane = 16 * NBT * 128;  // one part's rows of a step
  constexpr int kBuf = 3 * kPlane;        // the three parts
  constexpr int FA = WT == MOE_W_MXFP4 ? 4 : 0;  // operand format of the weights
  constexpr int RB = kDnRows / (16 * kGWaves);  // row blocks per wavefront
  // scale bytes of the weights as in down_item; PK: the packed copy, as in
  // gate/up
  constexpr bool kPK = PK && SC;
  constexpr bool kSC = SC && WT == MOE_W_MXFP4 && NBT <= 3 && !kPK;
  constexpr bool kCh = SC && (WT == MOE_W_MXFP4 ? NBT == 4 || kPK : true);
  constexpr int kLoads = (kSC || kCh) ? RB * Q : RB * (Q + 1);
  const int g = lane >> 4, r16 = lane & 15;
  const bool shared = it.seg == p.n_experts;
  const int kdim = shared ? p.shared_inter : p.inter;
  const int64_t cb = F::row_bytes(kdim), sb = F::scale_row_bytes(kdim);
  const int nks = kdim / 128;
  constexpr int nbt = NBT;
  const int64_t hs = p.h_stride;
  // row blocks of this wavefront inside the matrix (the last tile may be
  // short; blocks past the end reuse block 0's operands, are multiplied and
  // not stored, as in down_item)
  const int wrow0 = it.row0 + 64 * wave;
  const int nrb = uniform(max(0, min(RB, (p.hidden - wrow0) / 16)));
  const int64_t r0 = wrow0 + r16 < p.hidden ? wrow0 + r16 : r16;
  const int64_t lrow = (shared ? 0 : (int64_t)it.seg * p.hidden) + r0;
  // code bytes of a step: MXFP4 16 at 16g; fp8 16 at 16g and 16 at 64 + 16g
  const int64_t lc = lrow * cb + 16 * g, ls = lrow * sb + F::scale_off(0, g);
  const uint8_t* cbase = shared ? p.sdown_c : p.down_c;
  const uint8_t* sbase = shared ? p.sdown_s : p.down_s;
  // packed: the wavefront's first row block (its 64 rows are four blocks;
  // a wavefront past the matrix end reads block 0 and multiplies nothing)
  const uint8_t* pkc = nullptr;
  const uint8_t* pks = nullptr;
  if constexpr (kPK) {
    const int64_t blk = ((shared ? 0 : (int64_t)it.seg * p.hidden) + (nrb > 0 ? wrow0 : 0)) / 16;
    pkc = p.pk_c[shared ? 5 : 2] + blk * nks * 1024 * Q;
    pks = p.pk_s[shared ? 5 : 2] + blk * (nks / 4) * 256;
  }

  // h copies: one instruction fills 8 rows of a part (lane l: row + l / 8,
  // position l % 8); wavefront w fills the row groups w, w + W, ... of each
  // part (W wavefronts; the groups below the tile), rows past the tile's
  // tokens repeat row 0.  Scale bytes: 16 rows per instruction (four lanes
  // per row), groups w, w + W, ...
  constexpr int kRG = (2 * NBT + kGWaves - 1) / kGWaves;  // row groups of 8 per wavefront
  constexpr int kSG = (NBT + kGWaves - 1) / kGWaves;      // scale groups of 16 per wavefront
  int64_t hsrc[kRG];
#pragma unroll
  for (int e = 0; e < kRG; ++e) {
    const int n = 8 * (wave + kGWaves * e) + (lane >> 3);
    const int c = (lane & 7) ^ ((n >> 1) & 7);
    hsrc[e] = (int64_t)(it.slot0 + (n < it.m ? n : 0)) * 3 * hs + 16 * c;
  }
  const uint8_t* hss[kSG];
#pragma unroll
  for (int e = 0; e < kSG; ++e) {
    const int ns = 16 * (wave + kGWaves * e) + (lane >> 2);
    hss[e] = p.h3s + (int64_t)(it.slot0 + (ns < it.m ? ns : 0)) * (hs / 32) * 4 + 4 * (lane & 3);
  }
  // LDS: tiles, the weight scales (kSC), the tiles' scale bytes
  constexpr int kWScOff = 2 * kBuf;
  constexpr int kTScOff = kWScOff + (kSC ? kDnRows * (2048 / 32) : 0);
  static_assert(kTScOff + 2 * 16 * NBT * 16 <= kD3Lds, "down LDS");
  auto lds = [](char* q) { return (__attribute__((address_space(3))) void*)q; };
  auto hbuf = [&](int b) { return smem + (b & 1) * kBuf; };
  auto sbuf = [&](int b) { return smem + kTScOff + (b & 1) * (16 * NBT * 16); };
  auto copy_h = [&](int ks) {
    char* dst = hbuf(ks);
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int e = 0; e < kRG; ++e) {
        const int rg = wave + kGWaves * e;
        if (rg < 2 * nbt)
          __builtin_amdgcn_global_load_lds(p.h3 + hsrc[e] + ks * 384 + q * 128,
                                           lds(dst + q * kPlane + rg * 8 * 128), 16, 0, 0);
      }
#pragma unroll
    for (int e = 0; e < kSG; ++e) {
      const int sg = wave + kGWaves * e;
      if (sg < nbt)
        __builtin_amdgcn_global_load_lds(hss[e] + ks * 16, lds(sbuf(ks) + sg * 256), 4, 0, 0);
    }
  };

  // weight codes of the current step and the next
  u32x4 q0[RB][Q], q1[RB][Q];
  uint32_t u0[RB], u1[RB];
  auto load_w = [&](int ks, u32x4 (&q)[RB][Q], uint32_t (&u)[RB]) {
    const int k = min(ks, nks - 1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rr = rb < nrb ? rb : 0;
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        if constexpr (kPK)
          q[rb][i] = load16(pkc + (uint32_t)(((rr * nks + k) * Q + i) * 1024 + lane * 16));
        else
          q[rb][i] = load16(cbase + lc + 16 * rr * cb + F::code_off(k, 0) + 64 * i);
      }
      if (!kSC && !kCh) u[rb] = sbase[ls + 16 * rr * sb + F::scale_off(k, 0)];
    }
  };
  u32x4 scw[RB];
  uint32_t sp[RB], spn[RB];
  const int64_t srow = ls - F::scale_off(0, g);
  auto load_sc = [&](int c) {
    const int cc = min(c, nks / 4 - 1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rr = rb < nrb ? rb : 0;
      if constexpr (kPK)
        spn[rb] = *reinterpret_cast<const uint32_t*>(
            pks + (uint32_t)((rr * (nks / 4) + cc) * 256 + lane * 4));
      else if constexpr (WT == MOE_W_MXFP4)
        scw[rb] = load16(sbase + srow + 16 * rr * sb + 16 * cc);
      else
        scw[rb][0] = *reinterpret_cast<const uint32_t*>(sbase + srow + 16 * rr * sb + 4 * cc);
    }
  };
  auto take_sc = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (kPK) {
        sp[rb] = spn[rb];
      } else if constexpr (WT == MOE_W_MXFP4) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) v |= ((scw[rb][t] >> (8 * g)) & 0xFFu) << (8 * t);
        sp[rb] = v;
      } else {
        sp[rb] = scw[rb][0];
      }
    }
  };
  // weight scales (kSC): the item's rows as one contiguous block in LDS
  char* const sscale = smem + kWScOff;  // [kDnRows][sb]
  auto copy_scales = [&]() {
    const int64_t bytes = (int64_t)min(kDnRows, p.hidden - it.row0) * sb;
    const uint8_t* src = sbase + ((shared ? 0 : (int64_t)it.seg * p.hidden) + it.row0) * sb;
    for (int64_t o = (int64_t)wave * 1024; o < bytes; o += kGWaves * 1024)
      if (o + lane * 16 < bytes)
        __builtin_amdgcn_global_load_lds(src + o + lane * 16, lds(sscale + o), 16, 0, 0);
  };
  auto scale_byte = [&](int rb, int ks) -> uint32_t {
    const int rr = rb < nrb ? rb : 0;
    return *reinterpret_cast<const uint8_t*>(sscale + (64 * wave + 16 * rr + r16) * sb + ks * 4 +
                                             g);
  };

  f32x4 acc[RB][TB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[rb][tb] = f32x4{0, 0, 0, 0};

  auto step_mma = [&](int ks, const u32x4 (&qq)[RB][Q], const uint32_t (&uu)[RB]) {
    const char* cur = hbuf(ks);
    const char* cts = sbuf(ks);
    uint32_t sa[RB];
    i32x8 a[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      sa[rb] = kSC ? scale_byte(rb, ks) : kCh ? sp[rb] >> (8 * (ks & 3)) : uu[rb];
      a[rb] = weight_operand<WT>(qq[rb]);
    }
    // operand u = 3 tb + part (h part q = u % 3).  The lane's two chunk addresses in token block 0 of part 0 and its scale
    // bytes' address are formed once per step (the swizzle depends on the
    // row within the block only); part q and block tb lie q * kPlane +
    // tb * 2048 (scales tb * 256) bytes further: immediate offsets.
    lds_cptr pc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      pc[c] = to_lds(cur) + r16 * 128 + (((4 * c + g) ^ ((r16 >> 1) & 7)) << 4);
      opaque(pc[c]);
    }
    lds_cptr ps = to_lds(cts) + r16 * 16 + 4 * g;
    opaque(ps);
    // a ring of kAhead + 1 operands: operand u is read kAhead before use.
    // With one ahead, the three parts per token block (an odd count against
    // a ring of two) led the register allocator to move accumulators
    // through the operand registers, so most reads waited behind the MFMAs
    // before them; with two ahead every operand keeps its own registers.
    constexpr int kAhead = 2;
    i32x8 bop[kAhead + 1];
    uint32_t sbt[2];
    auto read_op = [&](int u) {
      const int tb = u / 3, q = u % 3;
      const int off = q * kPlane + tb * 2048;
      bop[u % (kAhead + 1)] = join8(*reinterpret_cast<const lds_u32x4*>(pc[0] + off),
                                    *reinterpret_cast<const lds_u32x4*>(pc[1] + off));
      if (q == 0) sbt[tb & 1] = *reinterpret_cast<const lds_u32*>(ps + tb * 256);
    };
#pragma unroll
    for (int u = 0; u < kAhead && u < 3 * TB; ++u) read_op(u);
#pragma unroll
    for (int u = 0; u < 3 * TB; ++u) {
      if (u + kAhead < 3 * TB) read_op(u + kAhead);
      const int tb = u / 3, q = u % 3;
      const i32x8& b = bop[u % (kAhead + 1)];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (q == 0)
          acc[rb][tb] = mfma_scaled<FA, 0, 0>(a[rb], b, acc[rb][tb], sa[rb], sbt[tb & 1]);
        else if (q == 1)
          acc[rb][tb] = mfma_scaled<FA, 0, 1>(a[rb], b, acc[rb][tb], sa[rb], sbt[tb & 1]);
        else
          acc[rb][tb] = mfma_scaled<FA, 0, 2>(a[rb], b, acc[rb][tb], sa[rb], sbt[tb & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (kSC) copy_scales();
  if (kCh) load_sc(0);
  load_w(0, q0, u0);
  copy_h(0);
  wait_vm<0>();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    if (kCh && (ks & 3) == 0) {
      take_sc();
      load_sc((ks >> 2) + 1);
    }
    if (ks + 1 < nks) copy_h(ks + 1);
    __builtin_amdgcn_sched_barrier(0);
    // the next step's weights (one step ahead: the step ends by moving them
    // into q0, so a deeper register ring would only wait for its loads there)
    load_w(ks + 1, q1, u1);
    __builtin_amdgcn_sched_barrier(0);
    step_mma(ks, q0, u0);
    step_barrier<kLoads>();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < Q; ++i) q0[rb][i] = q1[rb][i];
      u0[rb] = u1[rb];
    }
  }
  wait_vm<0>();
  take();  // the next item's ticket, in flight during the epilogue

  // the per-slot outputs, unweighted: the combine applies the routing
  // weights (so no item waits for them to arrive before its first step)
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int n = tb * 16 + r16;
    if (tb < nbt && n < it.m) {
      const int64_t slot = it.slot0 + n;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb < nrb)
          store_f24x4(p.obuf + (slot * p.hidden + wrow0 + 16 * rb + 4 * g) / 4 * 3, acc[rb][tb]);
      }
    }
  }
}

template <int WT, bool SC, bool PK>
__global__ __launch_bounds__(kGThreads, kGPerCU) void gemm_down3_kernel(FfnParams p, int seg_lo,
                                                                   int seg_hi, uint32_t* qctr) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_pref[kSegMax + 1];
  __shared__ int s_tmp[kGThreads / kWave];
  const int lane = threadIdx.x & 63, wave = wave_id();
  __shared__ QueueLds s_q;
  const int total = item_prefix<kD3Tok, kDnRows, true>(p, seg_lo, seg_hi, s_pref, s_tmp);
  run_queue(ItemQueue{qctr, total, qctr != nullptr}, &s_q, [&](int item, auto&& take) {
    const GItem it = find_item<kD3Tok, kDnRows, true>(p, seg_lo, seg_hi, s_pref, item);
    dispatch_nbt<kD3Tok / 16>((it.m + 15) >> 4, [&](auto nb) {
      down3_item<WT, decltype(nb)::value, SC, PK>(p, it, smem, wave, lane, take);
    });
  });
}

// ------------------------------------------------- down on E2M3 parts of h
//
// With the packed copy, the MXFP4 down multiplies h as three E2M3 parts
// (h6, written by the gate/up epilogue) on v_mfma_scale_f32_32x32x64_f8f6f4,
// which issues E2M1 x E2M3 at about twice the rate of any 16x16x128 form:
// 3 x 1/2 of the matrix time of one E4M3 product instead of 3 x 1.  A
// workgroup owns 256 hidden rows and up to 64 tokens (two 32-token blocks);
// wavefront w owns rows 64w .. 64w+63 (two 32-row blocks).  Per step of 128
// inputs a 32-row block is two instructions of 64 inputs per token block and
// part.
//  - A (weights): lane l holds row l % 32 and inputs 32 (l / 32) .. +31 of
//    the 64, i.e. the 16 bytes of lane 16 g + (l % 16) of the packed copy's
//    16-row block (l % 32) / 16, g = l / 32 (first 64 inputs) or 2 + l / 32;
//    its scale word is that lane's too.
//  - B (h): lane l holds token l % 32 and the same 32 inputs: 24 bytes of
//    one part; the step's four blocks of 32 inputs are copied into LDS as
//    planes [64 tokens][72 bytes] (a token's three parts), whose 72-byte
//    stride puts the 32 tokens of a read on distinct banks.  The LDS copy
//    instruction writes 16 bytes per lane (its 12-byte form also advances
//    16 bytes per lane), so the 4.5 KiB of a plane take five of them and the
//    plane is padded to 5 KiB.
//  - D: lane l holds token l % 32 and rows 8 j + 4 (l / 32) + 0..3.
// one block of 32 inputs: 64 tokens x 72 bytes, padded to whole copies of
// 1 KiB (16 bytes per lane)
constexpr int kD6Plane = (kD3Tok * 72 + 1023) / 1024 * 1024;
constexpr int kD6Buf = 4 * kD6Plane;             // a step (20 KiB)
constexpr int kD6Ring = 3;                       // steps in LDS: the current and two ahead
constexpr int kD6ScOff = kD6Ring * kD6Buf;
constexpr int kD6ScBuf = 4 * kD3Tok * 4;          // a step's scale words
// the weights' scale words of a chunk of four steps, per wavefront its four
// 16-row blocks x 256 bytes, two chunks
constexpr int kD6WsOff = kD6ScOff + kD6Ring * kD6ScBuf;
constexpr int kD6WsBuf = 4 * 4 * 256;
constexpr int kD6Lds = kD6WsOff + 2 * kD6WsBuf;
static_assert(kD6Lds <= kGemmLds, "down LDS");

template <int SB>
__device__ __forceinline__ f32x16 mfma32_e2m1_e2m3(i32x8 a, i32x8 b, f32x16 c, uint32_t sa,
                                                    uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 2, 0, (int)sa, SB, (int)sb);
}

// NB = 32-token blocks of the tile (ceil(m / 32)).
template <int NB, typename Take>
__device__ __forceinline__ void down6_item(const FfnParams& p, const GItem& it, char* smem,
                                           int wave, int lane, Take&& take) {
  constexpr int RB = 2;           // 32-row blocks per wavefront
  constexpr int kLoads = 2 * RB;  // loads of one step's weight codes
  const int hi = lane >> 5, l32 = lane & 31;
  const int b16 = (lane >> 4) & 1, r16 = lane & 15;
  const bool shared = it.seg == p.n_experts;
  const int kdim = shared ? p.shared_inter : p.inter;
  const int nks = kdim / 128;
  const int wrow0 = it.row0 + 64 * wave;
  // 16-row blocks of this wavefront inside the matrix (the last tile may be
  // short: blocks past the end reuse block 0's codes and are not stored)
  const int nrb16 = uniform(max(0, min(4, (p.hidden - wrow0) / 16)));
  const int64_t blk0 = ((shared ? 0 : (int64_t)it.seg * p.hidden) + (nrb16 > 0 ? wrow0 : 0)) / 16;
  const uint8_t* pkc = p.pk_c[shared ? 5 : 2] + blk0 * nks * 1024;
  const uint8_t* pks = p.pk_s[shared ? 5 : 2] + blk0 * (nks / 4) * 256;
  // the lane's code unit (step 0) for 32-row block rb and input half s of a
  // step, and its scale word in the wavefront's chunk of scales in LDS
  uint32_t aoff[RB][2], soff[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int bb = 2 * rb + b16;
    const int blk = bb < nrb16 ? bb : 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int unit = 16 * (hi + 2 * s) + r16;
      aoff[rb][s] = (uint32_t)(blk * nks * 1024 + unit * 16);
      soff[rb][s] = (uint32_t)(bb * 256 + unit * 4);
    }
  }
  auto lds = [](char* q) { return (__attribute__((address_space(3))) void*)q; };
  // step ks into buffer b: wavefront w copies block 4 ks + w of the tile's
  // m tokens (72 contiguous bytes each in h6, 16 bytes per lane and
  // instruction, whole KiB into the padded plane) and their scale words.
  // A lane whose 16 bytes start past the m tokens re-reads the tile's first
  // 16 (its LDS bytes only feed token columns never stored); the lane that
  // straddles the end reads up to 8 bytes past it, which h6 always holds
  // (the next slot's record, or the 16 bytes of padding after the last).
  // No lane branches.
  auto copy_h = [&](int ks, int b) {
    const int64_t kb = 4 * ks + wave;
    const uint8_t* src = p.h6 + (kb * p.n_slots + it.slot0) * 72;
    char* dst = smem + b * kD6Buf + wave * kD6Plane;
    const int nbytes = it.m * 72;
#pragma unroll
    for (int c = 0; c < kD6Plane / 1024; ++c) {
      const int o = 1024 * c + 16 * lane;
      __builtin_amdgcn_global_load_lds(src + (o < nbytes ? o : 0), lds(dst + 1024 * c), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(p.h6s + kb * p.n_slots + it.slot0 + (lane < it.m ? lane : 0),
                                     lds(smem + kD6ScOff + b * kD6ScBuf + wave * 256), 4, 0, 0);
  };
  // weight codes of three steps in registers (the current one and two
  // ahead)
  u32x4 qb[kD6Ring][RB][2];
  auto load_w = [&](int ks, u32x4 (&q)[RB][2]) {
    const uint32_t k = (uint32_t)min(ks, nks - 1);  // past the end: reload the last step
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < 2; ++s) q[rb][s] = load16(pkc + (aoff[rb][s] + k * 1024));
  };
  // the weights' scale words of chunk c (steps 4c .. 4c+3) into LDS buffer
  // c % 2: one 16-byte copy per lane, lane l taking bytes 16 (l % 16) .. of
  // 16-row block l / 16 of the wavefront (block 0 for blocks past the
  // matrix end); a lane's words are then read per step from LDS (they were
  // four requests per step)
  auto copy_ws = [&](int c) {
    const int bb = lane >> 4;
    const int blk = bb < nrb16 ? bb : 0;
    const uint8_t* src = pks + (blk * (nks / 4) + min(c, nks / 4 - 1)) * 256 + (lane & 15) * 16;
    __builtin_amdgcn_global_load_lds(src, lds(smem + kD6WsOff + (c & 1) * kD6WsBuf + wave * 1024),
                                     16, 0, 0);
  };

  f32x16 acc[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][tb][e] = 0.0f;

  auto step_mma = [&](int ks, int buf, const u32x4 (&q)[RB][2]) {
    const char* cur = smem + buf * kD6Buf;
    const char* cts = smem + kD6ScOff + buf * kD6ScBuf;
    const char* cws = smem + kD6WsOff + ((ks >> 2) & 1) * kD6WsBuf + wave * 1024;
    i32x8 a[RB][2];
    uint32_t sa[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        a[rb][s] = i32x8{(int)q[rb][s][0], (int)q[rb][s][1], (int)q[rb][s][2], (int)q[rb][s][3],
                         0, 0, 0, 0};
        sa[rb][s] = *reinterpret_cast<const lds_u32*>(to_lds(cws) + soff[rb][s]) >> (8 * (ks & 3));
      }
    // operand u = (3 s + q) NB + tb: token 32 tb + l32, block 2 s + hi of
    // the step, part q, at plane (2 s + hi) + token * 72 + q * 24.  Token
    // blocks innermost, so that consecutive instructions go to NB x RB
    // different accumulators (a 32x32 product waits for the one before on
    // its accumulator).
    lds_cptr pb = to_lds(cur) + hi * kD6Plane + l32 * 72;
    opaque(pb);
    lds_cptr ps = to_lds(cts) + hi * 256 + l32 * 4;
    opaque(ps);
    constexpr int kOps = 6 * NB;
    constexpr int kAhead = 2;
    i32x8 bop[kAhead + 1];
    uint32_t sbt[2][NB];
    auto read_op = [&](int u) {
      const int tb = u % NB, q = (u / NB) % 3, s = u / (3 * NB);
      const int off = 2 * s * kD6Plane + tb * 32 * 72 + q * 24;
      // (vector-typed LDS reads: the compiler then leaves the LDS copies in
      // flight; its wait for them is the end-of-step barrier's)
      const u32x2 w0 = *reinterpret_cast<const lds_u32x2*>(pb + off);
      const u32x2 w1 = *reinterpret_cast<const lds_u32x2*>(pb + off + 8);
      const u32x2 w2 = *reinterpret_cast<const lds_u32x2*>(pb + off + 16);
      bop[u % (kAhead + 1)] = i32x8{(int)w0.x, (int)w0.y, (int)w1.x, (int)w1.y,
                                    (int)w2.x, (int)w2.y, 0, 0};
      if (q == 0) sbt[s][tb] = *reinterpret_cast<const lds_u32*>(ps + 2 * s * 256 + tb * 128);
    };
#pragma unroll
    for (int u = 0; u < kAhead && u < kOps; ++u) read_op(u);
#pragma unroll
    for (int u = 0; u < kOps; ++u) {
      if (u + kAhead < kOps) read_op(u + kAhead);
      const int tb = u % NB, q = (u / NB) % 3, s = u / (3 * NB);
      const i32x8& b = bop[u % (kAhead + 1)];
      const uint32_t sb = sbt[s][tb];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (q == 0)
          acc[rb][tb] = mfma32_e2m1_e2m3<0>(a[rb][s], b, acc[rb][tb], sa[rb][s], sb);
        else if (q == 1)
          acc[rb][tb] = mfma32_e2m1_e2m3<1>(a[rb][s], b, acc[rb][tb], sa[rb][s], sb);
        else
          acc[rb][tb] = mfma32_e2m1_e2m3<2>(a[rb][s], b, acc[rb][tb], sa[rb][s], sb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // step ks (buffers B = ks % 3): at the start of a chunk the next chunk's
  // scale words, then step ks+2's copies and weights (the last steps'
  // copies clamped to a step that exists), then the step's products.  At
  // its end at most the kCopies + kLoads requests just issued remain in
  // flight: step ks+1's copies (issued a step earlier and followed by step
  // ks+1's weights and step ks+2's copies, at least that many requests;
  // the compiler drops the unused weight loads of steps past the end) and
  // the scale words have landed; the workgroup barrier frees buffer B for
  // the copies of step ks+3 and, at the end of a chunk, the scale buffer
  // for the chunk after next.
  constexpr int kCopies = kD6Plane / 1024 + 1;
  auto step = [&](auto B, auto K) {
    constexpr int b = decltype(B)::value, ks = decltype(K)::value;
    if constexpr (ks % 4 == 0) copy_ws(ks / 4 + 1);
    copy_h(min(ks + 2, nks - 1), (b + 2) % kD6Ring);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ks + 2, qb[(b + 2) % kD6Ring]);
    __builtin_amdgcn_sched_barrier(0);
    step_mma(ks, b, qb[b]);
    step_barrier<kCopies + kLoads>();
  };

  copy_ws(0);
  load_w(0, qb[0]);
  copy_h(0, 0);
  load_w(1, qb[1]);
  copy_h(1, 1);  // (a reduction has at least four steps)
  step_barrier<kCopies + kLoads>();  // chunk 0's scales and step 0's copies landed
  // The steps as straight-line code, four at a time (the reduction is 4, 8,
  // 12 or 16 steps), nested so that no join follows a step: in a loop, the
  // compiler's wait analysis, merging the entry and the back edge, took the
  // registers loaded two steps earlier for loads still in flight and,
  // with LDS copies pending, waited for every load (the ones just issued
  // too).  Here it knows them complete from the end-of-step waits.
  auto four = [&](auto C) {
    static_for<4 * decltype(C)::value, 4 * decltype(C)::value + 4>([&](auto K) {
      constexpr int k = decltype(K)::value;
      step(IntC<k % kD6Ring>{}, K);
    });
  };
  four(IntC<0>{});
  if (nks > 4) {
    four(IntC<1>{});
    if (nks > 8) {
      four(IntC<2>{});
      if (nks > 12) four(IntC<3>{});
    }
  }
  wait_vm<0>();
  take();  // the next item's ticket, in flight during the epilogue

  // the per-slot outputs, unweighted (the combine applies the routing
  // weights): rows 8 j + 4 hi .. +3 of each 32-row block.  (Staged through
  // LDS so that twelve lanes write a token's 192 contiguous bytes, the
  // stores measured slower: their cost is the bytes.)
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) {
    const int n = tb * 32 + l32;
    if (n < it.m) {
      const int64_t slot = it.slot0 + n;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 32 * rb + 8 * j + 4 * hi;
          if (row / 16 < nrb16)
            store_f24x4(p.obuf + (slot * p.hidden + wrow0 + row) / 4 * 3,
                        f32x4{acc[rb][tb][4 * j], acc[rb][tb][4 * j + 1], acc[rb][tb][4 * j + 2],
                              acc[rb][tb][4 * j + 3]});
        }
    }
  }
}

// MIX: the launch also takes an fp8 shared expert (h in E4M3 parts, its
// packed copy), whose items make up the last chunks of the queue.
template <bool MIX>
__global__ __launch_bounds__(kGThreads, kGPerCU) void gemm_down6_kernel(FfnParams p, int seg_lo,
                                                                   int seg_hi, uint32_t* qctr) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_pref[kSegMax + 1];
  __shared__ int s_tmp[kGThreads / kWave];
  __shared__ QueueLds s_q;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int total = item_prefix<kD3Tok, kDnRows, true>(p, seg_lo, seg_hi, s_pref, s_tmp);
  run_queue(ItemQueue{qctr, total, qctr != nullptr}, &s_q, [&](int item, auto&& take) {
    if (MIX && item >= s_pref[p.n_experts - seg_lo]) {
      // the shared expert's items in groups of eight token tiles, row
      // tiles outer within a group (as in the gate/up)
      const int ntt = (p.n_tokens + kD3Tok - 1) / kD3Tok, nrt = p.hidden / kDnRows;
      const int local = item - s_pref[p.n_experts - seg_lo], g = local / (8 * nrt);
      const int in = local - g * 8 * nrt, gn = min(8, ntt - 8 * g), rt = in / gn;
      const int tile = 8 * g + (in - rt * gn);
      GItem it;
      it.seg = p.n_experts;
      it.slot0 = uniform(p.n_tokens * p.top_k + tile * kD3Tok);
      it.m = uniform(min(kD3Tok, p.n_tokens - tile * kD3Tok));
      it.row0 = uniform(rt * kDnRows);
      dispatch_nbt<kD3Tok / 16>((it.m + 15) >> 4, [&](auto nb) {
        down3_item<MOE_W_FP8E4M3_B128, decltype(nb)::value, true, true>(p, it, smem, wave, lane,
                                                                       take);
      });
      return;
    }
    const GItem it = find_item<kD3Tok, kDnRows, true>(p, seg_lo, seg_hi, s_pref, item);
    dispatch_nbt<2>((it.m + 31) >> 5, [&](auto nb) {
      down6_item<decltype(nb)::value>(p, it, smem, wave, lane, take);
    });
  });
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

template <typename K>
hipError_t allow_lds(K kernel) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
}

// Upper bound on the items of segments seg_lo .. seg_hi-1: routed token
// tiles number at most N*k/TT + min(E, N*k); the shared expert has
// ceil(N/TT).
int64_t items_bound(const FfnParams& p, int seg_lo, int seg_hi, int tt, int rt, bool down) {
  int64_t items = 0;
  if (seg_lo < p.n_experts) {
    const int64_t nk = (int64_t)p.n_tokens * p.top_k;
    const int64_t tiles = nk / tt + (nk < p.n_experts ? nk : p.n_experts);
    const int64_t rows = down ? p.hidden : p.inter;
    items += tiles * ((rows + rt - 1) / rt);
  }
  if (seg_hi > p.n_experts) {
    const int64_t rows = down ? p.hidden : p.shared_inter;
    items += (p.n_tokens + tt - 1) / tt * ((rows + rt - 1) / rt);
  }
  return items;
}

constexpr int kGemmGrid = 256 * kGPerCU;  // 256 CUs

// The eight queue counters of a launch with the dynamic schedule, or null
// for the static one.  Dynamic: launches with the routed experts when they
// average at least 32 slots each (long items of uneven length); a launch of
// the shared expert alone has items of one size.  Counters: gate/up of the
// routed experts (with the shared one when it shares the launch), gate/up of
// a shared expert of another type, then the same two for the down
// projection.
uint32_t* queue_counters(const FfnParams& p, int seg_lo, bool down) {
  const bool shared_only = seg_lo >= p.n_experts;
  if (shared_only || (int64_t)p.n_tokens * p.top_k < 32 * (int64_t)p.n_experts) return nullptr;
  return p.qctr + 8 * ((down ? 2 : 0) + (shared_only ? 1 : 0));
}

int grid_for(int64_t items) {
  return (int)(items < kGemmGrid ? (items > 0 ? items : 1) : kGemmGrid);
}

template <int WT, int TT, bool SC, bool O32, bool LAZY, bool PK, bool H6>
hipError_t gate_up_range_as(const FfnParams& p, int seg_lo, int seg_hi, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop) {
  static const hipError_t attr = allow_lds(gemm_gate_up_kernel<WT, TT, SC, O32, LAZY, PK, H6>);
  if (attr != hipSuccess) return attr;
  const int grid = grid_for(items_bound(p, seg_lo, seg_hi, TT, kGuRows, false));
  return launch(gemm_gate_up_kernel<WT, TT, SC, O32, LAZY, PK, H6>, dim3(grid), dim3(kGThreads),
                (size_t)kGemmLds, stream, start, stop, p, seg_lo, seg_hi,
                queue_counters(p, seg_lo, false));
}

template <bool LAZY>
hipError_t gate_up_mix_as(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
  static const hipError_t attr = allow_lds(gemm_gate_up_mix_kernel<LAZY>);
  if (attr != hipSuccess) return attr;
  const int grid = grid_for(items_bound(p, 0, p.n_experts + 1, 64, kGuRows, false));
  return launch(gemm_gate_up_mix_kernel<LAZY>, dim3(grid), dim3(kGThreads), (size_t)kGemmLds,
                stream, start, stop, p, queue_counters(p, 0, false));
}

template <int WT, int TT, bool SC, bool O32, bool PK = false, bool H6 = false>
hipError_t gate_up_range(const FfnParams& p, int seg_lo, int seg_hi, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop) {
  if (p.lazy_tau > 0.0f)
    return gate_up_range_as<WT, TT, SC, O32, true, PK, H6>(p, seg_lo, seg_hi, stream, start, stop);
  return gate_up_range_as<WT, TT, SC, O32, false, PK, H6>(p, seg_lo, seg_hi, stream, start, stop);
}

template <bool MIX>
hipError_t down6_range(const FfnParams& p, int seg_lo, int seg_hi, hipStream_t stream,
                       hipEvent_t start, hipEvent_t stop) {
  constexpr int lds = MIX && kD3Lds > kD6Lds ? kD3Lds : kD6Lds;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_down6_kernel<MIX>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int grid = grid_for(items_bound(p, seg_lo, seg_hi, kD3Tok, kDnRows, true));
  return launch(gemm_down6_kernel<MIX>, dim3(grid), dim3(kGThreads), (size_t)lds, stream, start,
                stop, p, seg_lo, seg_hi, queue_counters(p, seg_lo, true));
}

template <int WT, bool SC, bool PK = false>
hipError_t down3_range(const FfnParams& p, int seg_lo, int seg_hi, hipStream_t stream,
                       hipEvent_t start, hipEvent_t stop) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_down3_kernel<WT, SC, PK>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kD3Lds);
  if (attr != hipSuccess) return attr;
  const int grid = grid_for(items_bound(p, seg_lo, seg_hi, kD3Tok, kDnRows, true));
  return launch(gemm_down3_kernel<WT, SC, PK>, dim3(grid), dim3(kGThreads), (size_t)kD3Lds,
                stream, start, stop, p, seg_lo, seg_hi, queue_counters(p, seg_lo, true));
}

template <int WT, int TT, bool SC>
hipError_t down_range(const FfnParams& p, int seg_lo, int seg_hi, hipStream_t stream,
                      hipEvent_t start, hipEvent_t stop) {
  static const hipError_t attr = allow_lds(gemm_down_kernel<WT, TT, SC>);
  if (attr != hipSuccess) return attr;
  const int grid = grid_for(items_bound(p, seg_lo, seg_hi, TT, kDnRows, true));
  return launch(gemm_down_kernel<WT, TT, SC>, dim3(grid), dim3(kGThreads), (size_t)kGemmLds,
                stream, start, stop, p, seg_lo, seg_hi, queue_counters(p, seg_lo, true));
}

// Segments of one weight type go through one launch: everything at once when
// the shared expert is stored like the routed ones, else the routed experts
// and then the shared expert.  start/stop go to the launch that holds the
// routed experts.
template <typename Range>
hipError_t by_type(const FfnParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                   Range run) {
  const int E = p.n_experts;
  if (!p.has_shared || p.sw_type == p.w_type) return run(p.w_type, 0, E + p.has_shared, start, stop);
  const hipError_t e = run(p.w_type, 0, E, start, stop);
  if (e != hipSuccess) return e;
  return run(p.sw_type, E, E + 1, nullptr, nullptr);
}

}  // namespace

// Scales in LDS need the scale block of an item to fit its place: H <= 4096
// (gate/up), I <= 2048 (down); scale chunks need 16-byte scale rows and
// whole chunks of four steps: a reduction dimension that is a multiple of
// 512.
// 32-bit offsets into the quantized activations (below 2 GiB: batches up
// to 262144 tokens at H 4096); the larger ones take 64-bit addresses and
// no LDS scales
static bool x_offsets_32(const FfnParams& p) {
  return (int64_t)p.n_tokens * 2 * p.hidden < ((int64_t)1 << 31);
}

// The MXFP4 gate/up of the packed copy writes h as three E2M3 parts (h6)
// for the down to multiply on the 32x32x64 instruction when the batch
// averages at least 16 slots per routed expert; every other grouped-GEMM
// gate/up writes the E4M3 parts (h3).  The 32x32 tiles pay off only when
// the down's items hold more than 16 tokens: with fewer, most of each
// 32-token block is padding and the 16x16x128 form multiplies less (on
// the 6-of-256 layer: equal at 12 slots per expert, the 16x16 form 6 %
// faster at 0.75).  The down's reduction is straight-line code of up to
// 16 steps: intermediate sizes up to 2048.
static bool gate_up_writes_h6(const FfnParams& p) {
  return p.packed && gate_up_writes_h3(p) && x_offsets_32(p) &&
         (int64_t)p.n_tokens * p.top_k >= 16 * (int64_t)p.n_experts && p.inter <= 2048 &&
         (!p.has_shared || p.shared_inter <= 2048);
}

hipError_t launch_gemm_gate_up(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop) {
  const bool sc = p.hidden <= 4096 && p.hidden % 512 == 0;
  const int64_t blocks = (int64_t)p.n_tokens * (p.hidden / 32);
  const hipError_t e = launch(quant_x_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256),
                              0, stream, nullptr, nullptr, p);
  if (e != hipSuccess) return e;
  const bool o32 = x_offsets_32(p);
  const bool h6 = gate_up_writes_h6(p);
  if (h6 && (p.h6 == nullptr || p.h6s == nullptr)) return hipErrorInvalidValue;
  // the h6-writing routed experts and a packed fp8 shared expert: one launch
  if (h6 && p.w_type == MOE_W_MXFP4 && p.has_shared && p.sw_type == MOE_W_FP8E4M3_B128)
    return p.lazy_tau > 0.0f ? gate_up_mix_as<true>(p, stream, start, stop)
                             : gate_up_mix_as<false>(p, stream, start, stop);
  return by_type(p, stream, start, stop, [&](int wt, int lo, int hi, hipEvent_t a, hipEvent_t b) {
    if (wt != MOE_W_MXFP4) {
      if (!o32) return gate_up_range<MOE_W_FP8E4M3_B128, 64, false, false>(p, lo, hi, stream, a, b);
      // packed fp8: only a shared expert (routed experts are packed only as
      // MXFP4), in a launch of its own
      if (p.packed && lo >= p.n_experts)
        return gate_up_range<MOE_W_FP8E4M3_B128, 64, true, true, true>(p, lo, hi, stream, a, b);
      return p.hidden % 512 == 0
                 ? gate_up_range<MOE_W_FP8E4M3_B128, 64, true, true>(p, lo, hi, stream, a, b)
                 : gate_up_range<MOE_W_FP8E4M3_B128, 64, false, true>(p, lo, hi, stream, a, b);
    }
    if (!o32) return gate_up_range<MOE_W_MXFP4, 112, false, false>(p, lo, hi, stream, a, b);
    // the packed copy (its shapes are multiples of 512, and every MXFP4
    // matrix of the launch is in it) needs no LDS scale block, so no bound
    // on H; it writes h6
    if (p.packed && h6)
      return gate_up_range<MOE_W_MXFP4, 112, true, true, true, true>(p, lo, hi, stream, a, b);
    if (p.packed) return gate_up_range<MOE_W_MXFP4, 112, true, true, true>(p, lo, hi, stream, a, b);
    return sc ? gate_up_range<MOE_W_MXFP4, 112, true, true>(p, lo, hi, stream, a, b)
              : gate_up_range<MOE_W_MXFP4, 112, false, true>(p, lo, hi, stream, a, b);
  });
}

hipError_t launch_gemm_down(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop) {
  const bool sc = p.inter <= 2048 && p.inter % 512 == 0 &&
                  (!p.has_shared || (p.shared_inter <= 2048 && p.shared_inter % 512 == 0));
  // h in three E4M3 parts (from the grouped-GEMM gate/up) or as the bf16
  // pair (fp32 x, or the decode gate/up of a small batch with many slots)
  const bool h3 = gate_up_writes_h3(p);
  const bool h6 = gate_up_writes_h6(p);
  if (h6 && (p.h6 == nullptr || p.h6s == nullptr)) return hipErrorInvalidValue;
  // The E2M3 routed down and the packed fp8 shared expert's down in one
  // launch (no launch boundary between the two).
  if (h6 && p.w_type == MOE_W_MXFP4 && p.has_shared && p.sw_type == MOE_W_FP8E4M3_B128)
    return down6_range<true>(p, 0, p.n_experts + 1, stream, start, stop);
  return by_type(p, stream, start, stop, [&](int wt, int lo, int hi, hipEvent_t a, hipEvent_t b) {
    if (wt != MOE_W_MXFP4) {
      // the fp8 segments of this launch: the routed ones, the shared one
      const bool sc8 = (lo >= p.n_experts || p.inter % 512 == 0) &&
                       (hi <= p.n_experts || p.shared_inter % 512 == 0);
      if (h3 && p.packed && lo >= p.n_experts)
        return down3_range<MOE_W_FP8E4M3_B128, true, true>(p, lo, hi, stream, a, b);
      if (h3)
        return sc8 ? down3_range<MOE_W_FP8E4M3_B128, true>(p, lo, hi, stream, a, b)
                   : down3_range<MOE_W_FP8E4M3_B128, false>(p, lo, hi, stream, a, b);
      return sc8 ? down_range<MOE_W_FP8E4M3_B128, 64, true>(p, lo, hi, stream, a, b)
                 : down_range<MOE_W_FP8E4M3_B128, 64, false>(p, lo, hi, stream, a, b);
    }
    if (h6) return down6_range<false>(p, lo, hi, stream, a, b);
    if (h3 && p.packed) return down3_range<MOE_W_MXFP4, true, true>(p, lo, hi, stream, a, b);
    if (h3)
      return sc ? down3_range<MOE_W_MXFP4, true>(p, lo, hi, stream, a, b)
                : down3_range<MOE_W_MXFP4, false>(p, lo, hi, stream, a, b);
    return sc ? down_range<MOE_W_MXFP4, 64, true>(p, lo, hi, stream, a, b)
              : down_range<MOE_W_MXFP4, 64, false>(p, lo, hi, stream, a, b);
  });
}

}  // namespace moe

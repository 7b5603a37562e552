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
// A work item is (segment, row tile, token tile of up to kTileTok slots).  A
// segment is a routed expert (slots offsets[e] .. offsets[e+1]) or the shared
// expert (slot N*k + t is token t).  Items of one row tile are consecutive, so
// the workgroups that multiply the same weights with different token tiles
// run at the same time and share them through the caches.  The grid is
// persistent; every workgroup rebuilds the item prefix from the device-side
// counts (no host synchronisation).
//
// Inside an item each wavefront owns whole output rows over the full
// reduction: no partial sums cross wavefronts.  The reduction runs in steps
// of 128.  The token operand of a step (activation rows gathered through
// perm, or the h rows of the slots) is staged in LDS, double buffered; the
// weight codes of step ks+1 and its token operand are in flight while step ks
// multiplies.
//
// Gate/up: a workgroup owns 128 intermediate rows and up to 128 tokens;
// wavefront w owns rows 32w .. 32w+31 of the gate and of the up matrix
// (four 16-row blocks), so one token fragment read from LDS feeds four
// MFMAs and one decoded weight fragment feeds up to eight token blocks.  The
// epilogue applies SwiGLU and writes h as a bf16 hi/lo pair.
//
// Down: a workgroup owns 256 hidden rows and up to 64 tokens; wavefront w
// owns rows 64w .. 64w+63 (four blocks) and multiplies them with h_hi and
// h_lo.  The epilogue scales each token column by its routing weight (1 for
// the shared expert) and writes the per-slot output; a separate pass sums
// the slots of every token in a fixed order.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_formats.h"
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kGThreads = 256;  // four wavefronts, two workgroups per CU
constexpr int kGWaves = kGThreads / kWave;
constexpr int kGuRows = 32 * kGWaves;  // intermediate rows per gate/up item
constexpr int kDnRows = 64 * kGWaves;  // hidden rows per down item
constexpr int kSegMax = MOE_MAX_EXPERTS + 1;
constexpr int kGemmLds = 72 * 1024;  // dynamic LDS of either kernel (two per CU)
// scale blocks in LDS: after two token tiles of up to five blocks (gate/up,
// 128 rows x H/32 bytes per matrix, H <= 4096) or two h_hi/h_lo pairs of up
// to three blocks (down, 256 rows x I/32 bytes, I <= 2048)
constexpr int kGuScaleOff = 2 * 16 * 5 * 256;
constexpr int kDnScaleOff = 2 * 2 * 16 * 3 * 256;
static_assert(kGuScaleOff + 2 * kGuRows * (4096 / 32) <= kGemmLds, "gate/up LDS");
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

// Token-operand staging: a tile of TT rows x 128 bf16 (256 bytes) per
// reduction step, copied straight from global memory into LDS (no register
// round trip).  One wavefront copy instruction fills four rows: lane l lands
// at byte 16 l of the block.  In round i wavefront w fills rows
// R i + 4w .. +3 (R = 4 * wavefronts), lane l row R i + 4w + (l >> 4),
// 16-byte position l & 15.  Positions are swizzled, chunk c of row n sits at
// position c ^ (n & 15), so the sixteen rows that one fragment read touches
// hit sixteen different bank groups; each lane therefore fetches the chunk
// that belongs at its position.  Only rows below 16 * nbt are copied; rows
// past the tile repeat a valid row: they only feed token columns that the
// epilogue drops.
template <int TT>
struct Stage {
  static constexpr int kRound = 4 * kGWaves;             // rows per round
  static constexpr int kPer = (TT + kRound - 1) / kRound;  // copy rounds
  int row[kPer];                                          // source row per round
  int chunk;                                              // source chunk of this lane

  __device__ static int row_of(int i, int wave, int lane) {
    return kRound * i + 4 * wave + (lane >> 4);
  }
  __device__ void init(int lane) { chunk = (lane & 15) ^ ((4 * wave_id() + (lane >> 4)) & 15); }
  __device__ void copy(const __bf16* base, int64_t stride, int ks, char* buf, int nbt) const {
    const int c = ks * 128 + chunk * 8;
    const int w = wave_id();
    char* dst = buf + (4 * w) * 256;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (kRound * i + 4 * w < 16 * nbt)
        __builtin_amdgcn_global_load_lds(
            base + (int64_t)row[i] * stride + c,
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
// (at most N later loads, the weights of a later step, still in flight),
// then the workgroup barrier.  A plain barrier, not __syncthreads(): its
// release fence would also wait for those later weight loads.  The LDS
// reads of the step are complete here, since the MFMAs consumed them.
template <int N>
__device__ __forceinline__ void step_barrier() {
  wait_vm<N>();
  __builtin_amdgcn_s_barrier();
}

// Workgroups are dealt to the eight XCDs round-robin (workgroup b runs on
// XCD b % 8), and each XCD has its own L2.  The item order is cut into eight
// contiguous chunks, one per XCD: the row tiles of one expert (which share
// its token rows) and the token tiles of one row tile (which share its
// weights) then meet in the same L2.  Returns -1 for the padding indices.
__device__ __forceinline__ int xcd_item(int i, int total) {
  const int per = (total + 7) >> 3;
  const int l = (i & 7) * per + (i >> 3);
  return l < total ? l : -1;
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

// ------------------------------------------------------------- gate/up

// NBT = token blocks of the tile (ceil(m / 16)), a compile-time constant so
// that a step's fragment reads and MFMAs form one branch-free block.
template <int WT, int TT, int NBT, bool SC>
__device__ __forceinline__ void gate_up_item(const FfnParams& p, const GItem& it, char* smem,
                                             int wave, int lane) {
  using F = Fmt<WT>;
  constexpr int Q = F::Q;
  constexpr int TB = NBT;
  // Scale bytes (SC: MXFP4, H a multiple of 512 and at most 4096):
  //  - up to five token blocks: the item's scales sit in LDS (kSC, below);
  //  - six: 16-byte chunks of four steps in registers (kCh, below);
  //  - otherwise (and seven blocks, whose registers are full): one byte per
  //    row and step, loaded with the step's codes.
  constexpr bool kSC = SC && WT == MOE_W_MXFP4 && NBT <= 5;
  constexpr bool kCh = SC && WT == MOE_W_MXFP4 && NBT == 6;
  constexpr int kLoads = (kSC || kCh) ? 4 * Q : 4 * (Q + 1);  // vector loads of one step's weights
  // weights by pairs of steps (below) for up to four token blocks and an
  // even number of steps
  constexpr bool kPair = kSC && NBT <= 4;
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
  const int64_t lc = lrow * cb + F::code_off(0, g), ls = lrow * sb + F::scale_off(0, g);
  const uint8_t* cbase[2] = {shared ? p.sgate_c : p.gate_c, shared ? p.sup_c : p.up_c};
  const uint8_t* sbase[2] = {shared ? p.sgate_s : p.gate_s, shared ? p.sup_s : p.up_s};

  // activation rows copied by this lane (rows past the tile repeat row 0)
  Stage<TT> st;
  st.init(lane);
  {
    // all perm loads first (clamped into perm; the shared expert needs none)
    int pv[Stage<TT>::kPer];
#pragma unroll
    for (int i = 0; i < Stage<TT>::kPer; ++i) {
      const int n = Stage<TT>::row_of(i, wave, lane);
      pv[i] = p.perm[min(it.slot0 + (n < it.m ? n : 0), nk - 1)];
    }
#pragma unroll
    for (int i = 0; i < Stage<TT>::kPer; ++i) {
      const int n = Stage<TT>::row_of(i, wave, lane);
      const int slot = it.slot0 + (n < it.m ? n : 0);
      st.row[i] = shared ? slot - nk : pv[i] / p.top_k;
    }
  }
  const __bf16* xb = static_cast<const __bf16*>(p.x);

  // weight codes: the current step and the next two
  u32x4 q0[2][2][Q], q1[2][2][Q], q2[2][2][Q];
  uint32_t u0[2][2], u1[2][2], u2[2][2];
  auto load_w = [&](int ks, u32x4 (&q)[2][2][Q], uint32_t (&u)[2][2]) {
    const int k = min(ks, nks - 1);  // past the end: reload the last step
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int i = 0; i < Q; ++i)
          q[mat][rb][i] = load16(cbase[mat] + lc + 16 * rb * cb + F::code_off(k, 0) + 16 * i);
        if (!kSC && !kCh) u[mat][rb] = sbase[mat][ls + 16 * rb * sb + F::scale_off(k, 0)];
      }
  };
  // scale chunks (kCh): the 16 scale bytes of steps 4c .. 4c+3 of a row in
  // one load shared by the row's four lanes, once per four steps; the lane
  // keeps its own byte of each of the four steps in sp.  (Their lines can
  // leave the L2 between two loads, so this costs re-fetches that the LDS
  // copy avoids; it is the fallback where that copy does not fit.)
  u32x4 scw[2][2];
  uint32_t sp[2][2];
  const int64_t srow = ls - F::scale_off(0, g);
  auto load_sc = [&](int c) {
    const int cc = min(c, nks / 4 - 1);
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        scw[mat][rb] = load16(sbase[mat] + srow + 16 * rb * sb + 16 * cc);
  };
  auto take_sc = [&]() {
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) v |= ((scw[mat][rb][t] >> (8 * g)) & 0xFFu) << (8 * t);
        sp[mat][rb] = v;
      }
  };
  // scales (kSC): the item's 128 rows of each matrix are consecutive, so
  // their scale bytes are one contiguous block (128 * H/32 bytes), copied
  // into LDS at the start of the item (1 KiB per copy instruction) and read
  // from there at every step.  Loaded from memory per step (one byte per
  // row) they doubled the weight stream's requests; loaded per four steps
  // (16 bytes) the lines left the L2 between loads and were fetched up to
  // eight times each.
  constexpr int kTokB = kSC ? 16 * NBT * 256 : TT * 256;  // bytes of one token tile
  char* const sscale = smem + kGuScaleOff;                // [mat][128 rows][sb]
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

  // buffer b at smem + b * TT * 256 (offsets from smem keep LDS addressing)
  auto buf = [&](int b) { return smem + (b & 1) * kTokB; };
  // one reduction step: step ks's weights qq (and their scale bytes uu, when
  // not chunked) times the token tile in LDS
  auto step_mma = [&](int ks, const u32x4 (&qq)[2][2][Q], const uint32_t (&uu)[2][2]) {
    const char* cur = buf(ks);
    float sc[2][2];
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        sc[mat][rb] = ue8m0_to_f32(kSC   ? scale_byte(mat, rb, ks)
                                   : kCh ? (sp[mat][rb] >> (8 * (ks & 3))) & 0xFFu
                                         : uu[mat][rb]);
    // sub-step j+1 is decoded while sub-step j multiplies, so the converts
    // overlap the matrix-core work
    bf16x8 a[2][2][2];
#pragma unroll
    for (int mat = 0; mat < 2; ++mat)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) a[0][mat][rb] = F::decode_j(qq[mat][rb], sc[mat][rb], 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j + 1 < 4) {
#pragma unroll
        for (int mat = 0; mat < 2; ++mat)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            a[(j + 1) & 1][mat][rb] = F::decode_j(qq[mat][rb], sc[mat][rb], j + 1);
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const bf16x8 b = token_frag(cur, tb, j, g, r16);
#pragma unroll
        for (int mat = 0; mat < 2; ++mat)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[mat][rb][tb] = mfma_bf16(a[j & 1][mat][rb], b, acc[mat][rb][tb]);
      }
      // keep two sub-steps' fragments live at a time
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (kSC) copy_scales();
  if (kCh) load_sc(0);
  load_w(0, q0, u0);
  load_w(1, q1, u1);
  st.copy(xb, p.hidden, 0, buf(0), nbt);
  wait_vm<0>();
  __syncthreads();
  const bool paired = kPair && (nks & 1) == 0;
  if (paired) {
    // weights by pairs of steps: the two halves of each 128-byte line of a
    // row (steps 2c and 2c+1) are requested together.  Requested one step
    // apart, about 40 % of the lines left the L2 in between and were fetched
    // twice.  q0/q1 hold pair c, q2/q3 receive pair c+1 during step 2c.
    u32x4 q3[2][2][Q];
    uint32_t u3[2][2];
    for (int ks = 0; ks < nks; ks += 2) {
      st.copy(xb, p.hidden, ks + 1, buf(ks + 1), nbt);
      __builtin_amdgcn_sched_barrier(0);
      load_w(ks + 2, q2, u2);
      load_w(ks + 3, q3, u3);
      __builtin_amdgcn_sched_barrier(0);
      step_mma(ks, q0, u0);
      step_barrier<2 * kLoads>();  // step ks+1's tile has landed
      if (ks + 2 < nks) st.copy(xb, p.hidden, ks + 2, buf(ks + 2), nbt);
      __builtin_amdgcn_sched_barrier(0);
      step_mma(ks + 1, q1, u1);
      step_barrier<0>();  // step ks+2's tile and pair c+1 have landed
#pragma unroll
      for (int mat = 0; mat < 2; ++mat)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < Q; ++i) {
            q0[mat][rb][i] = q2[mat][rb][i];
            q1[mat][rb][i] = q3[mat][rb][i];
          }
    }
  } else {
    for (int ks = 0; ks < nks; ++ks) {
      // every fourth step (kCh): this chunk's scales out of the load
      // registers, then the next chunk's requested (before the step's other
      // loads, so that the end-of-step wait below still counts only the
      // weights after the copy)
      if (kCh && (ks & 3) == 0) {
        take_sc();
        load_sc((ks >> 2) + 1);
      }
      // step ks+1's activations, then step ks+2's weights: the end-of-step
      // wait lets the weights stay in flight
      if (ks + 1 < nks) st.copy(xb, p.hidden, ks + 1, buf(ks + 1), nbt);
      __builtin_amdgcn_sched_barrier(0);
      load_w(ks + 2, q2, u2);
      __builtin_amdgcn_sched_barrier(0);
      step_mma(ks, q0, u0);
      step_barrier<kLoads>();
#pragma unroll
      for (int mat = 0; mat < 2; ++mat)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
          for (int i = 0; i < Q; ++i) {
            q0[mat][rb][i] = q1[mat][rb][i];
            q1[mat][rb][i] = q2[mat][rb][i];
          }
          u0[mat][rb] = u1[mat][rb];
          u1[mat][rb] = u2[mat][rb];
        }
    }
  }
  wait_vm<0>();  // the reloads past the end

  // SwiGLU; lane holds rows 4g .. 4g+3 of each block for token column r16
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int n = tb * 16 + r16;
      if (live && tb < nbt && n < it.m) {
        bf16x4 hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = acc[0][rb][tb][r];
          const float h = gv / (1.0f + expf(-gv)) * acc[1][rb][tb][r];
          __bf16 x, y;
          split_bf16(h, x, y);
          hi[r] = x;
          lo[r] = y;
        }
        const int64_t o =
            (int64_t)(it.slot0 + n) * p.h_stride + it.row0 + 32 * wave + 16 * rb + 4 * g;
        *reinterpret_cast<bf16x4*>(p.h_hi + o) = hi;
        *reinterpret_cast<bf16x4*>(p.h_lo + o) = lo;
      }
    }
}

template <int WT, int TT, bool SC>
__global__ __launch_bounds__(kGThreads, 2) void gemm_gate_up_kernel(FfnParams p, int seg_lo,
                                                                     int seg_hi) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_pref[kSegMax + 1];
  __shared__ int s_tmp[kGThreads / kWave];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int total = item_prefix<TT, kGuRows, false>(p, seg_lo, seg_hi, s_pref, s_tmp);
  const int slots = (total + 7) & ~7;
  for (int i = blockIdx.x; i < slots; i += gridDim.x) {
    const int item = xcd_item(i, total);
    if (item < 0) continue;
    const GItem it = find_item<TT, kGuRows, false>(p, seg_lo, seg_hi, s_pref, item);
    dispatch_nbt<TT / 16>((it.m + 15) >> 4, [&](auto nb) {
      gate_up_item<WT, TT, decltype(nb)::value, SC>(p, it, smem, wave, lane);
    });
    __syncthreads();  // the LDS tiles are reused by the next item
  }
}

// ------------------------------------------------------------- down

template <int WT, int TT, int NBT, bool SC>
__device__ __forceinline__ void down_item(const FfnParams& p, const GItem& it, char* smem,
                                          int wave, int lane) {
  using F = Fmt<WT>;
  constexpr int Q = F::Q;
  constexpr int TB = NBT;
  constexpr int RB = kDnRows / (16 * kGWaves);  // row blocks per wavefront
  // scale bytes as in gate/up (SC: I a multiple of 512 and at most 2048):
  // in LDS for up to three token blocks (kSC), in 16-byte chunks for four
  constexpr bool kSC = SC && WT == MOE_W_MXFP4 && NBT <= 3;
  constexpr bool kCh = SC && WT == MOE_W_MXFP4 && NBT == 4;
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

  // the lane's row in block 0 (blocks past the matrix end reuse it and are
  // not multiplied)
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

  // routing weight of each token column, fetched now, used by the epilogue
  float wcol[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int n = min(tb * 16 + r16, it.m - 1);
    wcol[tb] = shared ? 1.0f : p.topk_w[p.perm[it.slot0 + n]];
  }

  u32x4 q0[RB][Q], q1[RB][Q], q2[RB][Q];
  uint32_t u0[RB], u1[RB], u2[RB];
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
      scw[rb] = load16(sbase + srow + 16 * rr * sb + 16 * cc);
    }
  };
  auto take_sc = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      uint32_t v = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) v |= ((scw[rb][t] >> (8 * g)) & 0xFFu) << (8 * t);
      sp[rb] = v;
    }
  };
  // scales (kSC), as in gate/up: the item's rows (up to 256, fewer in the
  // last tile of the matrix) as one contiguous block in LDS
  constexpr int kTokB = kSC ? 16 * NBT * 256 : TT * 256;  // bytes of one h tile
  char* const sscale = smem + kDnScaleOff;                // [256 rows][sb]
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
  load_w(1, q1, u1);
  st.copy(p.h_hi, p.h_stride, 0, bh(0), nbt);
  st.copy(p.h_lo, p.h_stride, 0, bl(0), nbt);
  wait_vm<0>();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    if (kCh && (ks & 3) == 0) {
      take_sc();
      load_sc((ks >> 2) + 1);
    }
    if (ks + 1 < nks) {
      st.copy(p.h_hi, p.h_stride, ks + 1, bh(ks + 1), nbt);
      st.copy(p.h_lo, p.h_stride, ks + 1, bl(ks + 1), nbt);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_w(ks + 2, q2, u2);
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
          if (rb < nrb) {
            acc[rb][tb] = mfma_bf16(a[j & 1][rb], fh, acc[rb][tb]);
            acc[rb][tb] = mfma_bf16(a[j & 1][rb], fl, acc[rb][tb]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    step_barrier<kLoads>();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        q0[rb][i] = q1[rb][i];
        q1[rb][i] = q2[rb][i];
      }
      u0[rb] = u1[rb];
      u1[rb] = u2[rb];
    }
  }
  wait_vm<0>();

  // routing weight of each token column, then the per-slot outputs
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int n = tb * 16 + r16;
    if (tb < nbt && n < it.m) {
      const int64_t slot = it.slot0 + n;
      const float w = wcol[tb];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb < nrb) {
          *reinterpret_cast<f32x4*>(p.obuf + slot * p.hidden + wrow0 + 16 * rb + 4 * g) =
              acc[rb][tb] * w;
        }
      }
    }
  }
}

template <int WT, int TT, bool SC>
__global__ __launch_bounds__(kGThreads, 2) void gemm_down_kernel(FfnParams p, int seg_lo,
                                                                  int seg_hi) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_pref[kSegMax + 1];
  __shared__ int s_tmp[kGThreads / kWave];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int total = item_prefix<TT, kDnRows, true>(p, seg_lo, seg_hi, s_pref, s_tmp);
  const int slots = (total + 7) & ~7;
  for (int i = blockIdx.x; i < slots; i += gridDim.x) {
    const int item = xcd_item(i, total);
    if (item < 0) continue;
    const GItem it = find_item<TT, kDnRows, true>(p, seg_lo, seg_hi, s_pref, item);
    dispatch_nbt<TT / 16>((it.m + 15) >> 4, [&](auto nb) {
      down_item<WT, TT, decltype(nb)::value, SC>(p, it, smem, wave, lane);
    });
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

constexpr int kGemmGrid = 256 * 2;  // 256 CUs, two workgroups each

int grid_for(int64_t items) {
  return (int)(items < kGemmGrid ? (items > 0 ? items : 1) : kGemmGrid);
}

template <int WT, int TT, bool SC>
hipError_t gate_up_range(const FfnParams& p, int seg_lo, int seg_hi, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop) {
  static const hipError_t attr = allow_lds(gemm_gate_up_kernel<WT, TT, SC>);
  if (attr != hipSuccess) return attr;
  const int grid = grid_for(items_bound(p, seg_lo, seg_hi, TT, kGuRows, false));
  return launch(gemm_gate_up_kernel<WT, TT, SC>, dim3(grid), dim3(kGThreads),
                (size_t)kGemmLds, stream, start, stop, p, seg_lo, seg_hi);
}

template <int WT, int TT, bool SC>
hipError_t down_range(const FfnParams& p, int seg_lo, int seg_hi, hipStream_t stream,
                      hipEvent_t start, hipEvent_t stop) {
  static const hipError_t attr = allow_lds(gemm_down_kernel<WT, TT, SC>);
  if (attr != hipSuccess) return attr;
  const int grid = grid_for(items_bound(p, seg_lo, seg_hi, TT, kDnRows, true));
  return launch(gemm_down_kernel<WT, TT, SC>, dim3(grid), dim3(kGThreads), (size_t)kGemmLds,
                stream, start, stop, p, seg_lo, seg_hi);
}

// Segments of one weight type go through one launch: everything at once when
// the shared expert is stored like the routed ones, else the routed experts
// and then the shared expert.
template <typename Range>
hipError_t by_type(const FfnParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                   Range run) {
  const int E = p.n_experts;
  if (!p.has_shared || p.sw_type == p.w_type) return run(p.w_type, 0, E + p.has_shared, start, stop);
  const hipError_t e = run(p.w_type, 0, E, start, nullptr);
  if (e != hipSuccess) return e;
  return run(p.sw_type, E, E + 1, nullptr, stop);
}

}  // namespace

// Scales in LDS need the scale block of an item to fit its place: H <= 4096
// (gate/up), I <= 2048 (down); scale chunks need 16-byte scale rows and
// whole chunks of four steps: a reduction dimension that is a multiple of
// 512.
hipError_t launch_gemm_gate_up(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop) {
  const bool sc = p.hidden <= 4096 && p.hidden % 512 == 0;
  return by_type(p, stream, start, stop, [&](int wt, int lo, int hi, hipEvent_t a, hipEvent_t b) {
    if (wt != MOE_W_MXFP4) return gate_up_range<MOE_W_FP8E4M3_B128, 64, false>(p, lo, hi, stream, a, b);
    return sc ? gate_up_range<MOE_W_MXFP4, 112, true>(p, lo, hi, stream, a, b)
              : gate_up_range<MOE_W_MXFP4, 112, false>(p, lo, hi, stream, a, b);
  });
}

hipError_t launch_gemm_down(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop) {
  const bool sc = p.inter <= 2048 && p.inter % 512 == 0 &&
                  (!p.has_shared || (p.shared_inter <= 2048 && p.shared_inter % 512 == 0));
  return by_type(p, stream, start, stop, [&](int wt, int lo, int hi, hipEvent_t a, hipEvent_t b) {
    if (wt != MOE_W_MXFP4) return down_range<MOE_W_FP8E4M3_B128, 64, false>(p, lo, hi, stream, a, b);
    return sc ? down_range<MOE_W_MXFP4, 64, true>(p, lo, hi, stream, a, b)
              : down_range<MOE_W_MXFP4, 64, false>(p, lo, hi, stream, a, b);
  });
}

}  // namespace moe

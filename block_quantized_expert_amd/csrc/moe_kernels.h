// Internal launch interface between the C ABI (moe_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Everything the FFN kernels read, passed by value.
struct FfnParams {
  int n_tokens;
  int top_k;
  int n_experts;
  int hidden;
  int inter;         // routed intermediate size
  int shared_inter;  // shared intermediate size (0 without a shared expert)
  int has_shared;
  int w_type;   // routed weight type (moe_weight_type)
  int sw_type;  // shared weight type
  int x_f32;    // activations are fp32 (else bf16)
  const uint8_t *gate_c, *gate_s, *up_c, *up_s, *down_c, *down_s;
  const uint8_t *sgate_c, *sgate_s, *sup_c, *sup_s, *sdown_c, *sdown_s;
  const void* x;
  const float* topk_w;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* inv_perm;
  // bf16 activations of the grouped-GEMM path as two E4M3 parts:
  // xq [n_tokens][hidden/128][256] (per 128 inputs 128 hi bytes, 128 lo
  // bytes), xs [n_tokens][hidden/32][2] (their UE8M0 scale bytes)
  uint8_t* xq;
  uint8_t* xs;
  __bf16* h_hi;  // [slots][h_stride]
  __bf16* h_lo;
  int64_t h_stride;
  // grouped-GEMM path with bf16 x: h as three E4M3 parts in place of the
  // pair, h3 [slots][h_stride/128][3][128] (per 128 inputs the three parts'
  // bytes), h3s [slots][h_stride/32][4] (their UE8M0 scale bytes s, s-4,
  // s-8 and a zero byte)
  uint8_t* h3;
  uint8_t* h3s;
  // packed MXFP4 batches: h as three E2M3 parts for the 32x32x64 down,
  // 32-row-block major: h6 [h_stride/32][slots][3 parts][24 B] (part q of
  // the 32 values of block kb of a slot, 6 bits each, value i at bits
  // 6i .. 6i+5), h6s [h_stride/32][slots] (the parts' UE8M0 scale bytes in
  // bytes 0..2), 16 bytes of padding after h6; null unless the routed
  // experts are MXFP4 and the batch has at least 16 slots per expert
  uint8_t* h6;
  uint32_t* h6s;
  int64_t n_slots;  // N*k + N with a shared expert
  // [slots][hidden / 4][3 words] per-slot outputs, four features as 24-bit
  // floats in three words (store_f24x4); the combine weights them
  uint32_t* obuf;
  float* y;     // [n_tokens][hidden]
  // gate-first lazy skip: a routed slot whose gate output has
  // max_j |SiLU(g_j)| < lazy_tau contributes nothing (lazy_tau 0: off).
  // gmax [n_tokens*top_k] holds that maximum per slot (fp32 bits, zeroed
  // before the gate/up pass); gbuf [n_tokens*top_k][inter] the gate outputs
  // of the small-batch gate-first path
  float lazy_tau;
  uint32_t* gmax;
  float* gbuf;
  // the grouped GEMMs' item-queue counters, kQueueWords of them
  uint32_t* qctr;
  // packed copy of the MXFP4 matrices (moe_pack_experts), indexed gate, up,
  // down, shared gate, shared up, shared down; null when not packed
  const uint8_t* pk_c[6];
  const uint8_t* pk_s[6];
  bool packed;
};

constexpr int kQueueWords = 32;  // 4 launches x 8 XCD chunks

// Options of the learned router beyond plain top-k (moe_opts of the C ABI,
// checked on the host): expert groups with a selection-only bias, and tail
// pruning of the chosen experts.  plain(top_k) asks for neither.
struct RouteOpts {
  int n_group;        // >= 1; 1 = one group
  int topk_group;     // 1..n_group
  const float* bias;  // nullable, [n_experts]
  int keep_max;       // 1..top_k
  float min_w;        // >= 0
  static RouteOpts plain(int top_k) { return RouteOpts{1, 1, nullptr, top_k, 0.0f}; }
};

// Synchronisation words of the fused single-token decode (in the caller's
// workspace, zeroed once).  `launch` counts the kernel's launches on this
// workspace: a launch reads it at its start, uses launch + 1 as its epoch
// and stores that back once its grid barrier is over, so every launch has a
// new epoch without the host (a launch captured in a graph and replayed
// included).  arrive[b] holds the epoch of the launch whose workgroup b last
// arrived.
struct FusedSync {
  static constexpr int kMaxGrid = 1023;  // one workgroup per compute unit
  unsigned long long launch;
  unsigned long long arrive[kMaxGrid];
};

// The fused single-token decode (route + group + FFN in one kernel).  The
// routing outputs are written by the kernel; p's topk_w, counts, offsets,
// perm and inv_perm are not read.
struct FusedParams {
  FfnParams p;
  const float* logits;
  float routed_scale;
  RouteOpts ropts;
  int route_opts;  // 0: plain top-k on the logits; 1: ropts applies
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  FusedSync* sync;
  unsigned long long wait_xor;    // 0; a test sets a bit so that the barrier waits for
                                  // a value no workgroup posts (the give-up path)
  uint32_t spin_limit;            // polls of the flags before giving up
  int32_t* dev_error;             // nullable
  int grid;                       // set by the launcher
};

hipError_t launch_route(const float* logits, int n_tokens, int n_experts, int top_k,
                        float routed_scale, const RouteOpts& opts, int32_t* ids, float* w,
                        hipStream_t stream);
hipError_t launch_route_hash(const int32_t* token_ids, int n_tokens, const int32_t* tid2eid,
                             const float* tid2w, int vocab, int n_experts, int top_k,
                             int32_t* ids, float* w, int32_t* dev_error, hipStream_t stream);
hipError_t launch_group(const int32_t* ids, int n_tokens, int top_k, int n_experts,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        int32_t* dev_error, hipStream_t stream);
hipError_t launch_route_group(const float* logits, int n_tokens, int n_experts, int top_k,
                              float routed_scale, const RouteOpts& opts, int32_t* ids, float* w,
                              int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, int32_t* dev_error, hipStream_t stream);
// start/stop may be null; when given they record the kernel's own start and
// end times (taken from its dispatch, no extra packets on the stream)
hipError_t launch_ffn_gate_up(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                              hipEvent_t stop);
hipError_t launch_ffn_down(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop);
// steps per wavefront quarter (hidden/512) when the fused single-token
// decode applies to p (n_tokens == 1 and the formats it covers), else 0
int fused_decode_steps(const FfnParams& p);
hipError_t launch_decode_fused(const FusedParams& f, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop);
// true if launch_ffn_gate_up stores h as three E4M3 parts (h3, h3s: the
// grouped-GEMM gate/up), false if as the bf16 pair (h_hi, h_lo)
bool gate_up_writes_h3(const FfnParams& p);
// grouped-GEMM kernels for batches in which experts see many tokens
hipError_t launch_gemm_gate_up(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                               hipEvent_t stop);
hipError_t launch_gemm_down(const FfnParams& p, hipStream_t stream, hipEvent_t start,
                            hipEvent_t stop);

}  // namespace moe

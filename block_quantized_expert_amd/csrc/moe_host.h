// Host-side argument checks and workspace planning for the moe_* entry
// points.  Pure host C++: no HIP call is made here, so every rule can be
// exercised without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Byte layout of the moe_ffn workspace.
//   h_hi, h_lo : bf16 [slots][h_stride]   SwiGLU output split into a bf16
//                                         high part and a bf16 low part
//   obuf       : [slots][hidden] x 3 B    expert outputs before the routing
//                                         weight, 24-bit floats (used when the
//                                         batch is too large for the
//                                         single-pass down + combine)
//   xq         : u8 [n_tokens][2*hidden]  bf16 activations as E4M3 hi and lo
//                                         parts (grouped-GEMM gate/up)
//   xs         : u8 [n_tokens][hidden/16] their scale bytes
//   h3, h3s    : at off_h_hi, in place of h_hi/h_lo on the grouped-GEMM
//                path with bf16 x: h as three E4M3 parts
//                u8 [slots][h_stride/128][3][128] and their scale bytes
//                u8 [slots][h_stride/32][4]
//   gmax       : u32 [n_tokens*top_k]      gate-first lazy skip: the largest
//                                         |SiLU(g)| of each routed slot (fp32
//                                         bits)
//   qctr       : u32 [32]                  the grouped GEMMs' item-queue
//                                         counters (256 bytes)
//   gbuf       : fp32 [n_tokens*top_k][inter]  gate outputs kept between the
//                                         gate and up passes of the small-batch
//                                         lazy path (batches of up to
//                                         kGateFirstMaxTokens tokens; else
//                                         empty)
//   h6, h6s    : MXFP4 layers, batches of at least 16 slots per routed
//                expert: h as three E2M3 parts for the down of a layer
//                with the packed copy, u8 [h_stride/32][slots][3][24] (+16
//                bytes of padding) and their scale words u32
//                [h_stride/32][slots]
// A slot is one (token, routed expert) pair in grouped order
// (p in [0, n_tokens*top_k)) or, for the shared expert, n_tokens*top_k + t.
struct FfnPlan {
  int64_t slots;
  int64_t h_stride;
  size_t off_h_hi;
  size_t off_h_lo;
  size_t off_obuf;
  size_t off_xq;
  size_t off_xs;
  size_t off_h3s;
  size_t off_gmax;
  size_t off_gbuf;
  size_t off_qctr;
  size_t off_h6;   // 0 bytes unless the routed experts are MXFP4 and the batch large
  size_t off_h6s;
  size_t total;
};

// Batches up to this many tokens keep the gate outputs for a gate-first pass.
constexpr int kGateFirstMaxTokens = 16;

// moe_opts checked and with its defaults filled in.
struct OptsPlan {
  int n_group;
  int topk_group;
  const float* bias;
  int keep_max;
  float min_w;
  float lazy_tau;
};
// opts may be NULL (no options); the layer's n_experts and top_k, or a
// router's, bound the group and pruning parameters.
moe_status check_opts(const moe_opts* opts, int n_experts, int top_k, OptsPlan* out);

moe_status check_route_group(const float* logits, int n_tokens, int n_experts, int top_k,
                             float routed_scale, const int32_t* ids, const float* w,
                             const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                             const int32_t* inv_perm);
moe_status check_route(const float* logits, int n_tokens, int n_experts, int top_k,
                       float routed_scale, const int32_t* ids, const float* w);
moe_status check_route_hash(const int32_t* token_ids, int n_tokens, const int32_t* tid2eid,
                            const float* tid2w, int vocab, int n_experts, int top_k,
                            const int32_t* ids, const float* w);
moe_status check_group(const int32_t* ids, int n_tokens, int top_k, int n_experts,
                       const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                       const int32_t* inv_perm);
moe_status check_layer(const moe_layer* layer);

// Layout of a packed copy (moe_pack_experts): per matrix (gate, up, down,
// shared gate, shared up, shared down) the byte offset of its codes and of
// its scales, or -1 for a matrix that is not packed (no shared expert);
// rows, inputs and weight type of each matrix.
struct PackPlan {
  int64_t codes[6];
  int64_t scales[6];
  int64_t rows[6];
  int32_t cols[6];
  int32_t type[6];
  size_t total;
};
// MOE_OK with the plan for a layer that passed check_layer and can be
// packed; MOE_ERR_UNSUPPORTED otherwise.
moe_status plan_pack(const moe_layer* layer, PackPlan* plan);
// Fills `plan` for a valid layer; the layer must have passed check_layer.
moe_status plan_ffn(const moe_layer* layer, int n_tokens, FfnPlan* plan);
// Byte layout of the moe_forward workspace.
//   sync    : [0, MOE_FORWARD_SYNC_BYTES)  the flags of the single-token
//             kernel (FusedSync in moe_kernels.h)
//   ffn     : the moe_ffn workspace (FfnPlan), at off_ffn
struct ForwardPlan {
  FfnPlan ffn;
  size_t off_ffn;
  size_t total;
};
moe_status plan_forward(const moe_layer* layer, int n_tokens, ForwardPlan* plan);
moe_status check_forward(const moe_layer* layer, const float* logits, float routed_scale,
                         const void* x, int x_type, int n_tokens, const int32_t* ids,
                         const float* w, const int32_t* counts, const int32_t* offsets,
                         const int32_t* perm, const int32_t* inv_perm, const float* y,
                         const void* workspace, size_t workspace_bytes, ForwardPlan* plan);
moe_status check_ffn(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                     const float* topk_w, const int32_t* counts, const int32_t* offsets,
                     const int32_t* perm, const int32_t* inv_perm, const float* y,
                     const void* workspace, size_t workspace_bytes, FfnPlan* plan);

}  // namespace moe

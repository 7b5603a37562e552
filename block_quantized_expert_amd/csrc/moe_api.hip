// The extern "C" entry points of libmoe.so (declared in include/moe.h):
// validate on the host, then enqueue the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include "moe.h"
#include "moe_host.h"
#include "moe_kernels.h"

namespace {

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

moe::FfnParams make_params(const moe_layer* L, const void* x, int x_type, int n_tokens,
                           const float* topk_w, const int32_t* counts, const int32_t* offsets,
                           const int32_t* perm, const int32_t* inv_perm, float* y,
                           void* workspace, const moe::FfnPlan& plan) {
  moe::FfnParams p{};
  p.n_tokens = n_tokens;
  p.top_k = L->top_k;
  p.n_experts = L->n_experts;
  p.hidden = L->hidden;
  p.inter = L->inter;
  p.has_shared = L->has_shared;
  p.shared_inter = L->has_shared ? L->shared_inter : 0;
  p.w_type = L->gate.type;
  p.sw_type = L->has_shared ? L->shared_gate.type : MOE_W_MXFP4;
  p.x_f32 = x_type == MOE_ACT_F32;
  p.gate_c = L->gate.codes;
  p.gate_s = L->gate.scales;
  p.up_c = L->up.codes;
  p.up_s = L->up.scales;
  p.down_c = L->down.codes;
  p.down_s = L->down.scales;
  if (L->has_shared) {
    p.sgate_c = L->shared_gate.codes;
    p.sgate_s = L->shared_gate.scales;
    p.sup_c = L->shared_up.codes;
    p.sup_s = L->shared_up.scales;
    p.sdown_c = L->shared_down.codes;
    p.sdown_s = L->shared_down.scales;
  }
  p.x = x;
  p.topk_w = topk_w;
  p.counts = counts;
  p.offsets = offsets;
  p.perm = perm;
  p.inv_perm = inv_perm;
  char* ws = static_cast<char*>(workspace);
  p.h_hi = reinterpret_cast<__bf16*>(ws + plan.off_h_hi);
  p.h_lo = reinterpret_cast<__bf16*>(ws + plan.off_h_lo);
  p.h_stride = plan.h_stride;
  p.obuf = reinterpret_cast<float*>(ws + plan.off_obuf);
  p.y = y;
  return p;
}

enum Stage { kGateUp = 1, kDown = 2, kBoth = 3 };

moe_status ffn_stages(int stages, const moe_layer* layer, const void* x, int x_type,
                      int n_tokens, const float* topk_w, const int32_t* counts,
                      const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm,
                      float* y, void* workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t const* events = nullptr) {
  moe::FfnPlan plan;
  moe_status s = moe::check_ffn(layer, x, x_type, n_tokens, topk_w, counts, offsets, perm,
                                inv_perm, y, workspace, workspace_bytes, &plan);
  if (s != MOE_OK || n_tokens == 0) return s;
  const moe::FfnParams p = make_params(layer, x, x_type, n_tokens, topk_w, counts, offsets, perm,
                                       inv_perm, y, workspace, plan);
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  if (events)
    for (int i = 0; i < 4; ++i) ev[i] = events[i];
  if (stages & kGateUp) {
    if ((s = launched(moe::launch_ffn_gate_up(p, stream, ev[0], ev[1]))) != MOE_OK) return s;
  }
  if (stages & kDown) {
    if ((s = launched(moe::launch_ffn_down(p, stream, ev[2], ev[3]))) != MOE_OK) return s;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_route(const float* logits, int n_tokens, int n_experts, int top_k,
                     float routed_scale, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream) {
  moe_status s = moe::check_route(logits, n_tokens, n_experts, top_k, routed_scale, topk_ids,
                                  topk_w);
  if (s != MOE_OK || n_tokens == 0) return s;
  return launched(moe::launch_route(logits, n_tokens, n_experts, top_k, routed_scale, topk_ids,
                                    topk_w, stream));
}

moe_status moe_route_hash(const int32_t* token_ids, int n_tokens, const int32_t* tid2eid,
                          const float* tid2w, int vocab, int n_experts, int top_k,
                          int32_t* topk_ids, float* topk_w, int32_t* dev_error,
                          hipStream_t stream) {
  moe_status s = moe::check_route_hash(token_ids, n_tokens, tid2eid, tid2w, vocab, n_experts,
                                       top_k, topk_ids, topk_w);
  if (s != MOE_OK || n_tokens == 0) return s;
  return launched(moe::launch_route_hash(token_ids, n_tokens, tid2eid, tid2w, vocab, n_experts,
                                         top_k, topk_ids, topk_w, dev_error, stream));
}

moe_status moe_route_group(const float* logits, int n_tokens, int n_experts, int top_k,
                           float routed_scale, int32_t* topk_ids, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                           int32_t* dev_error, hipStream_t stream) {
  moe_status s = moe::check_route_group(logits, n_tokens, n_experts, top_k, routed_scale,
                                        topk_ids, topk_w, counts, offsets, perm, inv_perm);
  if (s != MOE_OK) return s;
  return launched(moe::launch_route_group(logits, n_tokens, n_experts, top_k, routed_scale,
                                          topk_ids, topk_w, counts, offsets, perm, inv_perm,
                                          dev_error, stream));
}

size_t moe_group_workspace_bytes(int n_tokens, int top_k, int n_experts) {
  (void)n_tokens;
  (void)top_k;
  (void)n_experts;
  return 0;
}

moe_status moe_group(const int32_t* topk_ids, int n_tokens, int top_k, int n_experts,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                     int32_t* dev_error, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  moe_status s = moe::check_group(topk_ids, n_tokens, top_k, n_experts, counts, offsets, perm,
                                  inv_perm);
  if (s != MOE_OK) return s;
  // also for n_tokens == 0: counts and offsets are then written as zeros
  return launched(moe::launch_group(topk_ids, n_tokens, top_k, n_experts, counts, offsets, perm,
                                    inv_perm, dev_error, stream));
}

size_t moe_ffn_workspace_bytes(const moe_layer* layer, int n_tokens) {
  moe::FfnPlan plan;
  if (moe::check_layer(layer) != MOE_OK) return 0;
  if (moe::plan_ffn(layer, n_tokens, &plan) != MOE_OK) return 0;
  return plan.total;
}

moe_status moe_ffn_forward(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                           const float* topk_w, const int32_t* counts, const int32_t* offsets,
                           const int32_t* perm, const int32_t* inv_perm, float* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ffn_stages(kBoth, layer, x, x_type, n_tokens, topk_w, counts, offsets, perm, inv_perm,
                    y, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_gate_up(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                           const float* topk_w, const int32_t* counts, const int32_t* offsets,
                           const int32_t* perm, const int32_t* inv_perm, float* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ffn_stages(kGateUp, layer, x, x_type, n_tokens, topk_w, counts, offsets, perm,
                    inv_perm, y, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_down(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                        const float* topk_w, const int32_t* counts, const int32_t* offsets,
                        const int32_t* perm, const int32_t* inv_perm, float* y,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ffn_stages(kDown, layer, x, x_type, n_tokens, topk_w, counts, offsets, perm, inv_perm,
                    y, workspace, workspace_bytes, stream);
}

moe_status moe_ffn_forward_timed(const moe_layer* layer, const void* x, int x_type,
                                 int n_tokens, const float* topk_w, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* perm,
                                 const int32_t* inv_perm, float* y, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t gate_up_start, hipEvent_t gate_up_stop,
                                 hipEvent_t down_start, hipEvent_t down_stop) {
  const hipEvent_t ev[4] = {gate_up_start, gate_up_stop, down_start, down_stop};
  return ffn_stages(kBoth, layer, x, x_type, n_tokens, topk_w, counts, offsets, perm, inv_perm,
                    y, workspace, workspace_bytes, stream, ev);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the supported range";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: a HIP call or kernel launch failed";
  }
  return "unknown moe_status";
}

}  // extern "C"

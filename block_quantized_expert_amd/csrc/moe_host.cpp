// Host-side argument checks and workspace planning (see moe_host.h).
#include "moe_host.h"

#include <math.h>

namespace moe {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool dim_ok(int v) { return v >= 128 && v <= MOE_MAX_DIM && v % 128 == 0; }

moe_status check_tokens_k(int n_tokens, int n_experts, int top_k) {
  if (n_tokens < 0 || n_experts <= 0 || top_k <= 0) return MOE_ERR_INVALID;
  if (top_k > n_experts) return MOE_ERR_INVALID;
  if (n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
  if (n_tokens > MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_proj(const moe_proj& p) {
  if (p.type != MOE_W_MXFP4 && p.type != MOE_W_FP8E4M3_B128) return MOE_ERR_UNSUPPORTED;
  if (p.codes == nullptr || p.scales == nullptr) return MOE_ERR_INVALID;
  if (!aligned16(p.codes) || !aligned16(p.scales)) return MOE_ERR_INVALID;
  return MOE_OK;
}

}  // namespace

moe_status check_route(const float* logits, int n_tokens, int n_experts, int top_k,
                       float routed_scale, const int32_t* ids, const float* w) {
  moe_status s = check_tokens_k(n_tokens, n_experts, top_k);
  if (s != MOE_OK) return s;
  if (!(routed_scale > 0.0f) || !isfinite(routed_scale)) return MOE_ERR_INVALID;
  if (n_tokens > 0 && (logits == nullptr || ids == nullptr || w == nullptr)) return MOE_ERR_INVALID;
  return MOE_OK;
}

moe_status check_route_group(const float* logits, int n_tokens, int n_experts, int top_k,
                             float routed_scale, const int32_t* ids, const float* w,
                             const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                             const int32_t* inv_perm) {
  moe_status s = check_route(logits, n_tokens, n_experts, top_k, routed_scale, ids, w);
  if (s != MOE_OK) return s;
  return check_group(ids, n_tokens, top_k, n_experts, counts, offsets, perm, inv_perm);
}

moe_status check_route_hash(const int32_t* token_ids, int n_tokens, const int32_t* tid2eid,
                            const float* tid2w, int vocab, int n_experts, int top_k,
                            const int32_t* ids, const float* w) {
  moe_status s = check_tokens_k(n_tokens, n_experts, top_k);
  if (s != MOE_OK) return s;
  if (vocab <= 0) return MOE_ERR_INVALID;
  if (n_tokens > 0 && (token_ids == nullptr || tid2eid == nullptr || tid2w == nullptr ||
                       ids == nullptr || w == nullptr))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

moe_status check_group(const int32_t* ids, int n_tokens, int top_k, int n_experts,
                       const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                       const int32_t* inv_perm) {
  moe_status s = check_tokens_k(n_tokens, n_experts, top_k);
  if (s != MOE_OK) return s;
  if (counts == nullptr || offsets == nullptr) return MOE_ERR_INVALID;
  if (n_tokens > 0 && (ids == nullptr || perm == nullptr || inv_perm == nullptr))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

moe_status check_layer(const moe_layer* layer) {
  if (layer == nullptr) return MOE_ERR_INVALID;
  moe_status s = check_tokens_k(0, layer->n_experts, layer->top_k);
  if (s != MOE_OK) return s;
  if (layer->hidden <= 0 || layer->inter <= 0) return MOE_ERR_INVALID;
  if (!dim_ok(layer->hidden) || !dim_ok(layer->inter)) return MOE_ERR_UNSUPPORTED;
  if ((s = check_proj(layer->gate)) != MOE_OK) return s;
  if ((s = check_proj(layer->up)) != MOE_OK) return s;
  if ((s = check_proj(layer->down)) != MOE_OK) return s;
  // the kernels read one weight type for the routed matrices and one for
  // the shared ones
  if (layer->up.type != layer->gate.type || layer->down.type != layer->gate.type)
    return MOE_ERR_UNSUPPORTED;
  if (layer->has_shared != 0 && layer->has_shared != 1) return MOE_ERR_INVALID;
  if (layer->has_shared) {
    if (layer->shared_inter <= 0) return MOE_ERR_INVALID;
    if (!dim_ok(layer->shared_inter)) return MOE_ERR_UNSUPPORTED;
    if ((s = check_proj(layer->shared_gate)) != MOE_OK) return s;
    if ((s = check_proj(layer->shared_up)) != MOE_OK) return s;
    if ((s = check_proj(layer->shared_down)) != MOE_OK) return s;
    if (layer->shared_up.type != layer->shared_gate.type ||
        layer->shared_down.type != layer->shared_gate.type)
      return MOE_ERR_UNSUPPORTED;
  }
  if (layer->packed_experts != nullptr) {
    if (reinterpret_cast<uintptr_t>(layer->packed_experts) % 256 != 0) return MOE_ERR_INVALID;
    PackPlan pk;
    if ((s = plan_pack(layer, &pk)) != MOE_OK) return s;
  }
  return MOE_OK;
}

moe_status plan_pack(const moe_layer* layer, PackPlan* plan) {
  if (layer->gate.type != MOE_W_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (layer->hidden % 512 != 0 || layer->inter % 512 != 0) return MOE_ERR_UNSUPPORTED;
  const bool sh = layer->has_shared != 0;
  if (sh && layer->shared_inter % 512 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t E = layer->n_experts, H = layer->hidden, I = layer->inter;
  const int64_t SI = sh ? layer->shared_inter : 0;
  const int64_t rows[6] = {E * I, E * I, E * H, SI, SI, sh ? H : 0};
  const int32_t cols[6] = {(int32_t)H, (int32_t)H, (int32_t)I, (int32_t)H, (int32_t)H,
                           (int32_t)SI};
  const int32_t st = sh ? layer->shared_gate.type : MOE_W_MXFP4;
  const int32_t type[6] = {MOE_W_MXFP4, MOE_W_MXFP4, MOE_W_MXFP4, st, st, st};
  size_t off = 0;
  for (int m = 0; m < 6; ++m) {
    plan->rows[m] = rows[m];
    plan->cols[m] = cols[m];
    plan->type[m] = type[m];
    if (rows[m] == 0) {
      plan->codes[m] = plan->scales[m] = -1;
      continue;
    }
    // codes: half a byte per input (MXFP4) or a byte (fp8); scale words: one
    // per lane, four steps and 16-row block, rows * cols / 32 bytes for both
    // (fp8 has a scale byte per 128 inputs of a row, and the four lanes of a
    // row hold the same word)
    const bool fp4 = type[m] == MOE_W_MXFP4;
    plan->codes[m] = (int64_t)off;
    off += align_up((size_t)rows[m] * (size_t)(fp4 ? cols[m] / 2 : cols[m]), 256);
    plan->scales[m] = (int64_t)off;
    off += align_up((size_t)rows[m] * (size_t)(cols[m] / 32), 256);
  }
  plan->total = off;
  return MOE_OK;
}

moe_status plan_ffn(const moe_layer* layer, int n_tokens, FfnPlan* plan) {
  if (n_tokens < 0) return MOE_ERR_INVALID;
  if (n_tokens > MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  const int64_t n = n_tokens;
  plan->slots = n * layer->top_k + (layer->has_shared ? n : 0);
  int64_t hs = layer->inter;
  if (layer->has_shared && layer->shared_inter > hs) hs = layer->shared_inter;
  plan->h_stride = hs;
  const size_t h_bytes = align_up((size_t)(plan->slots * hs) * 2u, 256);
  // per-slot outputs as 24-bit floats (three bytes a feature)
  const size_t o_bytes = align_up((size_t)(plan->slots * layer->hidden) * 3u, 256);
  const size_t xq_bytes = align_up((size_t)n * layer->hidden * 2u, 256);
  const size_t xs_bytes = align_up((size_t)n * (layer->hidden / 16), 256);
  // h as three E4M3 parts + 4 scale bytes per 32 fits in the bf16 pair's
  // place (3.125 against 4 bytes per element) except for tiny layers
  const size_t h3_bytes = align_up((size_t)(plan->slots * hs) * 3u, 256);
  const size_t h3s_bytes = align_up((size_t)(plan->slots * (hs / 32)) * 4u, 256);
  const size_t h_area = 2 * h_bytes > h3_bytes + h3s_bytes ? 2 * h_bytes : h3_bytes + h3s_bytes;
  plan->off_h_hi = 0;
  plan->off_h_lo = h_bytes;
  plan->off_h3s = h3_bytes;
  plan->off_obuf = h_area;
  plan->off_xq = h_area + o_bytes;
  plan->off_xs = plan->off_xq + xq_bytes;
  const int64_t nk = n * layer->top_k;
  const size_t gmax_bytes = align_up((size_t)nk * 4u, 256);
  const size_t gbuf_bytes =
      n <= kGateFirstMaxTokens ? align_up((size_t)nk * layer->inter * 4u, 256) : 0;
  plan->off_gmax = plan->off_xs + xs_bytes;
  plan->off_qctr = plan->off_gmax + gmax_bytes;
  plan->off_gbuf = plan->off_qctr + (n > 0 ? 256 : 0);
  // h as three E2M3 parts (24 bytes a part per 32 values) for the packed
  // MXFP4 down of batches with at least 16 slots per routed expert, with a
  // scale word per 32 values; 16 bytes of padding after the last record
  // (the down's 16-byte copies may read 8 bytes past a tile)
  const bool h6 = layer->gate.type == MOE_W_MXFP4 && plan->slots > 0 &&
                  n * layer->top_k >= 16 * (int64_t)layer->n_experts;
  const size_t h6_bytes =
      h6 ? align_up((size_t)(plan->slots * (hs / 32)) * 72u + 16u, 256) : 0;
  const size_t h6s_bytes = h6 ? align_up((size_t)(plan->slots * (hs / 32)) * 4u, 256) : 0;
  plan->off_h6 = plan->off_gbuf + gbuf_bytes;
  plan->off_h6s = plan->off_h6 + h6_bytes;
  plan->total = plan->off_h6s + h6s_bytes;
  return MOE_OK;
}

moe_status check_opts(const moe_opts* opts, int n_experts, int top_k, OptsPlan* out) {
  out->n_group = 1;
  out->topk_group = 1;
  out->bias = nullptr;
  out->keep_max = top_k;
  out->min_w = 0.0f;
  out->lazy_tau = 0.0f;
  if (opts == nullptr) return MOE_OK;
  const int ng = opts->n_group == 0 ? 1 : opts->n_group;
  if (ng < 1 || ng > 64 || n_experts % ng != 0) return MOE_ERR_INVALID;
  const int tg = opts->topk_group == 0 ? ng : opts->topk_group;
  if (tg < 1 || tg > ng) return MOE_ERR_INVALID;
  if ((int64_t)tg * (n_experts / ng) < top_k) return MOE_ERR_INVALID;
  if (opts->sel_bias != nullptr && (reinterpret_cast<uintptr_t>(opts->sel_bias) & 3u) != 0)
    return MOE_ERR_INVALID;
  const int km = opts->keep_max == 0 ? top_k : opts->keep_max;
  if (km < 1 || km > top_k) return MOE_ERR_INVALID;
  if (!isfinite(opts->min_w) || opts->min_w < 0.0f) return MOE_ERR_INVALID;
  if (!isfinite(opts->lazy_tau) || opts->lazy_tau < 0.0f) return MOE_ERR_INVALID;
  out->n_group = ng;
  out->topk_group = ng == 1 ? 1 : tg;
  out->bias = opts->sel_bias;
  out->keep_max = km;
  out->min_w = opts->min_w;
  out->lazy_tau = opts->lazy_tau;
  return MOE_OK;
}

moe_status check_ffn(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                     const float* topk_w, const int32_t* counts, const int32_t* offsets,
                     const int32_t* perm, const int32_t* inv_perm, const float* y,
                     const void* workspace, size_t workspace_bytes, FfnPlan* plan) {
  moe_status s = check_layer(layer);
  if (s != MOE_OK) return s;
  if (n_tokens < 0) return MOE_ERR_INVALID;
  if (x_type != MOE_ACT_F32 && x_type != MOE_ACT_BF16) return MOE_ERR_UNSUPPORTED;
  if ((s = plan_ffn(layer, n_tokens, plan)) != MOE_OK) return s;
  if (n_tokens == 0) return MOE_OK;
  if (x == nullptr || topk_w == nullptr || counts == nullptr || offsets == nullptr ||
      perm == nullptr || inv_perm == nullptr || y == nullptr)
    return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID;
  if (workspace == nullptr || workspace_bytes < plan->total) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_INVALID;
  return MOE_OK;
}

static_assert(MOE_FORWARD_SYNC_BYTES % 256 == 0, "sync area keeps the rest aligned");


moe_status plan_forward(const moe_layer* layer, int n_tokens, ForwardPlan* plan) {
  moe_status s = plan_ffn(layer, n_tokens, &plan->ffn);
  if (s != MOE_OK) return s;
  plan->off_ffn = MOE_FORWARD_SYNC_BYTES;
  plan->total = plan->off_ffn + align_up(plan->ffn.total, 256);
  return MOE_OK;
}

moe_status check_forward(const moe_layer* layer, const float* logits, float routed_scale,
                         const void* x, int x_type, int n_tokens, const int32_t* ids,
                         const float* w, const int32_t* counts, const int32_t* offsets,
                         const int32_t* perm, const int32_t* inv_perm, const float* y,
                         const void* workspace, size_t workspace_bytes, ForwardPlan* plan) {
  moe_status s = check_layer(layer);
  if (s != MOE_OK) return s;
  s = check_route_group(logits, n_tokens, layer->n_experts, layer->top_k, routed_scale, ids, w,
                        counts, offsets, perm, inv_perm);
  if (s != MOE_OK) return s;
  if (x_type != MOE_ACT_F32 && x_type != MOE_ACT_BF16) return MOE_ERR_UNSUPPORTED;
  if ((s = plan_forward(layer, n_tokens, plan)) != MOE_OK) return s;
  if (n_tokens == 0) return MOE_OK;
  if (x == nullptr || y == nullptr) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return MOE_ERR_INVALID;
  if (workspace == nullptr || workspace_bytes < plan->total) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_INVALID;
  return MOE_OK;
}

}  // namespace moe

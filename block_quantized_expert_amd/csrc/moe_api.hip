// The extern "C" entry points of libmoe.so (declared in include/moe.h):
// validate on the host, then enqueue the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <mutex>

#include "moe.h"
#include "moe_host.h"
#include "moe_kernels.h"

namespace {

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// Zeroes n 8-byte words: the barrier words of a forward workspace are
// cleared by a kernel, not a memset, so the clearing can sit in a captured
// graph too.
__global__ void zero_words_kernel(unsigned long long* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

hipError_t zero_sync_words(void* p, hipStream_t stream) {
  constexpr int kWords = MOE_FORWARD_SYNC_BYTES / 8;
  hipLaunchKernelGGL(zero_words_kernel, dim3((kWords + 255) / 256), dim3(256), 0, stream,
                     static_cast<unsigned long long*>(p), kWords);
  return hipGetLastError();
}

// Polls of the single-token kernel's grid-barrier flags before it gives up
// (about a second).
constexpr uint32_t kFusedSpinLimit = 1u << 20;

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
  p.obuf = reinterpret_cast<uint32_t*>(ws + plan.off_obuf);
  p.h3 = reinterpret_cast<uint8_t*>(ws + plan.off_h_hi);
  p.h3s = reinterpret_cast<uint8_t*>(ws + plan.off_h3s);
  p.xq = reinterpret_cast<uint8_t*>(ws + plan.off_xq);
  p.xs = reinterpret_cast<uint8_t*>(ws + plan.off_xs);
  p.y = y;
  p.lazy_tau = 0.0f;
  p.gmax = reinterpret_cast<uint32_t*>(ws + plan.off_gmax);
  p.gbuf = reinterpret_cast<float*>(ws + plan.off_gbuf);
  p.qctr = reinterpret_cast<uint32_t*>(ws + plan.off_qctr);
  p.n_slots = plan.slots;
  if (plan.off_h6s > plan.off_h6) {
    p.h6 = reinterpret_cast<uint8_t*>(ws + plan.off_h6);
    p.h6s = reinterpret_cast<uint32_t*>(ws + plan.off_h6s);
  }
  moe::PackPlan pk;
  if (L->packed_experts != nullptr && moe::plan_pack(L, &pk) == MOE_OK) {
    const uint8_t* base = static_cast<const uint8_t*>(L->packed_experts);
    for (int m = 0; m < 6; ++m) {
      p.pk_c[m] = pk.codes[m] >= 0 ? base + pk.codes[m] : nullptr;
      p.pk_s[m] = pk.scales[m] >= 0 ? base + pk.scales[m] : nullptr;
    }
    p.packed = true;
  }
  return p;
}

moe::RouteOpts route_opts(const moe::OptsPlan& o) {
  return moe::RouteOpts{o.n_group, o.topk_group, o.bias, o.keep_max, o.min_w};
}

bool route_opts_active(const moe::OptsPlan& o, int top_k) {
  return o.n_group > 1 || o.bias != nullptr || o.keep_max < top_k || o.min_w > 0.0f;
}

enum Stage { kGateUp = 1, kDown = 2, kBoth = 3 };

moe_status ffn_stages(int stages, const moe_layer* layer, const void* x, int x_type,
                      int n_tokens, const float* topk_w, const int32_t* counts,
                      const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm,
                      float* y, void* workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t const* events = nullptr, const moe_opts* opts = nullptr) {
  moe::FfnPlan plan;
  moe_status s = moe::check_ffn(layer, x, x_type, n_tokens, topk_w, counts, offsets, perm,
                                inv_perm, y, workspace, workspace_bytes, &plan);
  if (s != MOE_OK) return s;
  moe::OptsPlan o;
  if ((s = moe::check_opts(opts, layer->n_experts, layer->top_k, &o)) != MOE_OK) return s;
  if (n_tokens == 0) return MOE_OK;
  moe::FfnParams p = make_params(layer, x, x_type, n_tokens, topk_w, counts, offsets, perm,
                                 inv_perm, y, workspace, plan);
  p.lazy_tau = o.lazy_tau;
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

static_assert(sizeof(moe::FusedSync) <= MOE_FORWARD_SYNC_BYTES, "sync area of the workspace");

moe_status forward_impl(const moe_layer* layer, const float* logits, float routed_scale,
                        const void* x, int x_type, int n_tokens, int32_t* topk_ids,
                        float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, float* y, void* workspace, size_t workspace_bytes,
                        int32_t* dev_error, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop, const moe_opts* opts = nullptr) {
  moe::ForwardPlan plan;
  moe_status s = moe::check_forward(layer, logits, routed_scale, x, x_type, n_tokens, topk_ids,
                                    topk_w, counts, offsets, perm, inv_perm, y, workspace,
                                    workspace_bytes, &plan);
  if (s != MOE_OK) return s;
  moe::OptsPlan o;
  if ((s = moe::check_opts(opts, layer->n_experts, layer->top_k, &o)) != MOE_OK) return s;
  const moe::RouteOpts ro = route_opts(o);
  char* ws = static_cast<char*>(workspace);
  moe::FfnParams p{};
  if (n_tokens > 0) {
    p = make_params(layer, x, x_type, n_tokens, topk_w, counts, offsets, perm, inv_perm, y,
                    ws + plan.off_ffn, plan.ffn);
    p.lazy_tau = o.lazy_tau;
  }
  // the lazy skip needs the gate outputs of every row before the up pass:
  // the separate kernels
  const int steps = n_tokens > 0 && o.lazy_tau == 0.0f ? moe::fused_decode_steps(p) : 0;
  if (steps > 0) {
    moe::FusedParams f{};
    f.p = p;
    f.logits = logits;
    f.routed_scale = routed_scale;
    f.ropts = ro;
    f.route_opts = route_opts_active(o, layer->top_k) ? 1 : 0;
    f.topk_ids = topk_ids;
    f.topk_w = topk_w;
    f.counts = counts;
    f.offsets = offsets;
    f.perm = perm;
    f.inv_perm = inv_perm;
    f.sync = reinterpret_cast<moe::FusedSync*>(ws);
    f.wait_xor = 0;
    f.spin_limit = kFusedSpinLimit;
    // test hook: MOE_TEST_FUSED_GIVE_UP=<polls> makes the grid barrier wait
    // for a value no workgroup posts and give up after that many polls, so
    // the timeout path runs with every workgroup still exiting normally
    if (const char* v = getenv("MOE_TEST_FUSED_GIVE_UP")) {
      f.wait_xor = 0x8000000000000000ull;
      f.spin_limit = (uint32_t)strtoul(v, nullptr, 10);
    }
    f.dev_error = dev_error;
    return launched(moe::launch_decode_fused(f, stream, start, stop));
  }
  if (start && hipEventRecord(start, stream) != hipSuccess) return MOE_ERR_DEVICE;
  s = launched(moe::launch_route_group(logits, n_tokens, layer->n_experts, layer->top_k,
                                       routed_scale, ro, topk_ids, topk_w, counts, offsets,
                                       perm, inv_perm, dev_error, stream));
  if (s != MOE_OK) return s;
  if (n_tokens > 0) {
    if ((s = launched(moe::launch_ffn_gate_up(p, stream, nullptr, nullptr))) != MOE_OK) return s;
    if ((s = launched(moe::launch_ffn_down(p, stream, nullptr, nullptr))) != MOE_OK) return s;
  }
  if (stop && hipEventRecord(stop, stream) != hipSuccess) return MOE_ERR_DEVICE;
  return MOE_OK;
}

// ---------------------------------------------------------------- no-alloc

// moe_forward_noalloc's workspace: one array per GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The current device's scratch address; on the first call for a device it
// is looked up, and the barrier flags at its start are cleared on `stream`
// with a small kernel (no memset node, so the call can be captured in a
// graph; later calls need no clearing: every call stamps a new value).
moe_status device_scratch(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MOE_ERR_DEVICE;
    if (zero_sync_words(ptr, stream) != hipSuccess) return MOE_ERR_DEVICE;
    g_scratch[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch[dev]);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_route_ex(const float* logits, int n_tokens, int n_experts, int top_k,
                        float routed_scale, const moe_opts* opts, int32_t* topk_ids,
                        float* topk_w, hipStream_t stream) {
  moe_status s = moe::check_route(logits, n_tokens, n_experts, top_k, routed_scale, topk_ids,
                                  topk_w);
  if (s != MOE_OK) return s;
  moe::OptsPlan o;
  if ((s = moe::check_opts(opts, n_experts, top_k, &o)) != MOE_OK || n_tokens == 0) return s;
  return launched(moe::launch_route(logits, n_tokens, n_experts, top_k, routed_scale,
                                    route_opts(o), topk_ids, topk_w, stream));
}

moe_status moe_route(const float* logits, int n_tokens, int n_experts, int top_k,
                     float routed_scale, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream) {
  return moe_route_ex(logits, n_tokens, n_experts, top_k, routed_scale, nullptr, topk_ids,
                      topk_w, stream);
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

moe_status moe_route_group_ex(const float* logits, int n_tokens, int n_experts, int top_k,
                              float routed_scale, const moe_opts* opts, int32_t* topk_ids,
                              float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                              int32_t* inv_perm, int32_t* dev_error, hipStream_t stream) {
  moe_status s = moe::check_route_group(logits, n_tokens, n_experts, top_k, routed_scale,
                                        topk_ids, topk_w, counts, offsets, perm, inv_perm);
  if (s != MOE_OK) return s;
  moe::OptsPlan o;
  if ((s = moe::check_opts(opts, n_experts, top_k, &o)) != MOE_OK) return s;
  return launched(moe::launch_route_group(logits, n_tokens, n_experts, top_k, routed_scale,
                                          route_opts(o), topk_ids, topk_w, counts, offsets,
                                          perm, inv_perm, dev_error, stream));
}

moe_status moe_route_group(const float* logits, int n_tokens, int n_experts, int top_k,
                           float routed_scale, int32_t* topk_ids, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                           int32_t* dev_error, hipStream_t stream) {
  return moe_route_group_ex(logits, n_tokens, n_experts, top_k, routed_scale, nullptr, topk_ids,
                            topk_w, counts, offsets, perm, inv_perm, dev_error, stream);
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

moe_status moe_ffn_forward_ex(const moe_layer* layer, const void* x, int x_type, int n_tokens,
                              const float* topk_w, const int32_t* counts, const int32_t* offsets,
                              const int32_t* perm, const int32_t* inv_perm, float* y,
                              const moe_opts* opts, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, hipEvent_t gate_up_start,
                              hipEvent_t gate_up_stop, hipEvent_t down_start,
                              hipEvent_t down_stop) {
  const hipEvent_t ev[4] = {gate_up_start, gate_up_stop, down_start, down_stop};
  return ffn_stages(kBoth, layer, x, x_type, n_tokens, topk_w, counts, offsets, perm, inv_perm,
                    y, workspace, workspace_bytes, stream, ev, opts);
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

size_t moe_forward_workspace_bytes(const moe_layer* layer, int n_tokens) {
  moe::ForwardPlan plan;
  if (moe::check_layer(layer) != MOE_OK) return 0;
  if (moe::plan_forward(layer, n_tokens, &plan) != MOE_OK) return 0;
  return plan.total;
}

int moe_forward_single_kernel(const moe_layer* layer, int n_tokens, int x_type) {
  if (moe::check_layer(layer) != MOE_OK) return -1;
  if (n_tokens != 1 || (x_type != MOE_ACT_F32 && x_type != MOE_ACT_BF16)) return 0;
  moe::FfnPlan plan;
  if (moe::plan_ffn(layer, n_tokens, &plan) != MOE_OK) return -1;
  const moe::FfnParams p = make_params(layer, nullptr, x_type, n_tokens, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, nullptr, nullptr, plan);
  return moe::fused_decode_steps(p) > 0 ? 1 : 0;
}

moe_status moe_forward_workspace_init(void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (workspace == nullptr || workspace_bytes < MOE_FORWARD_SYNC_BYTES) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return MOE_ERR_INVALID;
  return launched(zero_sync_words(workspace, stream));
}

moe_status moe_forward(const moe_layer* layer, const float* logits, float routed_scale,
                       const void* x, int x_type, int n_tokens, int32_t* topk_ids,
                       float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv_perm, float* y, void* workspace, size_t workspace_bytes,
                       int32_t* dev_error, hipStream_t stream) {
  return forward_impl(layer, logits, routed_scale, x, x_type, n_tokens, topk_ids, topk_w, counts,
                      offsets, perm, inv_perm, y, workspace, workspace_bytes, dev_error, stream,
                      nullptr, nullptr);
}

moe_status moe_forward_timed(const moe_layer* layer, const float* logits, float routed_scale,
                             const void* x, int x_type, int n_tokens, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                             int32_t* inv_perm, float* y, void* workspace,
                             size_t workspace_bytes, int32_t* dev_error, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
  return forward_impl(layer, logits, routed_scale, x, x_type, n_tokens, topk_ids, topk_w, counts,
                      offsets, perm, inv_perm, y, workspace, workspace_bytes, dev_error, stream,
                      start, stop);
}

moe_status moe_forward_ex(const moe_layer* layer, const float* logits, float routed_scale,
                          const moe_opts* opts, const void* x, int x_type, int n_tokens,
                          int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv_perm, float* y, void* workspace,
                          size_t workspace_bytes, int32_t* dev_error, hipStream_t stream,
                          hipEvent_t start, hipEvent_t stop) {
  return forward_impl(layer, logits, routed_scale, x, x_type, n_tokens, topk_ids, topk_w, counts,
                      offsets, perm, inv_perm, y, workspace, workspace_bytes, dev_error, stream,
                      start, stop, opts);
}

moe_status moe_forward_noalloc(const moe_layer* layer, const float* logits, float routed_scale,
                               const void* x, int x_type, int n_tokens, int32_t* topk_ids,
                               float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv_perm, float* y, int32_t* dev_error,
                               hipStream_t stream) {
  // every argument is checked (the workspace against the scratch size)
  // before the first call on a device enqueues its clearing kernel; the
  // checks read only the workspace pointer's alignment, so an aligned
  // stand-in serves until the device address is known
  moe::ForwardPlan plan;
  moe_status s = moe::check_forward(layer, logits, routed_scale, x, x_type, n_tokens, topk_ids,
                                    topk_w, counts, offsets, perm, inv_perm, y,
                                    reinterpret_cast<void*>(uintptr_t{256}),
                                    MOE_NOALLOC_SCRATCH_BYTES, &plan);
  if (s != MOE_OK) return s;
  char* ws = nullptr;
  if ((s = device_scratch(stream, &ws)) != MOE_OK) return s;
  return forward_impl(layer, logits, routed_scale, x, x_type, n_tokens, topk_ids, topk_w, counts,
                      offsets, perm, inv_perm, y, ws, MOE_NOALLOC_SCRATCH_BYTES, dev_error,
                      stream, nullptr, nullptr);
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

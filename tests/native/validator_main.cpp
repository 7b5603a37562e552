// Drives the host-side validator of libmoe through accept and reject paths;
// built with address and undefined-behaviour sanitizers by test_abi_host.py.
#include <stdio.h>
#include <stdlib.h>

#include "moe_host.h"

static int failures = 0;

static void expect(moe_status got, moe_status want, const char* what) {
  if (got != want) {
    printf("FAIL %s: got %d want %d\n", what, (int)got, (int)want);
    ++failures;
  }
}

static moe_layer make_layer(const uint8_t* p) {
  moe_layer L = {};
  L.hidden = 4096;
  L.inter = 2048;
  L.n_experts = 256;
  L.top_k = 6;
  L.gate = L.up = L.down = moe_proj{MOE_W_MXFP4, p, p};
  L.has_shared = 1;
  L.shared_inter = 2048;
  L.shared_gate = L.shared_up = L.shared_down = moe_proj{MOE_W_FP8E4M3_B128, p, p};
  return L;
}

int main() {
  alignas(16) static uint8_t buf[64];
  const uint8_t* p = buf;
  const float* f = reinterpret_cast<const float*>(buf);
  const int32_t* i = reinterpret_cast<const int32_t*>(buf);
  moe_layer L = make_layer(p);
  moe::FfnPlan plan;

  expect(moe::check_layer(&L), MOE_OK, "valid layer");
  expect(moe::plan_ffn(&L, 4096, &plan), MOE_OK, "plan");
  if (plan.slots != 4096 * 7 || plan.h_stride != 2048 || plan.total < plan.off_obuf) {
    printf("FAIL plan values\n");
    ++failures;
  }
  expect(moe::check_ffn(&L, buf, MOE_ACT_BF16, 4, f, i, i, i, i, f, buf, plan.total, &plan),
         MOE_OK, "valid ffn");
  expect(moe::check_ffn(&L, buf + 4, MOE_ACT_BF16, 4, f, i, i, i, i, f, buf, plan.total, &plan),
         MOE_ERR_INVALID, "misaligned x");
  expect(moe::check_ffn(&L, buf, MOE_ACT_BF16, 4, f, i, i, i, i, f, buf, 10, &plan),
         MOE_ERR_WORKSPACE, "small workspace");
  expect(moe::check_ffn(nullptr, buf, MOE_ACT_BF16, 4, f, i, i, i, i, f, buf, 0, &plan),
         MOE_ERR_INVALID, "null layer");
  moe_layer bad = L;
  bad.hidden = 4000;
  expect(moe::check_layer(&bad), MOE_ERR_UNSUPPORTED, "hidden % 128");
  bad = L;
  bad.top_k = 9;
  expect(moe::check_layer(&bad), MOE_ERR_UNSUPPORTED, "top_k > 8");
  bad = L;
  bad.shared_down.type = MOE_W_MXFP4;
  expect(moe::check_layer(&bad), MOE_ERR_UNSUPPORTED, "mixed shared types");
  bad = L;
  bad.gate.codes = nullptr;
  expect(moe::check_layer(&bad), MOE_ERR_INVALID, "null codes");
  expect(moe::plan_ffn(&L, MOE_MAX_TOKENS + 1, &plan), MOE_ERR_UNSUPPORTED, "too many tokens");
  expect(moe::plan_ffn(&L, MOE_MAX_TOKENS, &plan), MOE_OK, "max tokens");
  expect(moe::check_route(f, 4, 256, 6, 1.5f, i, f), MOE_OK, "route ok");
  expect(moe::check_route(f, 4, 256, 6, -1.0f, i, f), MOE_ERR_INVALID, "route scale");
  expect(moe::check_route_hash(i, 4, i, f, 129280, 256, 6, i, f), MOE_OK, "hash ok");
  expect(moe::check_route_hash(i, 4, i, f, 0, 256, 6, i, f), MOE_ERR_INVALID, "hash vocab");
  expect(moe::check_group(i, 4, 6, 256, i, i, i, i), MOE_OK, "group ok");
  expect(moe::check_group(i, 0, 6, 256, i, i, nullptr, nullptr), MOE_OK, "group empty");
  expect(moe::check_group(i, 4, 6, 1025, i, i, i, i), MOE_ERR_UNSUPPORTED, "group experts");
  if (failures == 0) printf("validator ok\n");
  return failures == 0 ? 0 : 1;
}

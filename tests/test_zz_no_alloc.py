"""moe_forward_noalloc (the entry point for callers that cannot allocate)
against moe_forward on the same inputs, through the C ABI: two calls in a
row on the library's one scratch array, the second with a smaller batch, and
a batch beyond the array's size rejected before anything runs."""

import numpy as np
import pytest
import torch

from block_quantized_expert_amd import binding as B
from block_quantized_expert_amd import inputs as I
from moe_testlib import assert_y_close, gpu_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.empty_cache()


def _same(buf_a, buf_b):
    assert torch.equal(buf_a.ids, buf_b.ids)
    assert torch.equal(buf_a.w, buf_b.w)
    for a, b in zip(buf_a.grouping, buf_b.grouping):
        assert torch.equal(a, b)
    assert_y_close(buf_b.y.cpu().numpy(), buf_a.y.cpu().numpy().astype(np.float64))
    assert torch.equal(buf_a.y, buf_b.y), "same kernels, same order: bitwise equal expected"


def test_noalloc_matches_moe_forward_twice_then_rejects_too_large():
    wl = I.WORKLOADS["decode32"]
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    logits = routing_d["logits"]
    # call 1: 32 tokens (route+group kernel, grouped GEMMs, combine)
    print("case noalloc 32 tokens", flush=True)
    ref = B.moe_forward(layer, logits, x_d, wl.routed_scale)
    got = B.moe_forward_noalloc(layer, logits, x_d, wl.routed_scale)
    torch.cuda.synchronize()
    assert int(got.dev_error.item()) == 0
    _same(ref, got)
    # call 2, smaller: one token (the single fused kernel and its barrier
    # flags in the same array the first call used)
    print("case noalloc 1 token", flush=True)
    x1, l1 = x_d[5:6].contiguous(), logits[5:6].contiguous()
    ref1 = B.moe_forward(layer, l1, x1, wl.routed_scale)
    got1 = B.moe_forward_noalloc(layer, l1, x1, wl.routed_scale)
    torch.cuda.synchronize()
    assert int(got1.dev_error.item()) == 0
    _same(ref1, got1)
    # beyond the array: MOE_ERR_WORKSPACE, nothing written
    n_max = max(n for n in range(1, 1024)
                if layer.forward_workspace_bytes(n) <= B.MOE_NOALLOC_SCRATCH_BYTES)
    assert 300 < n_max < 512, n_max
    big = 512
    assert layer.forward_workspace_bytes(big) > B.MOE_NOALLOC_SCRATCH_BYTES
    xb = torch.zeros((big, wl.hidden), dtype=torch.bfloat16, device=x_d.device)
    lb = torch.zeros((big, wl.n_experts), dtype=torch.float32, device=x_d.device)
    buf = B.ForwardBuffers(layer, big, x_d.device, workspace=False)
    buf.y.fill_(7.0)
    with pytest.raises(B.MoeError) as e:
        B.moe_forward_noalloc(layer, lb, xb, wl.routed_scale, buffers=buf)
    assert e.value.status == B.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((buf.y == 7.0).all())
    # the array is still good afterwards
    again = B.moe_forward_noalloc(layer, l1, x1, wl.routed_scale)
    torch.cuda.synchronize()
    assert torch.equal(again.y, ref1.y)


"""GPU parity of moe_forward (routing + grouping + FFN in one call) against the
oracle, through the C ABI.  Single-token calls of the covered formats run as
one fused kernel with a grid barrier; the other calls go through the
separate route+group and FFN kernels."""

import ctypes
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_quantized_expert_amd import binding as B
from block_quantized_expert_amd import inputs as I
from moe_testlib import assert_w_close, assert_y_close, gpu_inputs, oracle_routing, oracle_y

pytestmark = pytest.mark.gpu

ONE = I.Workload("one", 1, 512, 512, 16, 2, 1.5, "bf16", "learned", 119, 124, "mxfp4", "none",
                 31)


def _check_routing(wl, routing, buf):
    ids_ref, w_ref = oracle_routing(wl, routing)
    ids = buf.ids.cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    assert_w_close(buf.w.cpu().numpy(), w_ref.astype(np.float32))
    counts, offsets, perm, inv_perm = [t.cpu().numpy() for t in buf.grouping]
    nk = ids.size
    flat = ids.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=wl.n_experts))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(perm[:nk], order)
    assert np.array_equal(inv_perm[:nk][order], np.arange(nk))
    return ids_ref, w_ref


def _run_and_check(wl, with_shared=True, copy=0):
    layer, x, x_d, routing, routing_d = gpu_inputs(wl, copy=copy, with_shared=with_shared)
    buf = B.moe_forward(layer, routing_d["logits"], x_d, wl.routed_scale)
    torch.cuda.synchronize()
    assert int(buf.dev_error.item()) == 0
    ids_ref, w_ref = _check_routing(wl, routing, buf)
    ref = oracle_y(wl, x, ids_ref, w_ref, with_shared=with_shared, copy=copy)
    assert_y_close(buf.y.cpu().numpy(), ref)


def test_decode1_full():
    _run_and_check(I.WORKLOADS["decode1"])


@pytest.mark.parametrize("wl,with_shared", [
    (ONE, True),                                                     # hidden 512: one step
    (ONE, False),                                                    # no shared expert
    (replace(ONE, hidden=1024, inter=1024, top_k=1, seed=32), True),
    (replace(ONE, hidden=2048, inter=512, top_k=8, seed=33), True),  # top-8
    (replace(ONE, n_experts=256, top_k=6, seed=34), True),
    (replace(ONE, n_experts=200, hidden=4096, inter=1536, seed=35), True),  # 12 down steps
    (replace(ONE, inter=384, seed=38), True),                        # 3 down steps
    # 1296 gate/up items: two rounds; 18 down steps: wavefronts 0-1 take two
    (replace(ONE, n_experts=64, hidden=1024, inter=2304, top_k=8, seed=40), True),
])
def test_single_token_shapes(wl, with_shared):
    _run_and_check(wl, with_shared)


@pytest.mark.parametrize("n_tokens", [32, 200])
def test_batches_take_the_grouped_gemms(n_tokens):
    """bf16 batches of more than 16 tokens through moe_forward: the
    route+group kernel(s), then the grouped-GEMM gate/up and down and the
    combine.  Routing exact; y on sampled tokens and rows."""
    wl = replace(I.WORKLOADS["decode32"], n_tokens=n_tokens)
    print("case forward batch", n_tokens, flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl, copy=5)
    buf = B.moe_forward(layer, routing_d["logits"], x_d, wl.routed_scale)
    torch.cuda.synchronize()
    assert int(buf.dev_error.item()) == 0
    ids_ref, w_ref = _check_routing(wl, routing, buf)
    tokens = sorted(np.random.default_rng(n_tokens).choice(n_tokens, 4, replace=False).tolist())
    rows = sorted(np.random.default_rng(n_tokens + 1).choice(wl.hidden, 512, replace=False).tolist())
    ref = oracle_y(wl, x, ids_ref, w_ref, tokens=tokens, rows=rows, copy=5)
    assert_y_close(buf.y.cpu().numpy()[tokens][:, rows], ref)


@pytest.mark.parametrize("wl", [
    replace(ONE, act="f32", seed=36),              # fp32 x: separate kernels
    replace(ONE, n_tokens=3, seed=37),             # several tokens: separate kernels
    replace(ONE, hidden=640, seed=38),             # hidden not a multiple of 512
])
def test_other_calls_take_the_separate_kernels(wl):
    _run_and_check(wl)


def test_many_calls_share_one_workspace():
    """The barrier flags carry over from call to call."""
    wl = replace(ONE, n_experts=64, top_k=4, seed=39)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    buf = B.ForwardBuffers(layer, 1, x_d.device)
    outs = []
    for c in range(12):
        xc = I.activations(wl, copy=c)
        lc = I.router_logits(wl, copy=c)
        B.moe_forward(layer, lc.cuda(), xc.cuda(), wl.routed_scale, buffers=buf)
        outs.append((xc, lc, buf.y.clone(), buf.ids.clone(), buf.w.clone()))
    torch.cuda.synchronize()
    assert int(buf.dev_error.item()) == 0
    for c in (0, 5, 11):
        xc, lc, y, ids, w = outs[c]
        ids_ref, w_ref = oracle_routing(wl, {"kind": "learned", "logits": lc})
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert_y_close(y.cpu().numpy(), oracle_y(wl, xc, ids_ref, w_ref))
    # the same input twice gives bitwise the same output
    assert torch.equal(outs[0][2], B.moe_forward(layer, outs[0][1].cuda(), outs[0][0].cuda(),
                                                 wl.routed_scale, buffers=buf).y)


def test_matches_separate_calls_bitwise_routing():
    wl = I.WORKLOADS["decode1"]
    layer, x, x_d, routing, routing_d = gpu_inputs(wl, copy=3)
    buf = B.moe_forward(layer, routing_d["logits"], x_d, wl.routed_scale)
    ids, w, grouping = B.moe_route_group(routing_d["logits"], wl.top_k, wl.routed_scale)
    y = B.moe_ffn_forward(layer, x_d, w, grouping)
    torch.cuda.synchronize()
    assert torch.equal(buf.ids, ids) and torch.equal(buf.w, w)
    for a, b in zip(buf.grouping, grouping):
        assert torch.equal(a, b)
    ref = y.cpu().numpy().astype(np.float64)
    assert_y_close(buf.y.cpu().numpy(), ref, tol=1e-4)


def test_zero_tokens_writes_empty_grouping():
    wl = replace(ONE, n_tokens=0)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    buf = B.ForwardBuffers(layer, 0, x_d.device)
    buf.grouping[0].fill_(7)
    buf.grouping[1].fill_(7)
    B.moe_forward(layer, routing_d["logits"], x_d, wl.routed_scale, buffers=buf)
    torch.cuda.synchronize()
    assert int(buf.grouping[0].abs().sum()) == 0 and int(buf.grouping[1].abs().sum()) == 0


def test_timed_entry_point():
    wl = I.WORKLOADS["decode1"]
    layer, x, x_d, routing, routing_d = gpu_inputs(wl, copy=4)
    ev = (B.HipEvent(), B.HipEvent())
    buf = B.moe_forward(layer, routing_d["logits"], x_d, wl.routed_scale, events=ev)
    torch.cuda.synchronize()
    t = ev[0].elapsed_ms(ev[1])
    assert 0.0 < t < 100.0
    ids_ref, w_ref = oracle_routing(wl, routing)
    assert_y_close(buf.y.cpu().numpy(), oracle_y(wl, x, ids_ref, w_ref, copy=4))


@pytest.mark.parametrize("with_dev_error", [True, False])
def test_barrier_give_up_writes_nan(monkeypatch, with_dev_error):
    """The single-token kernel's grid barrier is a bounded wait.  With the
    library's test hook the host asks it to wait for a value no workgroup
    posts and to give up after 16 polls: every workgroup then takes the
    give-up path and exits normally, sets MOE_DEVERR_SYNC and leaves NaN in
    its rows of y, so an incomplete y is visible without dev_error too.  The
    next call without the hook is correct again."""
    wl = replace(ONE, n_experts=64, top_k=4, seed=44)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    assert B.lib().moe_forward_single_kernel(ctypes.byref(layer.c), 1, B.MOE_ACT_BF16) == 1
    buf = B.ForwardBuffers(layer, 1, x_d.device)
    if not with_dev_error:
        buf.dev_error = None
    monkeypatch.setenv("MOE_TEST_FUSED_GIVE_UP", "16")
    B.moe_forward(layer, routing_d["logits"], x_d, wl.routed_scale, buffers=buf)
    torch.cuda.synchronize()
    assert torch.isnan(buf.y).all()
    if with_dev_error:
        assert int(buf.dev_error.item()) & B.MOE_DEVERR_SYNC
        buf.dev_error.zero_()
    monkeypatch.delenv("MOE_TEST_FUSED_GIVE_UP")
    B.moe_forward(layer, routing_d["logits"], x_d, wl.routed_scale, buffers=buf)
    torch.cuda.synchronize()
    if with_dev_error:
        assert int(buf.dev_error.item()) == 0
    ids_ref, w_ref = oracle_routing(wl, routing)
    assert_y_close(buf.y.cpu().numpy(), oracle_y(wl, x, ids_ref, w_ref))


@pytest.mark.parametrize("entry", ["moe_forward", "moe_forward_noalloc"])
@pytest.mark.parametrize("n_tokens", [1, 20])
def test_captured_graph_replays_match_eager(entry, n_tokens):
    """A call captured in a HIP graph (torch's CUDAGraph) is replayed four
    times on new inputs copied into its static buffers, with eager calls and
    synchronisations between the replays; every replay equals the eager call
    bitwise.  One token runs the fused kernel, whose barrier takes a new
    epoch from the workspace's launch counter at every launch (arguments are
    frozen in a graph); 20 tokens run the route+group and FFN kernels."""
    wl = replace(ONE, n_tokens=n_tokens, n_experts=64, top_k=4, seed=46)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    fn = getattr(B, entry)
    use_ws = entry == "moe_forward"
    buf = B.ForwardBuffers(layer, n_tokens, x_d.device, workspace=use_ws)
    x_s, l_s = x_d.clone(), routing_d["logits"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(layer, l_s, x_s, wl.routed_scale, buffers=buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(layer, l_s, x_s, wl.routed_scale, buffers=buf)
    for c in range(4):
        xc = I.activations(wl, copy=c + 1).to(x_d.device)
        lc = I.router_logits(wl, copy=c + 1).to(x_d.device)
        x_s.copy_(xc)
        l_s.copy_(lc)
        g.replay()
        torch.cuda.synchronize()
        ref = fn(layer, lc, xc, wl.routed_scale)
        torch.cuda.synchronize()
        assert int(buf.dev_error.item()) == 0
        assert torch.equal(buf.ids, ref.ids), c
        assert torch.equal(buf.y, ref.y), c
        if c == 3:
            ids_ref, w_ref = oracle_routing(wl, {"kind": "learned", "logits": lc.cpu()})
            assert_y_close(buf.y.cpu().numpy(), oracle_y(wl, xc.cpu(), ids_ref, w_ref))

"""GPU parity of the whole path (route -> group -> gate/up -> down ->
combine) against the fp64 oracle, plus metamorphic checks that need no
oracle.  Bar: max|err| <= 2e-3 * rms(oracle y) over the compared outputs."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from block_quantized_expert_amd import binding as B
from block_quantized_expert_amd import inputs as I

from moe_testlib import assert_y_close, gpu_inputs, oracle_routing, oracle_y

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.empty_cache()


def _run(wl, copy=0, with_shared=True):
    layer, x, x_d, routing, routing_d = gpu_inputs(wl, copy, with_shared)
    y, ids, w, grouping = B.forward(layer, x_d, routing_d, wl.routed_scale)
    torch.cuda.synchronize()
    return layer, x, routing, y, ids, w, grouping


def _sample(n, k, seed):
    return sorted(np.random.default_rng(seed).choice(n, size=min(n, k), replace=False).tolist())


# ----------------------------------------------------------------- full size


@pytest.mark.parametrize("with_shared", [True, False])
def test_tiny_full(with_shared):
    wl = I.WORKLOADS["tiny"]
    print("case tiny shared=%s" % with_shared, flush=True)
    _, x, routing, y, ids, w, _ = _run(wl, with_shared=with_shared)
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    ref = oracle_y(wl, x, rids, rw, with_shared=with_shared)
    assert_y_close(y.cpu().numpy(), ref)


def test_decode1_full():
    wl = I.WORKLOADS["decode1"]
    print("case decode1", flush=True)
    _, x, routing, y, ids, w, _ = _run(wl)
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    ref = oracle_y(wl, x, rids, rw)
    assert_y_close(y.cpu().numpy(), ref)


@pytest.mark.parametrize("name,n_tok,n_rows,with_shared", [
    ("decode32", 8, 1024, True),
    ("decode32", 4, 512, False),
    ("prefill512", 6, 512, True),
    ("hash4096", 4, 512, True),
])
def test_sampled_full_size(name, n_tok, n_rows, with_shared):
    wl = I.WORKLOADS[name]
    print("case %s sampled tokens=%d rows=%d shared=%s" % (name, n_tok, n_rows, with_shared),
          flush=True)
    _, x, routing, y, ids, w, _ = _run(wl, with_shared=with_shared)
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    tokens = _sample(wl.n_tokens, n_tok, 11)
    rows = _sample(wl.hidden, n_rows, 12)
    ref = oracle_y(wl, x, rids, rw, tokens=tokens, rows=rows, with_shared=with_shared)
    assert_y_close(y.cpu().numpy()[tokens][:, rows], ref)


def test_batch_past_32bit_activation_offsets():
    """263144 tokens at hidden 4096: the quantized activations (two bytes
    per input) pass 2^31 bytes, so the batched gate/up kernels (MXFP4 routed,
    fp8 shared) take their 64-bit-offset form.  Small experts keep the run
    short; sampled tokens on both sides of the 2^31-byte mark against the
    oracle."""
    wl = I.Workload("past2g", 263144, 4096, 128, 4, 1, 1.5, "bf16", "learned", 119, 124,
                    "fp8_e4m3_b128", "none", 27)
    first_past = (1 << 31) // (2 * wl.hidden)  # first token whose row starts at 2^31
    assert first_past < wl.n_tokens
    print("case past2g: %d tokens, hidden %d" % (wl.n_tokens, wl.hidden), flush=True)
    _, x, routing, y, ids, w, _ = _run(wl)
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    tokens = sorted(set(_sample(first_past, 3, 13) + [first_past - 1, first_past,
                                                       wl.n_tokens - 1]))
    rows = _sample(wl.hidden, 256, 14)
    got = y[torch.tensor(tokens, device=y.device)][:, torch.tensor(rows, device=y.device)]
    ref = oracle_y(wl, x, rids, rw, tokens=tokens, rows=rows)
    assert_y_close(got.cpu().numpy(), ref)


# ------------------------------------------------------- small, several tiles

SMALL = I.Workload("small", 100, 256, 128, 8, 2, 1.5, "bf16", "learned", 119, 124,
                   "mxfp4", "none", 21)


@pytest.mark.parametrize("wl", [
    SMALL,                                                       # 2 token tiles, ragged
    replace(SMALL, n_tokens=40, shared="fp8_e4m3_b128", seed=22),  # fp8 shared, 3 blocks
    replace(SMALL, n_tokens=33, shared_inter=256, seed=23),      # shared inter != inter
    replace(SMALL, n_tokens=17, act="f32", top_k=3, seed=24),     # fp32 x, hi/lo split
    replace(SMALL, n_tokens=130, n_experts=5, top_k=5, seed=25),  # every expert, 3 tiles
    replace(SMALL, n_tokens=1, hidden=512, inter=384, seed=26),   # K steps 4 and 3
    replace(SMALL, routed="fp8_e4m3_b128", seed=28),             # fp8 routed, grouped GEMM
    replace(SMALL, routed="fp8_e4m3_b128", act="f32", n_tokens=3, seed=29),   # small down
    replace(SMALL, routed="fp8_e4m3_b128", shared="fp8_e4m3_b128", act="f32", n_tokens=3,
            seed=30),
    replace(SMALL, shared="fp8_e4m3_b128", act="f32", n_tokens=3, seed=31),
    replace(SMALL, routed="fp8_e4m3_b128", act="f32", n_tokens=60, seed=32),  # bf16-pair down
    replace(SMALL, act="f32", n_tokens=40, inter=512, seed=33),  # pair down, scale chunks
    replace(SMALL, routed="fp8_e4m3_b128", act="f32", n_tokens=40, inter=512, seed=34),
    replace(SMALL, n_tokens=3, hidden=1024, seed=35),            # decode gate/up, 2 steps
    replace(SMALL, n_tokens=2, hidden=2048, seed=36),            # decode gate/up, 4 steps
], ids=["ragged100", "fp8shared40", "sharedinter33", "f32x17", "allexperts130", "odd_k1",
        "fp8routed100", "fp8routed_f32x3", "fp8both_f32x3", "fp8shared_f32x3",
        "fp8routed_f32x60", "f32x40_i512", "fp8routed_f32x40_i512", "decode_h1024",
        "decode_h2048"])
def test_small_layers_full(wl):
    print("case small", wl, flush=True)
    _, x, routing, y, ids, w, _ = _run(wl)
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    ref = oracle_y(wl, x, rids, rw)
    assert_y_close(y.cpu().numpy(), ref)


def _extreme_activations(n, h, seed):
    """bf16 rows of six kinds (by token index mod 6): zero, small (2^-40,
    the expert outputs stay normal fp32), bf16-subnormal (~2^-130: h
    underflows, the output is exactly zero on both sides), large (2^20),
    magnitudes log-uniform over 30 binades inside every 32-input block, and
    one nonzero per block.  The batched gate/up stores x as two E4M3 parts
    under a per-32 scale taken from the block's largest magnitude; these
    rows test that split at the ends of the exponent range and far below the
    block maximum."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, h))
    kind = np.arange(n) % 6
    x[kind == 0] = 0.0
    x[kind == 1] *= 2.0 ** -40
    x[kind == 2] *= 2.0 ** -130
    x[kind == 3] *= 2.0 ** 20
    m = kind == 4
    x[m] = np.sign(x[m]) * 2.0 ** rng.uniform(-30, 0, size=x[m].shape)
    m = kind == 5
    keep = np.zeros((n, h), dtype=bool)
    keep[:, ::32] = True
    x[m & ~keep.any(1)] = 0.0
    x[m] = np.where(keep[m], x[m], 0.0)
    x[0, 1] = -0.0
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def test_extreme_activations_per_token():
    # batched path (48 tokens > 16): activation quantization + grouped GEMMs
    wl = replace(SMALL, n_tokens=48, shared="mxfp4", seed=28)
    print("case extreme activations", flush=True)
    layer, _, _, routing, routing_d = gpu_inputs(wl)
    x = _extreme_activations(wl.n_tokens, wl.hidden, 29)
    y, ids, w, g = B.forward(layer, x.to(DEV), routing_d)
    torch.cuda.synchronize()
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    ref = oracle_y(wl, x, rids, rw)
    yh = y.cpu().numpy()
    assert np.all(np.isfinite(yh))
    for t in range(wl.n_tokens):
        rms = float(np.sqrt(np.mean(ref[t].astype(np.float64) ** 2)))
        err = float(np.max(np.abs(yh[t].astype(np.float64) - ref[t])))
        if rms == 0.0:
            assert err == 0.0, t
        else:
            assert err <= 2e-3 * rms, (t, err / rms)


def test_stages_equal_forward():
    wl = replace(SMALL, n_tokens=50, seed=27)
    print("case stages", flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    ids, w = B.moe_route(routing_d["logits"], wl.top_k)
    g = B.moe_group(ids, wl.n_experts)
    ws = torch.empty(layer.workspace_bytes(wl.n_tokens), dtype=torch.uint8, device=DEV)
    y1 = B.moe_ffn_forward(layer, x_d, w, g, workspace=ws)
    y2 = torch.empty_like(y1)
    B.moe_ffn_gate_up(layer, x_d, w, g, y=y2, workspace=ws)
    B.moe_ffn_down(layer, x_d, w, g, y=y2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_zero_tokens():
    wl = replace(SMALL, n_tokens=0)
    print("case zero tokens", flush=True)
    layer = B.Layer(I.make_layer(wl, device=DEV), wl.top_k)
    x = torch.zeros((0, wl.hidden), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((0, wl.top_k), dtype=torch.float32, device=DEV)
    z = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = torch.zeros((0, wl.hidden), dtype=torch.float32, device=DEV)
    ws = torch.zeros(1, dtype=torch.uint8, device=DEV)
    B.moe_ffn_forward(layer, x, w, (z, z, z, z), y=y, workspace=ws)
    torch.cuda.synchronize()


# ------------------------------------------------------- metamorphic checks


def _with_scales_bumped(weights, proj):
    out = dict(weights)
    out[proj] = dict(weights[proj], scales=weights[proj]["scales"] + 1)
    if weights.get("shared") is not None:
        sh = dict(weights["shared"])
        sh[proj] = dict(sh[proj], scales=sh[proj]["scales"] + 1)
        out["shared"] = sh
    return out


@pytest.mark.parametrize("proj", ["down", "up"])
def test_scale_increment_doubles_output_bitwise(proj):
    # one more in every UE8M0 byte of a linear projection multiplies every
    # expert output by exactly 2; the kernels' arithmetic commutes with that
    wl = I.WORKLOADS["decode32"]
    print("case doubling", proj, flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    y1, *_ = B.forward(layer, x_d, routing_d)
    layer2 = B.Layer(_with_scales_bumped(layer.weights, proj), wl.top_k)
    y2, *_ = B.forward(layer2, x_d, routing_d)
    torch.cuda.synchronize()
    assert torch.equal(y2, 2 * y1)


def test_repeat_runs_are_bitwise_equal():
    wl = I.WORKLOADS["prefill512"]
    print("case repeat", flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    y1, *_ = B.forward(layer, x_d, routing_d)
    y2, *_ = B.forward(layer, x_d, routing_d)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_shared_split_is_additive():
    # y(with shared) - y(routed only) equals the shared expert alone (a
    # layer whose routed weights are all zero), within the tolerance
    wl = replace(I.WORKLOADS["decode32"], n_tokens=8)
    print("case shared additivity", flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    y_all, ids, w, g = B.forward(layer, x_d, routing_d)
    layer_r = B.Layer(dict(layer.weights, shared=None), wl.top_k)
    y_r = B.moe_ffn_forward(layer_r, x_d, w, g)
    y_s = B.moe_ffn_forward(layer, x_d, torch.zeros_like(w), g)
    torch.cuda.synchronize()
    d = (y_all - y_r - y_s).abs().max().item()
    rms = y_all.pow(2).mean().sqrt().item()
    assert d <= 1e-5 * rms


def test_token_permutation_permutes_output():
    wl = I.WORKLOADS["decode32"]
    print("case permutation", flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    y, *_ = B.forward(layer, x_d, routing_d)
    p = torch.randperm(wl.n_tokens, generator=torch.Generator().manual_seed(3))
    yp, *_ = B.forward(layer, x_d[p.to(DEV)].contiguous(),
                       {"kind": "learned", "logits": routing_d["logits"][p.to(DEV)].contiguous()})
    torch.cuda.synchronize()
    d = (yp - y[p.to(DEV)]).abs().max().item()
    assert d <= 1e-5 * y.pow(2).mean().sqrt().item()


def test_timed_entry_point_matches_and_times():
    wl = I.WORKLOADS["decode1"]
    print("case timed", flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    y, ids, w, g = B.forward(layer, x_d, routing_d)
    evs = [B.HipEvent() for _ in range(4)]
    y2 = B.moe_ffn_forward_timed(layer, x_d, w, g, evs)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    gu = evs[0].elapsed_ms(evs[1])
    dn = evs[2].elapsed_ms(evs[3])
    assert 0 < gu < 100 and 0 < dn < 100, (gu, dn)  # milliseconds
    y3 = B.moe_ffn_forward_timed(layer, x_d, w, g, [None, None, None, None])
    torch.cuda.synchronize()
    assert torch.equal(y, y3)

"""GPU parity of the grouped-GEMM kernels in the forms the benchmark runs,
against the fp64 oracle on every compared output.

At hidden 4096 and intermediate 2048 the batched path takes the gate/up
kernel with the row block's scale bytes held in LDS (up to five 16-token
blocks per tile) or read in 16-byte chunks (six or seven), and the down
kernel on h in three E4M3 parts with the same two forms (up to three blocks,
four).  Those forms need a reduction dimension that is a multiple of 512, so
the layers here have hidden 1024 and intermediate 512, with the expert
counts fixed through a hash table so that every tile size of both kernels
occurs.  The full-size workloads are compared on every output (decode32) or
on tokens chosen so that every 16-slot block of every expert's group is hit
(prefill512, hash4096).

Bar: max|err| <= 2e-3 * rms(oracle y) ("Deep-Dive Mathematical & Kernel
Guide", section 4 SwiGLU equation and section 3.2 combine equation define
y)."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from block_quantized_expert_amd import binding as B
from block_quantized_expert_amd import inputs as I
from moe_testlib import (assert_y_close, block_tokens, gpu_inputs, oracle_routing,
                         oracle_y_host)
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.empty_cache()


# per-expert slot counts: gate/up tiles of 112 slots end in 1..7 blocks of 16
# (9, 20, 40, 60, 70, 90, 100 and 112 + 19), down tiles of 64 in 1..4 blocks
COUNTS = [9, 20, 40, 60, 70, 90, 100, 131]


def _table(counts, seed):
    """tid2eid rows (two distinct experts per token) realising `counts`, and
    positive weights: the sorted multiset of experts, slot i paired with
    slot i + N (no expert holds more than N slots)."""
    flat = np.repeat(np.arange(len(counts)), counts).astype(np.int32)
    n = flat.size // 2
    assert flat.size == 2 * n and max(counts) < n
    pairs = np.stack([flat[:n], flat[n:]], axis=1)
    rng = np.random.default_rng(seed)
    pairs = pairs[rng.permutation(n)]
    w = rng.uniform(0.1, 1.0, size=pairs.shape).astype(np.float32)
    return pairs, w


RAGGED = I.Workload("ragged", 260, 1024, 512, 8, 2, 1.5, "bf16", "hash", 119, 124, "mxfp4",
                    "none", 41, vocab=260)


@pytest.mark.parametrize("wl", [
    RAGGED,                                        # shared MXFP4: same launch as the routed
    replace(RAGGED, shared="fp8_e4m3_b128", seed=42),  # fp8 shared: own launch, 64-token tiles
], ids=["mxfp4_shared", "fp8_shared"])
def test_every_tile_size_of_the_grouped_gemms(wl):
    print("case tiles %s" % wl.shared, flush=True)
    layer = B.Layer(I.make_layer(wl, device=DEV), wl.top_k)
    pairs, wts = _table(COUNTS, wl.seed)
    x = I.activations(wl)
    tok = torch.arange(wl.n_tokens, dtype=torch.int32, device=DEV)
    t2e = torch.from_numpy(pairs).to(DEV)
    t2w = torch.from_numpy(wts).to(DEV)
    ids, w = B.moe_route_hash(tok, t2e, t2w, wl.n_experts)
    grouping = B.moe_group(ids, wl.n_experts)
    y = B.moe_ffn_forward(layer, x.to(DEV), w, grouping)
    torch.cuda.synchronize()
    rids, rw = O.route_hash(np.arange(wl.n_tokens), pairs, wts)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.array_equal(grouping[0].cpu().numpy(), np.array(COUNTS))
    ref = oracle_y_host(layer.weights, wl.act, x, rids, rw)
    assert_y_close(y.cpu().numpy(), ref)


def test_decode32_every_output():
    wl = I.WORKLOADS["decode32"]
    print("case decode32 all outputs", flush=True)
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    y, ids, w, _ = B.forward(layer, x_d, routing_d, wl.routed_scale)
    torch.cuda.synchronize()
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    ref = oracle_y_host(layer.weights, wl.act, x, rids, rw)
    assert_y_close(y.cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["prefill512", "hash4096"])
def test_every_block_of_every_expert(name):
    """Tokens owning the first slot of every 16-slot block of every expert
    (and of the shared expert), against the oracle on 1024 sampled output
    rows that cover every 256-row tile of the down kernel."""
    wl = I.WORKLOADS[name]
    layer, x, x_d, routing, routing_d = gpu_inputs(wl)
    y, ids, w, _ = B.forward(layer, x_d, routing_d, wl.routed_scale)
    torch.cuda.synchronize()
    rids, rw = oracle_routing(wl, routing)
    assert np.array_equal(ids.cpu().numpy(), rids)
    tokens = block_tokens(rids, wl.n_experts)
    rng = np.random.default_rng(17)
    rows = sorted(set(rng.choice(wl.hidden, 1024, replace=False).tolist())
                  | {256 * t for t in range(wl.hidden // 256)})
    print("case %s: %d tokens x %d rows" % (name, len(tokens), len(rows)), flush=True)
    ref = oracle_y_host(layer.weights, wl.act, x, rids, rw, tokens=tokens, rows=rows)
    got = y[torch.tensor(tokens, device=DEV)][:, torch.tensor(rows, device=DEV)]
    assert_y_close(got.cpu().numpy(), ref)

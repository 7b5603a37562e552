"""The E2M3 down projection (packed MXFP4 layers, batches of at least 16
routed slots per expert): every output against the oracle on layers whose
reductions take 4, 8, 12 and 16 steps of 128 (each a different stretch of
the kernel's straight-line steps and of its ring of buffers), with a shared
MXFP4 expert of the same or of a different width in the same launch, with
an fp8 shared expert whose gate/up and down items share the routed
launches (over one partial and over two groups of its token tiles), with
the gate-first lazy skip, and with tail-pruned slots."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from block_quantized_expert_amd import binding as B
from block_quantized_expert_amd import inputs as I
from moe_testlib import assert_y_close, oracle_y_host
from oracle import moe_oracle as O
from test_gpu_parity_tiles import COUNTS, RAGGED, _table

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.empty_cache()


BASE = replace(RAGGED, hidden=512, seed=61)


@pytest.mark.parametrize("inter,shared_inter,shared,lazy", [
    (512, 0, "mxfp4", 0.0),              # 4 steps
    (1024, 0, "mxfp4", 0.0),             # 8
    (1536, 0, "mxfp4", 0.0),             # 12
    (2048, 0, "mxfp4", 0.0),             # 16
    (512, 1536, "mxfp4", 0.0),           # routed 4 steps, shared 12, one launch
    (1536, 512, "mxfp4", 1e-3),          # routed 12, shared 4, lazy skip
    (512, 1536, "fp8_e4m3_b128", 0.0),   # fp8 shared down in the routed launch
    (2048, 512, "fp8_e4m3_b128", 1e-3),  # the same, routed 16 steps, lazy skip
], ids=["I512", "I1024", "I1536", "I2048", "I512_S1536", "I1536_S512_lazy",
        "I512_S1536_fp8", "I2048_S512_fp8_lazy"])
def test_e2m3_down_against_the_oracle(inter, shared_inter, shared, lazy):
    wl = replace(BASE, inter=inter, shared_inter=shared_inter, shared=shared)
    print("case e2m3 down I=%d SI=%d %s lazy=%g" % (inter, shared_inter, shared, lazy),
          flush=True)
    _check(wl, COUNTS, lazy)


# 600 tokens: ten 64-token tiles of the shared expert (the last of 24), so
# its items form one group of eight token tiles and one of two
COUNTS600 = [20, 46, 92, 138, 162, 208, 231, 303]


def test_e2m3_down_fp8_shared_over_two_item_groups():
    wl = replace(BASE, n_tokens=600, vocab=600, inter=1024, shared_inter=512,
                 shared="fp8_e4m3_b128", seed=67)
    print("case e2m3 down fp8 shared, 600 tokens", flush=True)
    _check(wl, COUNTS600, 0.0)


def _check(wl, counts, lazy):
    layer = B.Layer(I.make_layer(wl, device=DEV), wl.top_k)
    assert layer.pack()
    x = I.activations(wl)
    pairs, wts = _table(counts, wl.seed)
    assert pairs.shape[0] * wl.top_k >= 16 * wl.n_experts  # the E2M3 path's batch size
    tok = torch.arange(wl.n_tokens, dtype=torch.int32, device=DEV)
    ids, w = B.moe_route_hash(tok, torch.from_numpy(pairs).to(DEV),
                              torch.from_numpy(wts).to(DEV), wl.n_experts)
    grouping = B.moe_group(ids, wl.n_experts)
    opts = B.make_opts(lazy_tau=lazy) if lazy > 0 else B.make_opts()
    y = B.moe_ffn_forward_ex(layer, x.to(DEV), w, grouping, opts)
    torch.cuda.synchronize()
    rids, rw = O.route_hash(np.arange(wl.n_tokens), pairs, wts)
    assert_y_close(y.cpu().numpy(),
                   oracle_y_host(layer.weights, wl.act, x, rids, rw, lazy_tau=lazy))


def test_e2m3_down_with_pruned_slots():
    """Learned routing with tail pruning (keep_max 1 of 2) on a packed layer
    whose batch takes the E2M3 path: the dropped slots leave the grouping,
    the kept ones are rescaled; ids and y against the oracle."""
    wl = replace(BASE, routing="learned", seed=63)
    print("case e2m3 down pruned", flush=True)
    layer = B.Layer(I.make_layer(wl, device=DEV), wl.top_k)
    assert layer.pack()
    x = I.activations(wl)
    rng = np.random.default_rng(64)
    lg = I.spaced_logits(rng, wl.n_tokens, 0.5 * rng.standard_normal(wl.n_experts), 1e-3)
    buf = B.moe_forward_ex(layer, torch.from_numpy(lg).to(DEV), x.to(DEV),
                           B.make_opts(keep_max=1), wl.routed_scale)
    torch.cuda.synchronize()
    ids_ref, w_ref = O.route_topk(lg, wl.top_k, wl.routed_scale)
    ids_ref, w_ref = O.prune_tail(ids_ref, w_ref, 1, np.float32(0.0))
    assert np.array_equal(buf.ids.cpu().numpy(), ids_ref)
    assert_y_close(buf.y.cpu().numpy(), oracle_y_host(layer.weights, wl.act, x, ids_ref, w_ref))

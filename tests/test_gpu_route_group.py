"""GPU parity of the routers and the grouping against the oracle: bit-exact
ids, counts, offsets and permutations; weights within one fp32 ulp."""

import numpy as np
import pytest
import torch

from block_quantized_expert_amd import binding as B
from block_quantized_expert_amd import inputs as I
from oracle import moe_oracle as O

from moe_testlib import assert_w_close, oracle_routing

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _route(logits_np, k, scale=1.5):
    ids, w = B.moe_route(torch.from_numpy(logits_np).to(DEV), k, scale)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "decode1", "decode32", "prefill512"])
def test_route_workloads(name):
    wl = I.WORKLOADS[name]
    print("case route", name, flush=True)
    lg = I.router_logits(wl).numpy()
    ids, w = _route(lg, wl.top_k, wl.routed_scale)
    rids, rw = O.route_topk(lg, wl.top_k, wl.routed_scale)
    assert np.array_equal(ids, rids)
    assert_w_close(w, rw)


@pytest.mark.parametrize("n,e,k", [(37, 16, 1), (9, 100, 8), (5, 1024, 8), (70, 257, 6),
                                   (3, 64, 64 // 8)])
def test_route_shapes(n, e, k):
    print("case route shapes", n, e, k, flush=True)
    lg = np.random.default_rng(n * 1000 + e).standard_normal((n, e)).astype(np.float32)
    ids, w = _route(lg, k)
    rids, rw = O.route_topk(lg, k, 1.5)
    assert np.array_equal(ids, rids)
    assert_w_close(w, rw)


def test_route_ties_and_signed_zero():
    print("case route ties", flush=True)
    lg = np.zeros((4, 130), dtype=np.float32)
    lg[0, [5, 70, 129]] = 2.0                 # three-way tie across lanes and words
    lg[1, :] = -0.0
    lg[1, [64, 3]] = 0.0                      # +0 and -0 tie: index order decides
    lg[2, :] = 0.75                           # everything tied
    lg[3, :] = np.linspace(-1, 1, 130, dtype=np.float32)
    lg[3, [0, 128]] = 5.0
    ids, w = _route(lg, 6)
    rids, rw = O.route_topk(lg, 6, 1.5)
    assert np.array_equal(ids, rids)
    assert ids[0, :3].tolist() == [5, 70, 129]
    assert ids[2].tolist() == [0, 1, 2, 3, 4, 5]
    assert_w_close(w, rw)


def test_route_hash_workload_and_bad_tokens():
    wl = I.WORKLOADS["hash4096"]
    print("case route_hash", flush=True)
    r = I.routing_inputs(wl)
    tok = r["token_ids"].clone()
    tok[7] = -3
    tok[100] = wl.vocab
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids, w = B.moe_route_hash(tok.to(DEV), r["tid2eid"].to(DEV), r["tid2w"].to(DEV),
                              wl.n_experts, dev_error=err)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    good = np.ones(wl.n_tokens, bool)
    good[[7, 100]] = False
    rids, rw = O.route_hash(tok.numpy()[good], r["tid2eid"].numpy(), r["tid2w"].numpy())
    assert np.array_equal(ids[good], rids) and np.array_equal(w[good], rw)
    assert np.all(ids[~good] == -1) and np.all(w[~good] == 0)
    assert int(err.item()) == B.MOE_DEVERR_TOKEN_ID


def _group(ids_np, e, err=None):
    out = B.moe_group(torch.from_numpy(ids_np.astype(np.int32)).to(DEV), e, dev_error=err)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _check_group(ids_np, e):
    counts, offsets, perm, inv = _group(ids_np, e)
    rc, ro, rp, ri = O.group(ids_np, e)
    assert np.array_equal(counts, rc)
    assert np.array_equal(offsets, ro)
    assert np.array_equal(perm, rp)
    assert np.array_equal(inv, ri)


@pytest.mark.parametrize("name", ["tiny", "decode1", "decode32", "prefill512", "hash4096"])
def test_group_workloads(name):
    wl = I.WORKLOADS[name]
    print("case group", name, flush=True)
    rids, _ = oracle_routing(wl, I.routing_inputs(wl))
    _check_group(rids, wl.n_experts)


@pytest.mark.parametrize("n,k,e,seed", [(3000, 8, 1000, 1), (129, 8, 1024, 2), (500, 1, 1, 3),
                                        (1, 8, 8, 4), (2049, 3, 7, 5), (4096, 6, 256, 6),
                                        (70001, 6, 256, 7)])
def test_group_random(n, k, e, seed):
    print("case group random", n, k, e, flush=True)
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    _check_group(ids, e)


def test_group_skewed_and_repeated_ids():
    # one expert takes almost everything (repeats are not excluded here)
    print("case group skewed", flush=True)
    rng = np.random.default_rng(9)
    ids = np.where(rng.random((2500, 4)) < 0.9, 17, rng.integers(0, 64, (2500, 4))).astype(np.int32)
    _check_group(ids, 64)


def test_group_out_of_range_ids():
    print("case group bad ids", flush=True)
    rng = np.random.default_rng(4)
    ids = rng.integers(0, 32, size=(300, 4)).astype(np.int32)
    ids[5, 1] = -1
    ids[250, 3] = 32
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    counts, offsets, perm, inv = _group(ids, 32, err)
    flat = ids.reshape(-1)
    good = (flat >= 0) & (flat < 32)
    assert int(err.item()) == B.MOE_DEVERR_EXPERT_ID
    assert np.all(inv[~good] == -1)
    assert counts.sum() == good.sum() == offsets[-1]
    ref = np.flatnonzero(good)[np.argsort(flat[good], kind="stable")]
    assert np.array_equal(perm[:good.sum()], ref)
    assert np.array_equal(inv[perm[:good.sum()]], np.arange(good.sum()))


def test_group_empty():
    print("case group empty", flush=True)
    dev_ids = torch.zeros((0, 6), dtype=torch.int32, device=DEV)
    counts = torch.full((256,), 7, dtype=torch.int32, device=DEV)
    offsets = torch.full((257,), 7, dtype=torch.int32, device=DEV)
    perm = torch.zeros(1, dtype=torch.int32, device=DEV)
    inv = torch.zeros(1, dtype=torch.int32, device=DEV)
    B.moe_group(dev_ids, 256, out=(counts, offsets, perm, inv))
    torch.cuda.synchronize()
    assert counts.abs().sum().item() == 0 and offsets.abs().sum().item() == 0


def test_route_and_group_deterministic():
    wl = I.WORKLOADS["prefill512"]
    print("case determinism route+group", flush=True)
    lg = I.router_logits(wl).to(DEV)
    a = B.moe_route(lg, wl.top_k)
    ga = B.moe_group(a[0], wl.n_experts)
    b = B.moe_route(lg, wl.top_k)
    gb = B.moe_group(b[0], wl.n_experts)
    torch.cuda.synchronize()
    for x, y in zip(list(a) + list(ga), list(b) + list(gb)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name,n_tokens", [("tiny", None), ("tiny", 32), ("tiny", 33),
                                           ("decode1", None), ("decode32", None),
                                           ("decode32", 17), ("decode32", 64),
                                           ("decode32", 65), ("prefill512", None),
                                           ("prefill512", 1000)])
def test_route_group_fused_equals_oracle(name, n_tokens):
    # up to 64 flat entries: one wavefront; up to 64 tokens (one to four per
    # wavefront) and 4096 entries: one workgroup; more tokens: a routing
    # kernel and a grouping kernel
    wl = I.WORKLOADS[name]
    print("case route_group", name, n_tokens, flush=True)
    lg = I.router_logits(wl, n_tokens=n_tokens)
    ids, w, g = B.moe_route_group(lg.to(DEV), wl.top_k, wl.routed_scale)
    torch.cuda.synchronize()
    rids, rw = O.route_topk(lg.numpy(), wl.top_k, wl.routed_scale)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert_w_close(w.cpu().numpy(), rw)
    for got, ref in zip(g, O.group(rids, wl.n_experts)):
        assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("n,e,k", [
    (10, 16, 8), (20, 16, 8), (12, 256, 6),              # 1 and 4 experts a lane
    (2, 100, 8), (12, 100, 8), (30, 100, 8), (60, 100, 8),     # 2 experts a lane
    (3, 500, 6), (14, 500, 6), (25, 500, 6), (50, 500, 6),     # 8
    (7, 1000, 8), (16, 1000, 8), (31, 1000, 8), (64, 1000, 8),  # 16
])
def test_route_group_fused_expert_widths(n, e, k):
    """The fused route+group kernels at every experts-per-lane width and
    tokens-per-wavefront count: N*k <= 64 runs on one wavefront, else one
    workgroup takes one, two or four tokens per wavefront."""
    print("case route_group widths", n, e, k, flush=True)
    lg = torch.from_numpy(I.spaced_logits(np.random.default_rng(7000 + 13 * n + e), n,
                                          np.zeros(e), 1e-3))
    ids, w, g = B.moe_route_group(lg.to(DEV), k, 1.5)
    torch.cuda.synchronize()
    rids, rw = O.route_topk(lg.numpy(), k, 1.5)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert_w_close(w.cpu().numpy(), rw)
    for got, ref in zip(g, O.group(rids, e)):
        assert np.array_equal(got.cpu().numpy(), ref)

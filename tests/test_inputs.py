"""The seeded input generator: determinism, the recipe's properties, and
that per-expert regeneration reproduces the stacked layer bytes."""

import numpy as np
import pytest
import torch

from block_quantized_expert_amd import inputs as I
from oracle import moe_oracle as O


def test_hash_words_known_values():
    # fmix32 of the Weyl sequence is exact integer arithmetic; the torch
    # version must agree with plain Python integers.
    key = I.stream_key(1, 2, 3)
    got = I.hash_words(key, 5, 4, "cpu").tolist()
    exp = [I._py_fmix32((((5 + j) * I._GOLDEN) + key) & I._M32) for j in range(4)]
    assert got == exp


def test_bytes_reproducible_and_uniform():
    a = I.random_bytes(I.stream_key(9), 0, 1 << 20, "cpu")
    b = I.random_bytes(I.stream_key(9), 0, 1 << 20, "cpu")
    assert torch.equal(a, b)
    hist = torch.bincount(a.long(), minlength=256).double()
    assert hist.min() > 0.9 * hist.mean() and hist.max() < 1.1 * hist.mean()
    # an offset start continues the same stream
    c = I.random_bytes(I.stream_key(9), 4096, 1024, "cpu")
    assert torch.equal(c, a[4096:4096 + 1024])


def test_single_expert_matches_stacked_layer():
    wl = I.WORKLOADS["tiny"]
    full = I.make_layer(wl)
    part = I.make_layer(wl, experts=[3, 11])
    for proj in ("gate", "up", "down"):
        for e in (3, 11):
            assert torch.equal(full[proj]["codes"][e], part[proj]["codes"][e])
            assert torch.equal(full[proj]["scales"][e], part[proj]["scales"][e])
    assert full["gate"]["codes"].shape == (16, 128, 128)
    assert full["down"]["scales"].shape == (16, 256, 4)
    s = full["gate"]["scales"]
    assert int(s.min()) == 121 and int(s.max()) == 124


def test_fp8_routed_experts_match_stacked_layer():
    # routed experts in fp8-e4m3 (one UE8M0 per 1x128): regenerating some
    # alone gives the stacked bytes; matrix 0 of the shared expert's stream
    # is the one-matrix shared generator
    from dataclasses import replace
    wl = replace(I.WORKLOADS["tiny"], routed="fp8_e4m3_b128")
    full = I.make_layer(wl)
    part = I.make_layer(wl, experts=[0, 9])
    for proj in ("gate", "up", "down"):
        assert full[proj]["type"] == "fp8_e4m3_b128"
        for e in (0, 9):
            assert torch.equal(full[proj]["codes"][e], part[proj]["codes"][e])
            assert torch.equal(full[proj]["scales"][e], part[proj]["scales"][e])
    assert full["gate"]["codes"].shape == (16, 128, 256)
    assert full["gate"]["scales"].shape == (16, 128, 2)
    assert full["down"]["codes"].shape == (16, 256, 128)
    assert full["down"]["scales"].shape == (16, 256, 1)
    c, sc = I._fp8_matrix(wl, "shared_up", 0, "cpu")
    cb, sb = I._fp8_block(wl, "shared_up", 0, 0, 1, "cpu")
    assert torch.equal(c, cb[0]) and torch.equal(sc, sb[0])


def test_fp8_shared_codes_are_finite_and_cover_subnormals():
    wl = I.WORKLOADS["hash4096"]
    c, s = I._fp8_matrix(wl, "shared_gate", 0, "cpu")
    assert c.shape == (2048, 4096) and s.shape == (2048, 32)
    cc = c.numpy()
    assert not np.any((cc & 0x7F) == 0x7F)
    e = (cc >> 3) & 15
    assert e.min() == 0 and e.max() == 10
    assert int(s.min()) == 119 and int(s.max()) == 123


def test_logits_spacing_and_bf16_activations():
    wl = I.WORKLOADS["decode32"]
    lg = I.router_logits(wl).numpy()
    srt = np.sort(lg.astype(np.float64), axis=1)
    assert np.diff(srt, axis=1).min() >= 1e-3
    x = I.activations(wl)
    assert x.dtype == torch.bfloat16 and x.shape == (32, 4096)
    assert torch.equal(I.activations(wl), x)


def test_decode32_routing_recipe_property():
    # counts in 0..6 with some odd count >= 3 (uneven, odd per-expert counts)
    wl = I.WORKLOADS["decode32"]
    ids, _ = O.route_topk(I.router_logits(wl).numpy(), wl.top_k, wl.routed_scale)
    counts = np.bincount(ids.reshape(-1), minlength=wl.n_experts)
    assert counts.max() <= 6
    assert any(c % 2 == 1 and c >= 3 for c in counts)


def test_prefill512_routing_recipe_property():
    # Zipf popularity: some experts get 40+ tokens, many get 1..11
    wl = I.WORKLOADS["prefill512"]
    ids, _ = O.route_topk(I.router_logits(wl).numpy(), wl.top_k, wl.routed_scale)
    counts = np.bincount(ids.reshape(-1), minlength=wl.n_experts)
    assert counts.max() >= 40
    assert ((counts >= 1) & (counts <= 11)).sum() >= 100


def test_hash_table_rows_distinct():
    wl = I.WORKLOADS["hash4096"]
    tid2eid, tid2w = I.hash_table(wl)
    t = tid2eid.numpy()
    assert t.shape == (129280, 6) and t.min() >= 0 and t.max() < 256
    srt = np.sort(t, axis=1)
    assert np.all(np.diff(srt, axis=1) > 0)
    assert np.all(tid2w.numpy() == np.float32(0.25))
    tok = I.token_ids(wl).numpy()
    assert tok.shape == (4096,) and tok.min() >= 0 and tok.max() < 129280

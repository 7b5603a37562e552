"""Pins of the oracle's group-limited routing, tail pruning, dropped-slot
grouping and gate-first lazy skip against what the pages and the
mathematics fix: brute force over subsets on tiny inputs, hand-worked
examples, closed forms and invariants (no GPU).

Pages: "DeepSeek-V4-Flash 284B (13.17B Active) -- Deep-Dive Mathematical &
Kernel Guide", section 1 (SQRT_SOFTPLUS gating with expert group top-k
selection) and section 3.2 item 3 (L2-quadrature rescaling after pruning,
and the hash weight list [0.30, 0.29, 0.24, 0.23, 0.22, 0.22]); "[RFC /
Benchmarks] Fitting 284B DeepSeek-V4-Flash in 57.61 GiB RAM", section 5
(p_early pruning, gate-first lazy SwiGLU skip when max |SiLU(g)| < 1e-3).
"""

import math
from itertools import combinations

import numpy as np
import pytest

from block_quantized_expert_amd import inputs as I
from oracle import moe_oracle as O


def _s(v):
    # sqrt(softplus(v)) straight from its definition, for hand cases
    return math.sqrt(math.log(1.0 + math.exp(v)))


# ------------------------------------------------------- group-limited routing


def test_one_group_without_bias_is_plain_top_k():
    rng = np.random.default_rng(21)
    for e, k in [(16, 2), (64, 6), (256, 6), (256, 8)]:
        lg = I.spaced_logits(rng, 8, np.zeros(e), 1e-3)
        ids_a, w_a = O.route_grouped(lg, k, 1.5, n_group=1, topk_group=1)
        ids_b, w_b = O.route_topk(lg, k, 1.5)
        assert np.array_equal(ids_a, ids_b)
        assert np.array_equal(w_a, w_b)


def test_all_groups_kept_is_top_k_of_the_keys_by_rank_count():
    # expert e is chosen iff fewer than k experts beat it (a larger key, or
    # an equal key and a lower index); slots in that rank order
    rng = np.random.default_rng(22)
    for _ in range(50):
        e, ng = 16, 4
        lg = rng.integers(-4, 5, size=(1, e)).astype(np.float32) / 2
        b = rng.integers(-2, 3, size=e).astype(np.float32) / 4
        k = int(rng.integers(1, 7))
        ids, _ = O.route_grouped(lg, k, 1.5, n_group=ng, topk_group=ng, bias=b)
        key = [_s(float(lg[0, j])) + float(b[j]) for j in range(e)]
        rank = [sum(1 for j in range(e) if key[j] > key[x] or (key[j] == key[x] and j < x))
                for x in range(e)]
        expect = sorted((x for x in range(e) if rank[x] < k), key=lambda x: rank[x])
        assert ids[0].tolist() == expect


def test_grouped_selection_brute_force():
    # group score = the largest sum over pairs of distinct members' keys;
    # the chosen groups are those fewer than topk_group groups beat; the
    # experts are the best k-subset of their members by exhaustive search
    rng = np.random.default_rng(23)
    for _ in range(150):
        ng = int(rng.choice([2, 4]))
        e = ng * int(rng.choice([2, 3]))
        gs = e // ng
        tg = int(rng.integers(1, ng + 1))
        k = int(rng.integers(1, tg * gs + 1))
        lg = rng.integers(-3, 4, size=(1, e)).astype(np.float32) / 2  # many ties
        b = rng.integers(-2, 3, size=e).astype(np.float32) / 2
        ids, w = O.route_grouped(lg, k, 1.5, n_group=ng, topk_group=tg, bias=b)
        key = [_s(float(lg[0, j])) + float(b[j]) for j in range(e)]
        score = [max(key[a] + key[c] for a, c in combinations(range(g * gs, (g + 1) * gs), 2))
                 for g in range(ng)]
        chosen_g = [g for g in range(ng)
                    if sum(1 for h in range(ng)
                           if score[h] > score[g] or (score[h] == score[g] and h < g)) < tg]
        cand = [x for g in chosen_g for x in range(g * gs, (g + 1) * gs)]
        best = None
        for sub in combinations(cand, k):
            order = sorted(((-key[j], j) for j in sub))
            if best is None or order < best[0]:
                best = (order, [j for _, j in order])
        assert ids[0].tolist() == best[1]
        s = [_s(float(lg[0, j])) for j in best[1]]
        assert np.allclose(w[0], [1.5 * v / sum(s) for v in s], rtol=1e-6, atol=0)


def test_group_score_is_the_sum_of_the_two_largest_keys():
    # equal logits, so the keys differ by the bias alone.  Group scores by
    # top-2 sum: g0 .3, g1 3.0, g2 3.2, g3 1.0 -> groups 2 and 1, experts
    # 2 (3.0), then 4 and 5 (1.6 each, lower index first).  Scoring groups
    # by their maximum alone would pick groups 1 and 3 and experts 2, 6, 3.
    lg = np.zeros((1, 8), dtype=np.float32)
    b = np.array([0.1, 0.2, 3.0, 0.0, 1.6, 1.6, 2.0, -1.0], dtype=np.float32)
    ids, w = O.route_grouped(lg, 3, 1.5, n_group=4, topk_group=2, bias=b)
    assert ids.tolist() == [[2, 4, 5]]
    assert np.allclose(w, 0.5, rtol=0, atol=1e-7)  # equal unbiased scores


def test_tied_group_scores_go_to_the_lower_group():
    # every key equal: every group scores the same, groups 0 and 1 are kept
    lg = np.zeros((1, 8), dtype=np.float32)
    ids, _ = O.route_grouped(lg, 3, 1.5, n_group=4, topk_group=2)
    assert ids.tolist() == [[0, 1, 2]]
    # groups 1 and 3 tie above the rest: group 1 first, then group 3 over 2
    b = np.array([0.0, 0.0, 1.0, 1.0, 0.5, 0.5, 1.0, 1.0], dtype=np.float32)
    ids, _ = O.route_grouped(lg, 4, 1.5, n_group=4, topk_group=2, bias=b)
    assert ids.tolist() == [[2, 3, 6, 7]]
    ids, _ = O.route_grouped(lg, 2, 1.5, n_group=4, topk_group=1, bias=b)
    assert ids.tolist() == [[2, 3]]


def test_selection_bias_does_not_enter_the_weights():
    # scores: s = 2 (softplus = 4), s = 1 (softplus = 1), s(-3), s(-5); a bias
    # of 10 on expert 3 puts it first; its weight uses s(-5) only
    lg = np.array([[math.log(math.e ** 4 - 1.0), math.log(math.e - 1.0), -3.0, -5.0]],
                  dtype=np.float32)
    b = np.array([0.0, 0.0, 0.0, 10.0], dtype=np.float32)
    ids, w = O.route_grouped(lg, 2, 1.5, n_group=1, topk_group=1, bias=b)
    assert ids.tolist() == [[3, 0]]
    s3 = _s(float(lg[0, 3]))
    assert w[0, 0] == pytest.approx(1.5 * s3 / (s3 + 2.0), rel=1e-6)
    assert w[0, 1] == pytest.approx(1.5 * 2.0 / (s3 + 2.0), rel=1e-6)
    assert float(np.sum(w, dtype=np.float64)) == pytest.approx(1.5, abs=1e-6)


# ------------------------------------------------------------- tail pruning


def test_prune_equal_weights_closed_form():
    # six equal weights, four kept: alpha = sqrt(6/4); the lower slots win ties
    ids = np.arange(6, dtype=np.int32)[None, :]
    w = np.full((1, 6), 0.25, dtype=np.float32)
    pid, pw = O.prune_tail(ids, w, 4, 0.0)
    assert pid.tolist() == [[0, 1, 2, 3, -1, -1]]
    assert np.allclose(pw[0, :4], 0.30618621784789724, rtol=1e-7)  # 0.25 * sqrt(1.5)
    assert pw[0, 4] == 0 and pw[0, 5] == 0


def test_prune_the_guides_flat_hash_list():
    # the Guide's per-rank hash weights [0.30, 0.29, 0.24, 0.23, 0.22, 0.22]
    # kept to four: sum of squares 0.3814 over 0.2846 (by hand),
    # alpha = 1.1576383...
    ids = np.array([[7, 3, 11, 0, 5, 9]], dtype=np.int32)
    w = np.array([[0.30, 0.29, 0.24, 0.23, 0.22, 0.22]], dtype=np.float32)
    pid, pw = O.prune_tail(ids, w, 4, 0.0)
    assert pid.tolist() == [[7, 3, 11, 0, -1, -1]]
    assert np.allclose(pw[0, :4], np.array([0.30, 0.29, 0.24, 0.23]) * 1.1576383,
                       rtol=2e-7)


def test_prune_threshold_and_at_least_one_kept():
    ids = np.array([[4, 1, 2, 0, 3, 5]], dtype=np.int32)
    w = np.array([[0.5, 0.4, 0.3, 0.15, 0.1, 0.05]], dtype=np.float32)
    pid, _ = O.prune_tail(ids, w, 6, 0.11)  # the Guide's adaptive tail min_w
    assert pid.tolist() == [[4, 1, 2, 0, -1, -1]]
    # "below the threshold" is strict: a weight equal to min_w stays
    pid, _ = O.prune_tail(ids, w, 6, np.float32(0.15))
    assert pid.tolist() == [[4, 1, 2, 0, -1, -1]]
    pid, _ = O.prune_tail(ids, w, 6, np.float32(0.1))
    assert pid.tolist() == [[4, 1, 2, 0, 3, -1]]
    pid, pw = O.prune_tail(ids, w, 6, 10.0)  # nothing reaches it: keep the largest
    assert pid.tolist() == [[4, -1, -1, -1, -1, -1]]
    # alpha = sqrt(sum w^2) / 0.5 = 0.7353910...: the kept weight alone
    # carries the whole L2 norm
    assert pw[0, 0] == pytest.approx(math.sqrt(0.25 + 0.16 + 0.09 + 0.0225 + 0.01 + 0.0025),
                                     rel=1e-6)


def test_prune_keeps_the_l2_norm_and_the_ratios():
    rng = np.random.default_rng(24)
    lg = rng.standard_normal((200, 64)).astype(np.float32)
    ids, w = O.route_topk(lg, 6, 1.5)
    pid, pw = O.prune_tail(ids, w, 4, 0.2)
    w64, p64 = w.astype(np.float64), pw.astype(np.float64)
    assert np.allclose((p64 ** 2).sum(1), (w64 ** 2).sum(1), rtol=1e-6)
    for t in range(200):
        kept = pid[t] >= 0
        assert 1 <= kept.sum() <= 4
        assert np.array_equal(pid[t][kept], ids[t][kept])
        ratio = p64[t][kept] / w64[t][kept]
        assert np.allclose(ratio, ratio[0], rtol=1e-6) and ratio[0] >= 1.0
        # dropped: below the threshold, or beyond the four largest
        if (~kept).any():
            assert w[t][~kept].max() <= w[t][kept].min()


def test_no_pruning_is_the_identity():
    rng = np.random.default_rng(25)
    lg = rng.standard_normal((50, 32)).astype(np.float32)
    ids, w = O.route_topk(lg, 6, 1.5)
    pid, pw = O.prune_tail(ids, w, 6, 0.0)
    assert np.array_equal(pid, ids) and np.array_equal(pw, w)


# ------------------------------------------------------- dropped slots, lazy


def test_group_skips_dropped_slots():
    ids = np.array([[3, -1, 0], [0, 3, -1], [-1, -1, 2]], dtype=np.int32)
    counts, offsets, perm, inv = O.group(ids, 4)
    assert counts.tolist() == [2, 0, 1, 2]
    assert offsets.tolist() == [0, 2, 2, 3, 5]
    flat = ids.reshape(-1)
    valid = np.nonzero(flat >= 0)[0]
    assert perm.tolist() == valid[np.argsort(flat[valid], kind="stable")].tolist()
    assert inv.tolist() == [3, -1, 0, 1, 4, -1, -1, -1, 2]


def _layer(rng, h=64, i=32, e=4):
    def proj(rows, cols, n):
        return {"type": "mxfp4", "codes": rng.integers(0, 256, (n, rows, cols // 2), dtype=np.uint8),
                "scales": rng.integers(121, 125, (n, rows, cols // 32), dtype=np.uint8)}
    return {"hidden": h, "inter": i, "n_experts": e, "gate": proj(i, h, e), "up": proj(i, h, e),
            "down": proj(h, i, e),
            "shared": {"inter": i, "gate": proj(i, h, 1), "up": proj(i, h, 1),
                       "down": proj(h, i, 1)}}


def _unstack_shared(layer):
    for m in ("gate", "up", "down"):
        layer["shared"][m]["codes"] = layer["shared"][m]["codes"][0]
        layer["shared"][m]["scales"] = layer["shared"][m]["scales"][0]
    return layer


def test_dropped_slot_equals_zero_weight():
    rng = np.random.default_rng(26)
    layer = _unstack_shared(_layer(rng))
    x = rng.standard_normal((3, 64)).astype(np.float32)
    ids = np.array([[1, 3], [0, 1], [3, 2]], dtype=np.int32)
    w = np.array([[1.0, 0.5], [0.9, 0.6], [1.25, 0.25]], dtype=np.float32)
    dropped = ids.copy()
    dropped[0, 1] = -1
    dropped[2, 0] = -1
    w0 = w.copy()
    w0[0, 1] = 0.0
    w0[2, 0] = 0.0
    assert np.array_equal(O.ffn(layer, x, "f32", dropped, w), O.ffn(layer, x, "f32", ids, w0))


def test_lazy_skip_of_a_gate_dead_expert():
    # expert 2's gate rows all hold code 0x22 (every weight 1.0 with scale
    # byte 127), so g_j = sum(x) for every row j; its up rows likewise with
    # scale byte 135 (every weight 256), so u_j = 256 sum(x).  Token 0 has
    # sum(x) = -10: |SiLU(-10)| = 10 / (1 + e^10) = 4.54e-4, below 1e-3 (the
    # RFC's threshold), so expert 2 is skipped for it although its h_j =
    # SiLU(-10) * (-2560) = 1.16 is not small; token 1 has sum(x) = 2:
    # SiLU(2) = 1.76, kept.
    rng = np.random.default_rng(27)
    layer = _unstack_shared(_layer(rng))
    layer["gate"]["codes"][2][:] = 0x22
    layer["gate"]["scales"][2][:] = 127
    layer["up"]["codes"][2][:] = 0x22
    layer["up"]["scales"][2][:] = 135
    x = rng.standard_normal((2, 64)).astype(np.float32)
    x[0] += np.float32((-10.0 - float(x[0].astype(np.float64).sum())) / 64)
    x[1] += np.float32((2.0 - float(x[1].astype(np.float64).sum())) / 64)
    assert abs(x[0].astype(np.float64).sum() + 10) < 1e-3
    ids = np.array([[2, 0], [2, 1]], dtype=np.int32)
    w = np.array([[0.9, 0.6], [1.0, 0.5]], dtype=np.float32)
    y_lazy = O.ffn(layer, x, "f32", ids, w, lazy_tau=1e-3)
    w_ref = w.copy()
    w_ref[0, 0] = 0.0  # token 0 without expert 2
    assert np.array_equal(y_lazy, O.ffn(layer, x, "f32", ids, w_ref))
    y_full = O.ffn(layer, x, "f32", ids, w)
    assert not np.allclose(y_lazy[0], y_full[0], rtol=1e-3)  # the skip is visible
    assert np.array_equal(y_lazy[1], y_full[1])
    # a threshold below |SiLU(-10)| keeps it
    assert np.array_equal(O.ffn(layer, x, "f32", ids, w, lazy_tau=4e-4), y_full)
    # an all-zero gate is dead for every token; a threshold of 0 skips nothing
    layer["gate"]["codes"][0][:] = 0
    y2 = O.ffn(layer, x, "f32", ids, w, lazy_tau=1e-3)
    w2 = w_ref.copy()
    w2[0, 1] = 0.0
    assert np.array_equal(y2, O.ffn(layer, x, "f32", ids, w2))
    assert np.array_equal(O.ffn(layer, x, "f32", ids, w, lazy_tau=0.0),
                          O.ffn(layer, x, "f32", ids, w))

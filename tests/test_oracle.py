"""Pins of the fp64 oracle against things other than itself.

Each test names what fixes the expected value: a format specification table
(tests/golden), a closed form, a value the pages print, an invariant the
pages state, a library routine, or brute force written independently of the
oracle's vectorised code.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((a, float(b)))
    return rows


# ---------------------------------------------------------------- formats


def test_e2m1_matches_ocp_table():
    for code, val in _read_table("e2m1_table.txt"):
        got = O.e2m1_value(int(code))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_matches_ocp_points():
    for code, val in _read_table("e4m3_points.txt"):
        got = O.e4m3_value(int(code, 16))
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_all_codes_structure():
    # 126 positive finite codes, strictly increasing; negatives mirror them;
    # exactly two NaN codes.
    pos = [O.e4m3_value(c) for c in range(0x00, 0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    for c in range(0x00, 0x7F):
        assert O.e4m3_value(c | 0x80) == -O.e4m3_value(c)
    nans = [c for c in range(256) if math.isnan(O.e4m3_value(c))]
    assert nans == [0x7F, 0xFF]
    # steps are m * 2**-9 below 2**-6 and 2**(e-10) above: max 448
    assert max(pos) == 448.0


def test_ue8m0_is_power_of_two_with_bias_127():
    assert O.ue8m0_value(127) == 1.0
    assert O.ue8m0_value(128) == 2.0
    assert O.ue8m0_value(0) == 2.0 ** -127
    assert O.ue8m0_value(254) == 2.0 ** 127
    assert math.isnan(O.ue8m0_value(255))


def test_bf16_widening_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_mxfp4_every_code_and_every_finite_scale():
    # One row per scale byte 0..254; each 32-block holds codes 0..15 twice.
    # The expected value of element j is the format table value of the code
    # at j times 2**(u-127), read element by element from the bytes.
    table = dict((int(c), v) for c, v in _read_table("e2m1_table.txt"))
    cols = 32
    rows = 255
    elem_codes = np.array([j % 16 for j in range(cols)], dtype=np.uint8)
    packed = (elem_codes[0::2] | (elem_codes[1::2] << 4)).astype(np.uint8)
    codes = np.tile(packed, (rows, 1))
    scales = np.arange(rows, dtype=np.uint8).reshape(rows, 1)
    got = O.decode_mxfp4(codes, scales, cols)
    for u in range(rows):
        for j in range(cols):
            exp = table[j % 16] * (2.0 ** (u - 127))
            assert got[u, j] == exp, (u, j)


def test_mxfp4_hand_example_nibble_order_and_block_axis():
    # Row of 64 elements = two 32-blocks.  Byte 0 = 0x72: element 0 is the
    # low nibble (code 2 -> 1.0), element 1 the high nibble (code 7 -> 6.0).
    # Byte 16 = 0x9C opens block 1: element 32 code 0xC (-2.0), element 33
    # code 0x9 (-0.5).  Block 0 scale 2**1, block 1 scale 2**-2.
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x72
    codes[0, 16] = 0x9C
    scales = np.array([[128, 125]], dtype=np.uint8)
    got = O.decode_mxfp4(codes, scales, 64)[0]
    assert got[0] == 2.0 and got[1] == 12.0
    assert got[32] == -0.5 and got[33] == -0.125
    assert np.count_nonzero(got) == 4


def test_fp8_block128_scale_axis():
    codes = np.full((2, 256), 0x38, dtype=np.uint8)  # 1.0 everywhere
    scales = np.array([[127, 129], [120, 126]], dtype=np.uint8)
    got = O.decode_fp8_b128(codes, scales, 256)
    assert np.all(got[0, :128] == 1.0) and np.all(got[0, 128:] == 4.0)
    assert np.all(got[1, :128] == 2.0 ** -7) and np.all(got[1, 128:] == 0.5)


def test_products_are_exact_in_bf16_for_workload_scales():
    # Every e2m1 value times every UE8M0 byte 119..124, and every finite
    # e4m3 value times bytes 119..123, is a bf16 number: bf16 keeps 8
    # significant bits and the exponent range of fp32.
    vals = [O.e2m1_value(c) * 2.0 ** (u - 127) for c in range(16) for u in range(119, 125)]
    vals += [O.e4m3_value(c) * 2.0 ** (u - 127) for c in range(256) for u in range(119, 124)
             if not math.isnan(O.e4m3_value(c))]
    t = torch.tensor(vals, dtype=torch.float64)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)


# ---------------------------------------------------------------- SwiGLU


def test_silu_minimum_matches_printed_value():
    # The Kernel Guide (section 4) prints max over g<=0 of |SiLU(g)| = 0.2785.
    g = np.linspace(-6.0, 0.0, 600001)
    s = O.silu(g)
    assert abs(-s.min() - 0.2785) < 5e-5
    assert abs(g[np.argmin(s)] - (-1.27846)) < 1e-4


def test_silu_second_moment_near_printed_constant():
    # The RFC (section 1) states E[SiLU(z)^2] = 7/20 = 0.35 for unit
    # variance; a Monte-Carlo estimate lands near 0.356.
    z = np.random.default_rng(0).standard_normal(2_000_000)
    m = float(np.mean(O.silu(z) ** 2))
    assert abs(m - 0.35) < 0.01


def test_silu_limits():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([-1000.0]))[0] == 0.0
    assert O.silu(np.array([50.0]))[0] == pytest.approx(50.0, rel=1e-15)


# ---------------------------------------------------------------- routing


def test_softplus_closed_forms():
    assert O.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert O.softplus(math.log(math.e - 1.0)) == pytest.approx(1.0, rel=1e-14)
    assert O.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-12)
    assert O.softplus(40.0) == pytest.approx(40.0, rel=1e-15)


def test_route_weight_closed_form():
    # softplus(ln(e^4-1)) = 4 and softplus(ln(e-1)) = 1, so the scores are
    # 2 and 1 and the weights 1.5*2/3 = 1.0 and 1.5*1/3 = 0.5.
    lg = np.array([[math.log(math.e - 1.0), -3.0, math.log(math.e ** 4 - 1.0), -5.0]],
                  dtype=np.float32)
    ids, w = O.route_topk(lg, 2, 1.5)
    assert ids.tolist() == [[2, 0]]
    assert w[0, 0] == pytest.approx(1.0, abs=1e-6)
    assert w[0, 1] == pytest.approx(0.5, abs=1e-6)


def test_route_ties_go_to_lower_index():
    lg = np.array([[0.5, 1.0, 1.0, 0.25, 1.0, -0.0, 0.0]], dtype=np.float32)
    ids, w = O.route_topk(lg, 5, 1.5)
    assert ids.tolist() == [[1, 2, 4, 0, 3]]
    lg2 = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)  # -0 equals +0
    ids2, _ = O.route_topk(lg2, 1, 1.5)
    assert ids2.tolist() == [[0]]


def test_route_all_equal_logits():
    lg = np.full((3, 8), 0.75, dtype=np.float32)
    ids, w = O.route_topk(lg, 6, 1.5)
    assert ids.tolist() == [[0, 1, 2, 3, 4, 5]] * 3
    assert np.allclose(w, 0.25, rtol=0, atol=1e-7)


def test_route_brute_force_tiny():
    # Brute force: the chosen set is the k-subset whose sorted logits are
    # lexicographically largest with ties broken by index; check against an
    # exhaustive search over all subsets.
    from itertools import combinations
    rng = np.random.default_rng(7)
    for _ in range(200):
        e = int(rng.integers(2, 8))
        k = int(rng.integers(1, e + 1))
        lg = rng.integers(-3, 4, size=(1, e)).astype(np.float32) / 2  # many ties
        ids, w = O.route_topk(lg, k, 1.5)
        best = None
        for sub in combinations(range(e), k):
            key = sorted(((-float(lg[0, j]), j) for j in sub))
            if best is None or key < best[0]:
                best = (key, [j for _, j in key])
        assert ids[0].tolist() == best[1]
        assert abs(float(np.sum(w, dtype=np.float64)) - 1.5) < 1e-6


def test_route_weights_sum_to_routed_scale_and_descend():
    # The Kernel Guide (section 3.2) states sum_i w_i = 1.5.
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((64, 256)).astype(np.float32)
    ids, w = O.route_topk(lg, 6, 1.5)
    assert np.allclose(w.astype(np.float64).sum(1), 1.5, atol=2e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(64):
        assert len(set(ids[t].tolist())) == 6
        assert lg[t, ids[t]].min() >= np.delete(lg[t], ids[t]).max()


def test_route_hash_is_table_lookup():
    tid2eid = np.array([[3, 1], [0, 2], [2, 3]], dtype=np.int32)
    tid2w = np.array([[0.75, 0.75], [0.5, 1.0], [1.2, 0.3]], dtype=np.float32)
    ids, w = O.route_hash(np.array([2, 0, 2]), tid2eid, tid2w)
    assert ids.tolist() == [[2, 3], [3, 1], [2, 3]]
    assert w.tolist() == [[np.float32(1.2), np.float32(0.3)], [0.75, 0.75],
                          [np.float32(1.2), np.float32(0.3)]]


# ---------------------------------------------------------------- grouping


def test_group_matches_stable_argsort_and_invariants():
    rng = np.random.default_rng(11)
    for n, k, e in [(1, 6, 256), (8, 2, 16), (32, 6, 256), (100, 3, 7), (0, 4, 5)]:
        ids = np.stack([rng.permutation(e)[:k] for _ in range(n)]) if n else np.zeros((0, k), np.int32)
        counts, offsets, perm, inv = O.group(ids, e)
        flat = ids.reshape(-1)
        assert counts.sum() == n * k
        assert offsets[0] == 0 and offsets[-1] == n * k
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(inv[perm], np.arange(n * k))
        # every token appears exactly top_k times
        assert np.array_equal(np.bincount(perm // k, minlength=n), np.full(n, k))
        for x in range(e):
            seg = perm[offsets[x]:offsets[x + 1]]
            assert np.all(flat[seg] == x) and np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------- FFN


def _tiny_layer(rng, h, i, e, shared=True, shared_type="mxfp4", scale_range=(121, 125)):
    def mx(rows, cols, n=None):
        shp = (rows, cols // 2) if n is None else (n, rows, cols // 2)
        shs = (rows, cols // 32) if n is None else (n, rows, cols // 32)
        return {"type": "mxfp4",
                "codes": rng.integers(0, 256, size=shp, dtype=np.uint8),
                "scales": rng.integers(*scale_range, size=shs, dtype=np.uint8)}

    def f8(rows, cols):
        codes = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x3C
        return {"type": "fp8_e4m3_b128", "codes": codes,
                "scales": rng.integers(*scale_range, size=(rows, cols // 128), dtype=np.uint8)}

    layer = {"hidden": h, "inter": i, "n_experts": e,
             "gate": mx(i, h, e), "up": mx(i, h, e), "down": mx(h, i, e), "shared": None}
    if shared:
        mk = mx if shared_type == "mxfp4" else f8
        layer["shared"] = {"inter": i, "gate": mk(i, h), "up": mk(i, h), "down": mk(h, i)}
    return layer


def _scalar_element(proj, e, r, c):
    """Element (r, c) of expert e read straight from the bytes."""
    codes = proj["codes"] if e is None else proj["codes"][e]
    scales = proj["scales"] if e is None else proj["scales"][e]
    if proj["type"] == "mxfp4":
        byte = int(codes[r][c // 2])
        nib = (byte >> 4) & 15 if c % 2 else byte & 15
        return O.e2m1_value(nib) * 2.0 ** (int(scales[r][c // 32]) - 127)
    return O.e4m3_value(int(codes[r][c])) * 2.0 ** (int(scales[r][c // 128]) - 127)


def _brute_force_y(layer, xf, ids, w):
    """Scalar loops straight from the SwiGLU and combine equations."""
    h, i = layer["hidden"], layer["inter"]
    n, k = ids.shape
    dense = {}

    def mat(name, e, rows, cols):
        key = (name, e)
        if key not in dense:
            proj = layer[name] if e is not None else layer["shared"][name]
            dense[key] = [[_scalar_element(proj, e, r, c) for c in range(cols)] for r in range(rows)]
        return dense[key]

    def expert(e, x):
        wg, wu, wd = mat("gate", e, i, h), mat("up", e, i, h), mat("down", e, h, i)
        hv = []
        for r in range(i):
            g = sum(wg[r][c] * x[c] for c in range(h))
            u = sum(wu[r][c] * x[c] for c in range(h))
            hv.append(g / (1.0 + math.exp(-g)) * u)
        return [sum(wd[q][r] * hv[r] for r in range(i)) for q in range(h)]

    y = np.zeros((n, h))
    for t in range(n):
        x = [float(v) for v in xf[t]]
        acc = [0.0] * h
        for j in range(k):
            o = expert(int(ids[t, j]), x)
            for q in range(h):
                acc[q] += float(w[t, j]) * o[q]
        if layer["shared"] is not None:
            o = expert(None, x)
            for q in range(h):
                acc[q] += o[q]
        y[t] = acc
    return y


@pytest.mark.parametrize("shared_type", ["mxfp4", "fp8_e4m3_b128"])
def test_ffn_against_scalar_brute_force(shared_type):
    rng = np.random.default_rng(5)
    # fp8 blocks span 128 elements of a row, so that case needs 128 columns
    h, i = (64, 32) if shared_type == "mxfp4" else (128, 128)
    e, n, k = 4, 3, 2
    layer = _tiny_layer(rng, h, i, e, shared_type=shared_type)
    x = rng.standard_normal((n, h)).astype(np.float32)
    ids = np.array([[1, 3], [0, 1], [3, 2]], dtype=np.int32)
    w = np.array([[1.0, 0.5], [0.9, 0.6], [1.25, 0.25]], dtype=np.float32)
    y = O.ffn(layer, x, "f32", ids, w)
    yb = _brute_force_y(layer, x.astype(np.float64), ids, w)
    assert np.allclose(y, yb, rtol=1e-6, atol=1e-6 * np.abs(yb).max())


def test_ffn_all_ones_closed_form():
    # codes 0x22 (both nibbles code 2 = 1.0) with scale byte 127: every
    # weight is 1, so g = u = sum(x), h = SiLU(s) s, o = inter * h.
    h, i, e = 64, 32, 2
    ones = lambda rows, cols, n: {"type": "mxfp4",  # noqa: E731
                                  "codes": np.full((n, rows, cols // 2), 0x22, np.uint8),
                                  "scales": np.full((n, rows, cols // 32), 127, np.uint8)}
    layer = {"hidden": h, "inter": i, "n_experts": e, "gate": ones(i, h, e),
             "up": ones(i, h, e), "down": ones(h, i, e), "shared": None}
    x = np.random.default_rng(1).standard_normal((2, h)).astype(np.float32)
    ids = np.array([[0, 1], [1, 0]], dtype=np.int32)
    w = np.array([[1.0, 0.5], [0.75, 0.75]], dtype=np.float32)
    y = O.ffn(layer, x, "f32", ids, w)
    for t in range(2):
        s = float(np.sum(x[t].astype(np.float64)))
        o = i * s / (1.0 + math.exp(-s)) * s
        assert np.allclose(y[t], np.float32(1.5 * o), rtol=1e-7)


def test_ffn_zero_gate_leaves_only_shared():
    rng = np.random.default_rng(2)
    layer = _tiny_layer(rng, 64, 32, 3)
    for e in range(3):
        layer["gate"]["codes"][e][:] = 0
    x = rng.standard_normal((2, 64)).astype(np.float32)
    ids = np.array([[0, 2], [1, 0]], dtype=np.int32)
    w = np.array([[1.0, 0.5], [0.75, 0.75]], dtype=np.float32)
    y = O.ffn(layer, x, "f32", ids, w)
    ys = O.ffn(layer, x, "f32", ids, np.zeros_like(w))
    assert np.array_equal(y, ys)
    y_routed = O.ffn(layer, x, "f32", ids, w, with_shared=False)
    assert np.all(y_routed == 0)


def test_ffn_scale_byte_increment_doubles_output():
    # Raising every down (or every up) scale byte by one multiplies every
    # expert output by exactly 2, so y doubles exactly in fp64.
    rng = np.random.default_rng(4)
    layer = _tiny_layer(rng, 64, 32, 3)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    ids = np.array([[0, 2], [1, 0], [2, 1]], dtype=np.int32)
    w = np.array([[1.0, 0.5], [0.75, 0.75], [1.1, 0.4]], dtype=np.float32)
    y = O.ffn(layer, x, "f32", ids, w)
    for name in ("down", "up"):
        l2 = {**layer, name: {**layer[name], "scales": layer[name]["scales"] + 1},
              "shared": {**layer["shared"], name: {**layer["shared"][name],
                                                   "scales": layer["shared"][name]["scales"] + 1}}}
        assert np.array_equal(O.ffn(l2, x, "f32", ids, w), 2 * y)


def test_ffn_token_order_and_subsets():
    rng = np.random.default_rng(6)
    layer = _tiny_layer(rng, 64, 32, 4)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    ids = np.array([[0, 1], [2, 3], [1, 2], [3, 0], [0, 2]], dtype=np.int32)
    w = rng.uniform(0.1, 1.0, size=(5, 2)).astype(np.float32)
    y = O.ffn(layer, x, "f32", ids, w)
    p = np.array([3, 0, 4, 1, 2])
    assert np.array_equal(O.ffn(layer, x[p], "f32", ids[p], w[p]), y[p])
    sub = O.ffn(layer, x, "f32", ids, w, tokens=[4, 1], out_rows=[5, 0, 63])
    assert np.array_equal(sub, y[[4, 1]][:, [5, 0, 63]])


def test_bf16_activation_path_equals_f32_path_on_bf16_values():
    rng = np.random.default_rng(8)
    layer = _tiny_layer(rng, 64, 32, 2)
    xb = torch.from_numpy(rng.standard_normal((2, 64)).astype(np.float32)).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    ids = np.array([[0, 1], [1, 0]], dtype=np.int32)
    w = np.array([[1.0, 0.5], [0.75, 0.75]], dtype=np.float32)
    y1 = O.ffn(layer, bits, "bf16", ids, w)
    y2 = O.ffn(layer, xb.float().numpy(), "f32", ids, w)
    assert np.array_equal(y1, y2)

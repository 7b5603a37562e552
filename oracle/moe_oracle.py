"""Plain, slow, fp64 CPU oracle for the routed Mixture-of-Experts FFN.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library; the only thing both sides consume is the seeded
input data made by ``block_quantized_expert_amd.inputs``.

What it computes, and where the pages define it (pages cited by title):

* [Kernel Guide] "DeepSeek-V4-Flash 284B (13.17B Active) -- Deep-Dive
  Mathematical & Kernel Guide" (llama-modchip):
  - section 1 (Architectural Profile): 256 routed experts + 1 shared, 6 routed
    experts active, routed weight scale 1.5; learned layers gate with
    SQRT_SOFTPLUS; hash layers map a token id to 6 experts through the
    ``ffn_gate_tid2eid`` table.
  - section 3.2, MoE combine equation: y = e_shared(x) + sum_i w_i e_{k_i}(x)
    with sum_i w_i = 1.5.
  - section 4, SwiGLU equation: h = SiLU(W_gate x) * (W_up x), y = W_down h,
    h_j = g_j / (1 + exp(-g_j)) * u_j.
* [colibri] "DeepSeek V4 target engine (CPU + optional CUDA tier)",
  introduction: routed experts are native fp4 (MXFP4); the dense set is
  fp8-e4m3 with UE8M0 block scales.
* [cism] "Development Snapshot Validation", 4-bit quantization scheme study
  table: MXFP4 is E2M1 elements with E8M0 scales, one per block of 32, at 4.25 bits per weight.

Readings taken where the pages are silent:

* E2M1 element: sign bit 3, two exponent bits (bias 1), one mantissa bit,
  i.e. the OCP MX v1.0 element; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
* UE8M0 scale byte u means 2**(u - 127); u = 255 is NaN (never generated).
* Packing: row-major ``[out][in]`` rows; byte b of a row holds element 2b in
  its low nibble and element 2b+1 in its high nibble; scale j of a row covers
  elements 32j .. 32j+31 (blocks run along the reduction dimension).
* fp8 e4m3 is the OCP "fn" variant (bias 7, max 448, no infinities, S.1111.111
  is NaN); one UE8M0 scale per 128 consecutive elements of a row.
* Learned routing selects on the raw fp32 logits (sqrt o softplus is strictly
  increasing, so the set equals selection on scores); ties go to the lower
  expert index; output slot i = 0 holds the largest.  Without expert groups
  and bias this is plain top-k over all experts (route_topk).
* Group-limited selection ([Kernel Guide] section 1 names "expert group top-k
  selection" and gives no parameters; route_grouped): experts form n_group
  contiguous groups; the selection key of expert e is s_e + b_e in fp64 with
  an optional per-expert bias b that enters the selection only; a group's
  score is the sum of its two largest keys (its one key for a group of one
  expert); the topk_group groups of largest score are kept (ties to the
  lower group index) and the top_k largest keys among their experts are
  chosen (ties to the lower expert index); the weights use the unbiased s.
* Tail pruning ([Kernel Guide] section 3.2 item 3 and its configuration
  table; [RFC] section 5; prune_tail): a token keeps the routed experts whose
  weight is at least min_w, at most keep_max of them (the largest weights,
  ties to the lower slot) and at least one (the largest); kept weights are
  multiplied by alpha = sqrt(sum_all w^2 / sum_kept w^2); a dropped slot
  has expert id -1 and weight 0.  p_early = 0.025 of the RFC (weights that
  sum to 1) is min_w = 0.025 * routed_scale here.
* Gate-first lazy skip ([RFC] section 5; ffn(lazy_tau=...)): a routed
  expert whose gate output g for a token has max_j |SiLU(g_j)| < lazy_tau
  contributes nothing to that token (its up and down projections are not
  needed).  The shared expert is never skipped.
* Weights: s = sqrt(softplus(logit)), w = scale * s / sum(s) over the top-k,
  evaluated in fp64 and rounded to fp32 once.
* Grouping: perm lists flat indices f = t*top_k + i stably sorted by expert
  (ascending f inside an expert); inv_perm[perm[p]] = p.  An id of -1 (a
  slot dropped by tail pruning) belongs to no expert: it is not counted, not
  in perm, and its inv_perm is -1.
* The shared expert sees every token with weight 1 and has its own
  intermediate size.  No clamp is applied to the SwiGLU gate.
* y is accumulated in fp64 and rounded to fp32 (round-to-nearest-even) once.
"""

from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------
# Element formats (closed forms, one value at a time)
# ----------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code (OCP MX element; [cism] 4-bit study)."""
    code = int(code)
    if not 0 <= code < 16:
        raise ValueError("e2m1 code out of range")
    sign = -1.0 if code & 0x8 else 1.0
    exp_field = (code >> 1) & 0x3
    mant = code & 0x1
    if exp_field == 0:
        mag = 0.5 * mant  # subnormal: 0 or 0.5
    else:
        mag = math.ldexp(1.0 + 0.5 * mant, exp_field - 1)
    return sign * mag  # code 8 gives -0.0


def ue8m0_value(u: int) -> float:
    """Value of one UE8M0 scale byte: 2**(u-127); 255 is NaN."""
    u = int(u)
    if not 0 <= u < 256:
        raise ValueError("ue8m0 byte out of range")
    if u == 255:
        return math.nan
    return math.ldexp(1.0, u - 127)


def e4m3_value(code: int) -> float:
    """Value of one OCP fp8 E4M3 ("fn") byte: bias 7, no inf, S.1111.111 NaN."""
    code = int(code)
    if not 0 <= code < 256:
        raise ValueError("e4m3 code out of range")
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        mag = math.ldexp(mant / 8.0, 1 - 7)  # subnormal: m * 2**-9
    else:
        mag = math.ldexp(1.0 + mant / 8.0, exp_field - 7)
    return sign * mag


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper 16 bits of an IEEE binary32; widen exactly."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Block decode (tables built from the closed forms above)
# ----------------------------------------------------------------------------

_E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_UE8M0_TABLE = np.array([ue8m0_value(u) for u in range(256)], dtype=np.float64)
_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_mxfp4(codes: np.ndarray, scales: np.ndarray, cols: int) -> np.ndarray:
    """Decode an MXFP4 matrix ``[rows][cols/2]`` codes + ``[rows][cols/32]``
    scales to fp64 ``[rows][cols]`` (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    if codes.shape != (rows, cols // 2) or scales.shape != (rows, cols // 32):
        raise ValueError("mxfp4 shapes do not match cols")
    vals = np.empty((rows, cols), dtype=np.float64)
    vals[:, 0::2] = _E2M1_TABLE[codes & 0x0F]  # low nibble: even element
    vals[:, 1::2] = _E2M1_TABLE[codes >> 4]  # high nibble: odd element
    vals = vals.reshape(rows, cols // 32, 32) * _UE8M0_TABLE[scales][:, :, None]
    return vals.reshape(rows, cols)


def decode_fp8_b128(codes: np.ndarray, scales: np.ndarray, cols: int) -> np.ndarray:
    """Decode fp8-e4m3 ``[rows][cols]`` with one UE8M0 per 128 elements of a
    row to fp64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    if codes.shape != (rows, cols) or scales.shape != (rows, cols // 128):
        raise ValueError("fp8 shapes do not match cols")
    vals = _E4M3_TABLE[codes].reshape(rows, cols // 128, 128)
    vals = vals * _UE8M0_TABLE[scales][:, :, None]
    return vals.reshape(rows, cols)


def decode_proj(proj: dict, index, cols: int, rows_subset=None) -> np.ndarray:
    """Decode one expert matrix of a projection description.

    ``proj`` = {"type": "mxfp4" | "fp8_e4m3_b128", "codes": ..., "scales": ...};
    ``codes[index]`` / ``scales[index]`` select the expert (``index`` None for
    an unstacked matrix).  ``rows_subset`` restricts the decoded rows.
    """
    codes = proj["codes"] if index is None else proj["codes"][index]
    scales = proj["scales"] if index is None else proj["scales"][index]
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    if rows_subset is not None:
        codes = codes[rows_subset]
        scales = scales[rows_subset]
    if proj["type"] == "mxfp4":
        return decode_mxfp4(codes, scales, cols)
    if proj["type"] == "fp8_e4m3_b128":
        return decode_fp8_b128(codes, scales, cols)
    raise ValueError("unknown weight type %r" % (proj["type"],))


def decode_activations(x: np.ndarray, act_type: str) -> np.ndarray:
    """Activations as given: fp32 values or bf16 bit patterns -> fp64."""
    if act_type == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if act_type == "bf16":
        return bf16_bits_to_f64(x)
    raise ValueError("unknown activation type %r" % (act_type,))


# ----------------------------------------------------------------------------
# Routing ([Kernel Guide] section 1 and section 3.2)
# ----------------------------------------------------------------------------


def softplus(v: float) -> float:
    """log(1 + e^v) written so that it neither overflows nor cancels."""
    return max(v, 0.0) + math.log1p(math.exp(-abs(v)))


def route_topk(logits: np.ndarray, top_k: int, routed_scale: float):
    """Learned SQRT_SOFTPLUS router.

    For each token: the ``top_k`` largest fp32 logits (ties to the lower
    expert index, slot 0 = largest), s_i = sqrt(softplus(l_i)),
    w_i = routed_scale * s_i / sum_j s_j.  Returns ids int32 [N][k] and
    weights fp32 [N][k].
    """
    logits = np.asarray(logits, dtype=np.float32)
    n_tokens, n_experts = logits.shape
    if not 0 < top_k <= n_experts:
        raise ValueError("bad top_k")
    ids = np.zeros((n_tokens, top_k), dtype=np.int32)
    w = np.zeros((n_tokens, top_k), dtype=np.float32)
    for t in range(n_tokens):
        row = [float(v) for v in logits[t]]
        order = sorted(range(n_experts), key=lambda e: (-row[e], e))
        chosen = order[:top_k]
        s = [math.sqrt(softplus(row[e])) for e in chosen]
        total = 0.0
        for si in s:
            total += si
        for i, e in enumerate(chosen):
            ids[t, i] = e
            w[t, i] = np.float32(routed_scale * s[i] / total)
    return ids, w


def route_hash(token_ids: np.ndarray, tid2eid: np.ndarray, tid2w: np.ndarray):
    """Token-id hash routing: the table row of the token, in table order."""
    token_ids = np.asarray(token_ids)
    ids = np.asarray(tid2eid)[token_ids].astype(np.int32)
    w = np.asarray(tid2w)[token_ids].astype(np.float32)
    return ids, w


def gate_score(v: float) -> float:
    """s = sqrt(softplus(v)) in fp64 ([Kernel Guide] section 1, SQRT_SOFTPLUS)."""
    return math.sqrt(softplus(v))


def route_grouped(logits: np.ndarray, top_k: int, routed_scale: float, n_group: int = 1,
                  topk_group: int = 1, bias=None):
    """Group-limited SQRT_SOFTPLUS router with a selection-only bias.

    For each token, in fp64: s_e = sqrt(softplus(l_e)); key_e = s_e + b_e;
    group g holds experts g*G .. g*G+G-1 (G = E / n_group) and scores the sum
    of its two largest keys (largest first; one key if G == 1); the
    topk_group best groups (score descending, ties to the lower group) are
    kept; the top_k experts of those groups by key (descending, ties to the
    lower expert) are chosen, slot 0 the largest; w_i = routed_scale * s_i /
    sum_j s_j over the chosen (unbiased scores, summed in slot order),
    rounded to fp32 once.
    """
    logits = np.asarray(logits, dtype=np.float32)
    n_tokens, n_experts = logits.shape
    if n_group < 1 or n_experts % n_group != 0:
        raise ValueError("n_group must divide n_experts")
    gsize = n_experts // n_group
    if not 1 <= topk_group <= n_group or not 0 < top_k <= topk_group * gsize:
        raise ValueError("bad topk_group / top_k")
    b = [0.0] * n_experts if bias is None else [float(v) for v in np.asarray(bias, np.float32)]
    ids = np.zeros((n_tokens, top_k), dtype=np.int32)
    w = np.zeros((n_tokens, top_k), dtype=np.float32)
    for t in range(n_tokens):
        s = [gate_score(float(v)) for v in logits[t]]
        key = [s[e] + b[e] for e in range(n_experts)]
        gscore = []
        for g in range(n_group):
            members = sorted(key[g * gsize:(g + 1) * gsize], reverse=True)
            gscore.append(members[0] + members[1] if gsize > 1 else members[0])
        groups = sorted(range(n_group), key=lambda g: (-gscore[g], g))[:topk_group]
        cand = [e for g in sorted(groups) for e in range(g * gsize, (g + 1) * gsize)]
        chosen = sorted(cand, key=lambda e: (-key[e], e))[:top_k]
        total = 0.0
        for e in chosen:
            total += s[e]
        for i, e in enumerate(chosen):
            ids[t, i] = e
            w[t, i] = np.float32(routed_scale * s[e] / total)
    return ids, w


def prune_tail(ids: np.ndarray, w: np.ndarray, keep_max: int, min_w: float):
    """Tail pruning with L2-quadrature rescaling of the kept weights.

    Per token: the slots with w >= min_w are candidates; at most keep_max of
    them are kept (the largest weights, ties to the lower slot), and at least
    one (the slot of the largest weight).  alpha = sqrt(sum_all w^2 /
    sum_kept w^2) from the fp32 weights in fp64; kept w becomes
    fp32(w * alpha); dropped slots get id -1 and weight 0.  Slots keep their
    positions.
    """
    ids = np.array(ids, dtype=np.int32)
    w = np.array(w, dtype=np.float32)
    n_tokens, top_k = ids.shape
    if not 1 <= keep_max <= top_k:
        raise ValueError("keep_max must be in 1..top_k")
    for t in range(n_tokens):
        wt = [float(v) for v in w[t]]
        by_weight = sorted(range(top_k), key=lambda i: (-wt[i], i))
        kept = [i for i in by_weight if wt[i] >= min_w][:keep_max]
        if not kept:
            kept = by_weight[:1]
        all_sq = 0.0
        for v in wt:
            all_sq += v * v
        kept_sq = 0.0
        for i in sorted(kept):
            kept_sq += wt[i] * wt[i]
        alpha = math.sqrt(all_sq / kept_sq)
        for i in range(top_k):
            if i in kept:
                w[t, i] = np.float32(wt[i] * alpha)
            else:
                ids[t, i] = -1
                w[t, i] = 0.0
    return ids, w


# ----------------------------------------------------------------------------
# Grouping (token-to-expert bucketing)
# ----------------------------------------------------------------------------


def group(ids: np.ndarray, n_experts: int):
    """counts, exclusive offsets, stable permutation and its inverse.

    Two plain passes: count, then place each flat index f = t*k + i (in
    ascending f) at the next free position of its expert.  Ids of -1 (slots
    dropped by tail pruning) are skipped: perm has offsets[E] entries and
    their inv_perm is -1.
    """
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * n_experts
    for e in flat:
        if e >= 0:
            counts[e] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:n_experts]
    perm = [0] * offsets[n_experts]
    inv_perm = [-1] * len(flat)
    for f, e in enumerate(flat):
        if e < 0:
            continue
        p = fill[e]
        perm[p] = f
        inv_perm[f] = p
        fill[e] = p + 1
    as_i32 = lambda v: np.array(v, dtype=np.int32)  # noqa: E731
    return as_i32(counts), as_i32(offsets), as_i32(perm), as_i32(inv_perm)


# ----------------------------------------------------------------------------
# Expert FFN and combine ([Kernel Guide] section 4 and section 3.2)
# ----------------------------------------------------------------------------


def silu(g: np.ndarray) -> np.ndarray:
    """g / (1 + exp(-g)) in fp64 (the SwiGLU gate, no clamp)."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(xs: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
               w_down: np.ndarray) -> np.ndarray:
    """o = W_down (SiLU(W_gate x) * (W_up x)) for each row x of ``xs``."""
    g = xs @ w_gate.T
    u = xs @ w_up.T
    h = silu(g) * u
    return h @ w_down.T


def ffn(layer: dict, x: np.ndarray, act_type: str, ids: np.ndarray,
        w: np.ndarray, tokens=None, out_rows=None, with_shared: bool = True,
        lazy_tau: float = 0.0):
    """MoE FFN output y (fp32) for ``tokens`` (default: all) and output
    features ``out_rows`` (default: all).

    y_t = e_shared(x_t) + sum_i w[t,i] e_{ids[t,i]}(x_t), accumulated in fp64,
    rounded to fp32 once.  Each routed expert's three matrices are decoded to
    fp64 once; the tokens that chose it are found by scanning ``ids``.  A slot
    with id -1 (dropped by tail pruning) has no expert.  With lazy_tau > 0 a
    routed expert whose gate output for a token has max_j |SiLU(g_j)| <
    lazy_tau is left out of that token's sum (gate-first lazy skip).
    """
    hidden, inter = layer["hidden"], layer["inter"]
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float32)
    n_tokens, top_k = ids.shape
    tokens = list(range(n_tokens)) if tokens is None else [int(t) for t in tokens]
    xs = decode_activations(np.asarray(x)[tokens], act_type)
    n_out = hidden if out_rows is None else len(out_rows)
    y = np.zeros((len(tokens), n_out), dtype=np.float64)

    members = {}  # expert -> list of (row in xs, weight)
    for j, t in enumerate(tokens):
        for i in range(top_k):
            if int(ids[t, i]) >= 0:
                members.setdefault(int(ids[t, i]), []).append((j, float(w[t, i])))
    for e in sorted(members):
        wg = decode_proj(layer["gate"], e, hidden)
        wu = decode_proj(layer["up"], e, hidden)
        wd = decode_proj(layer["down"], e, inter, out_rows)
        rows = [j for j, _ in members[e]]
        o = expert_ffn(xs[rows], wg, wu, wd)
        if lazy_tau > 0.0:
            gate_max = np.max(np.abs(silu(xs[rows] @ wg.T)), axis=1)
        for r, (j, wt) in enumerate(members[e]):
            if lazy_tau > 0.0 and gate_max[r] < lazy_tau:
                continue
            y[j] += wt * o[r]

    shared = layer.get("shared")
    if with_shared and shared is not None:
        s_inter = shared["inter"]
        wg = decode_proj(shared["gate"], None, hidden)
        wu = decode_proj(shared["up"], None, hidden)
        wd = decode_proj(shared["down"], None, s_inter, out_rows)
        y += expert_ffn(xs, wg, wu, wd)
    return y.astype(np.float32)


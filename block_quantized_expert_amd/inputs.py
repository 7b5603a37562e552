"""Seeded synthetic inputs for the routed MoE FFN workloads.

This module is the only thing the HIP path and the fp64 oracle share.  It
holds none of the method's arithmetic: it draws random bytes and normals,
rounds activations to bf16 (a storage format), spaces router logits apart and
draws distinct experts for the hash table (input conditioning).  Routing,
decode, matmul, SwiGLU and combine live elsewhere.

Weight bytes come from a counter-based generator (a Weyl sequence through
the MurmurHash3 32-bit finaliser, ``fmix32``), evaluated with exact integer
tensor ops, so any expert of any layer copy can be regenerated alone, on the
CPU or on a GPU, bit for bit.  Normals come from NumPy's PCG64 generator
seeded per (workload seed, stream, copy).

Workload shapes follow the DeepSeek-V4-Flash layer described in "DeepSeek-V4-Flash
284B -- Deep-Dive Mathematical & Kernel Guide", section 1 (hidden 4096,
256 routed experts + 1 shared, top-6, routed scale 1.5), and the expert
formats of "DeepSeek V4 target engine (CPU + optional CUDA tier)" (routed
experts in MXFP4, dense weights in fp8-e4m3 with UE8M0 block scales).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    routed_scale: float
    act: str  # "f32" or "bf16"
    routing: str  # "learned" or "hash"
    scale_lo: int  # UE8M0 bytes drawn uniformly from [scale_lo, scale_hi]
    scale_hi: int
    shared: str  # weight type of the shared expert
    bias: str  # "none", "normal" (std 0.5) or "zipf"
    seed: int
    vocab: int = 129280
    min_gap: float = 1e-3  # every pair of logits of a token differs by this
    shared_inter: int = 0  # 0: same as inter
    routed: str = "mxfp4"  # weight type of the routed experts


WORKLOADS = {
    # 8 tokens, hidden 256, 16 routed experts + 1 shared, intermediate 128,
    # top-2; fp32 activations; scale exponents -6..-3.
    "tiny": Workload("tiny", 8, 256, 128, 16, 2, 1.5, "f32", "learned",
                     121, 124, "mxfp4", "none", 1),
    # DeepSeek-V4-Flash-shaped layer, single-token decode; exponents -8..-4.
    "decode1": Workload("decode1", 1, 4096, 2048, 256, 6, 1.5, "bf16",
                        "learned", 119, 123, "mxfp4", "none", 2),
    # Batched decode of 32 tokens with a per-expert N(0, 0.5^2) logit bias.
    # The seed is one whose realised routing has every count in 0..6 and
    # some odd count >= 3 (checked by the test suite with the oracle).
    "decode32": Workload("decode32", 32, 4096, 2048, 256, 6, 1.5, "bf16",
                         "learned", 119, 123, "mxfp4", "normal", 4),
    # Prefill of 512 tokens with a Zipf-like popularity bias
    # b_e = -1.1 * 0.3 * ln(rank_e) over a seeded rank permutation.
    "prefill512": Workload("prefill512", 512, 4096, 2048, 256, 6, 1.5, "bf16",
                           "learned", 119, 123, "mxfp4", "zipf", 4),
    # Hash-routed prefill of 4096 tokens; shared expert in fp8-e4m3 with one
    # UE8M0 scale per 1x128 row block.
    "hash4096": Workload("hash4096", 4096, 4096, 2048, 256, 6, 1.5, "bf16",
                         "hash", 119, 123, "fp8_e4m3_b128", "none", 5),
}

WORKLOAD_ORDER = ["tiny", "decode1", "decode32", "prefill512", "hash4096"]

# ----------------------------------------------------------------------------
# Counter-based bytes
# ----------------------------------------------------------------------------

_M32 = 0xFFFFFFFF
_GOLDEN = 0x9E3779B1


def _py_fmix32(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x85EBCA6B) & _M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & _M32
    x ^= x >> 16
    return x


def stream_key(*parts: int) -> int:
    """32-bit key for one stream, folded from small integers."""
    k = 0x243F6A88
    for p in parts:
        k = _py_fmix32((k * _GOLDEN + (int(p) & _M32) + 0x7F4A7C15) & _M32)
    return k


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    # low 32 bits of x*c for x < 2**32 without leaving int64 range
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & _M32


def _fmix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x85EBCA6B)
    x = x ^ (x >> 13)
    x = _mul32(x, 0xC2B2AE35)
    return x ^ (x >> 16)


def hash_words(key: int, start: int, count: int, device) -> torch.Tensor:
    """``count`` 32-bit words (as int64) of stream ``key`` from ``start``."""
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    return _fmix32((_mul32(i & _M32, _GOLDEN) + key) & _M32)


def random_bytes(key: int, start_byte: int, n: int, device) -> torch.Tensor:
    """``n`` uniform bytes of stream ``key`` starting at byte ``start_byte``
    (a multiple of 4)."""
    assert start_byte % 4 == 0
    words = hash_words(key, start_byte // 4, (n + 3) // 4, device)
    parts = [((words >> s) & 0xFF) for s in (0, 8, 16, 24)]
    return torch.stack(parts, dim=1).reshape(-1)[:n].to(torch.uint8)


def uniform_small(key: int, start: int, n: int, n_values: int, device) -> torch.Tensor:
    """``n`` integers in [0, n_values), one per word."""
    words = hash_words(key, start, n, device)
    return ((words & 0xFFFF) * n_values) >> 16


# ----------------------------------------------------------------------------
# Expert weights
# ----------------------------------------------------------------------------

PROJ_IDS = {"gate": 0, "up": 1, "down": 2,
            "shared_gate": 3, "shared_up": 4, "shared_down": 5}


def proj_shape(wl: Workload, proj: str):
    """(rows, cols) of one expert matrix: rows are output features."""
    inter = wl.inter
    if proj.startswith("shared_") and wl.shared_inter:
        inter = wl.shared_inter
    base = proj.replace("shared_", "")
    if base in ("gate", "up"):
        return inter, wl.hidden
    return wl.hidden, inter


def _mxfp4_block(wl, proj, copy, first, n_exp, device):
    rows, cols = proj_shape(wl, proj)
    cb = rows * cols // 2
    sb = rows * cols // 32
    pid = PROJ_IDS[proj]
    codes = random_bytes(stream_key(wl.seed, copy, pid, 0), first * cb, n_exp * cb, device)
    nval = wl.scale_hi - wl.scale_lo + 1
    sc = uniform_small(stream_key(wl.seed, copy, pid, 1), first * sb, n_exp * sb, nval, device)
    scales = (sc + wl.scale_lo).to(torch.uint8)
    return (codes.view(n_exp, rows, cols // 2), scales.view(n_exp, rows, cols // 32))


def _fp8_block(wl, proj, copy, first, n_exp, device):
    """fp8-e4m3 codes of matrices first .. first+n_exp-1 of a projection:
    sign uniform, exponent field uniform in 0..10 (so zeros and subnormals
    occur), mantissa uniform; never NaN.  One UE8M0 scale per 1x128 block."""
    rows, cols = proj_shape(wl, proj)
    pid = PROJ_IDS[proj]
    n = rows * cols
    w = hash_words(stream_key(wl.seed, copy, pid, 0), first * n, n_exp * n, device)
    sign = w & 1
    mant = (w >> 1) & 7
    expf = (((w >> 8) & 0xFFFF) * 11) >> 16
    codes = ((sign << 7) | (expf << 3) | mant).to(torch.uint8).view(n_exp, rows, cols)
    nval = wl.scale_hi - wl.scale_lo + 1
    sb = rows * (cols // 128)
    sc = uniform_small(stream_key(wl.seed, copy, pid, 1), first * sb, n_exp * sb, nval, device)
    scales = (sc + wl.scale_lo).to(torch.uint8).view(n_exp, rows, cols // 128)
    return codes, scales


def _fp8_matrix(wl, proj, copy, device):
    c, s = _fp8_block(wl, proj, copy, 0, 1, device)
    return c[0], s[0]


def _routed_block(wl, proj, copy, first, n_exp, device):
    """Codes and scales of routed experts first .. first+n_exp-1."""
    if wl.routed == "mxfp4":
        return _mxfp4_block(wl, proj, copy, first, n_exp, device)
    if wl.routed == "fp8_e4m3_b128":
        return _fp8_block(wl, proj, copy, first, n_exp, device)
    raise ValueError(wl.routed)


def expert_weights(wl: Workload, proj: str, experts, device="cpu", copy: int = 0):
    """{e: (codes, scales)} for the listed routed experts of ``proj``."""
    return {int(e): tuple(t[0] for t in _routed_block(wl, proj, copy, int(e), 1, device))
            for e in experts}


def make_layer(wl: Workload, device="cpu", copy: int = 0, experts=None,
               with_shared: bool = True, chunk: int = 16) -> dict:
    """One layer's weights.

    ``experts=None`` gives stacked tensors ``[E][rows][...]`` for every routed
    expert; a list gives dicts ``{e: tensor}`` holding only those experts (the
    bytes are the same either way).
    """
    layer = {"hidden": wl.hidden, "inter": wl.inter, "n_experts": wl.n_experts}
    for proj in ("gate", "up", "down"):
        if experts is None:
            codes = scales = None
            for e0 in range(0, wl.n_experts, chunk):
                n = min(chunk, wl.n_experts - e0)
                c, s = _routed_block(wl, proj, copy, e0, n, device)
                if codes is None:
                    codes = torch.empty((wl.n_experts,) + tuple(c.shape[1:]), dtype=torch.uint8,
                                        device=device)
                    scales = torch.empty((wl.n_experts,) + tuple(s.shape[1:]),
                                         dtype=torch.uint8, device=device)
                codes[e0:e0 + n] = c
                scales[e0:e0 + n] = s
        else:
            ew = expert_weights(wl, proj, experts, device, copy)
            codes = {e: v[0] for e, v in ew.items()}
            scales = {e: v[1] for e, v in ew.items()}
        layer[proj] = {"type": wl.routed, "codes": codes, "scales": scales}
    if with_shared:
        shared = {"inter": wl.shared_inter or wl.inter}
        for proj in ("shared_gate", "shared_up", "shared_down"):
            if wl.shared == "mxfp4":
                c, s = _mxfp4_block(wl, proj, copy, 0, 1, device)
                c, s = c[0], s[0]
            elif wl.shared == "fp8_e4m3_b128":
                c, s = _fp8_matrix(wl, proj, copy, device)
            else:
                raise ValueError(wl.shared)
            shared[proj.replace("shared_", "")] = {"type": wl.shared, "codes": c, "scales": s}
        layer["shared"] = shared
    else:
        layer["shared"] = None
    return layer


def layer_to_numpy(layer: dict) -> dict:
    """Same layer description with every tensor moved to host NumPy."""
    def conv(v):
        if isinstance(v, torch.Tensor):
            return v.cpu().numpy()
        if isinstance(v, dict):
            return {k: conv(x) for k, x in v.items()}
        return v
    return conv(layer)


# ----------------------------------------------------------------------------
# Activations and routing inputs
# ----------------------------------------------------------------------------

STREAM_X, STREAM_LOGITS, STREAM_BIAS, STREAM_TOKENS, STREAM_TABLE = 1, 2, 3, 4, 5
STREAM_SEL_BIAS = 6


def _rng(wl: Workload, stream: int, copy: int) -> np.random.Generator:
    return np.random.default_rng([wl.seed, stream, copy])


def activations(wl: Workload, copy: int = 0, n_tokens=None) -> torch.Tensor:
    """N(0,1) activations [N][H] on the CPU: fp32, or bf16 (round to nearest
    even of the fp32 draw)."""
    n = wl.n_tokens if n_tokens is None else n_tokens
    x = _rng(wl, STREAM_X, copy).standard_normal((n, wl.hidden), dtype=np.float32)
    t = torch.from_numpy(x)
    return t if wl.act == "f32" else t.to(torch.bfloat16)


def expert_bias(wl: Workload) -> np.ndarray:
    """Per-expert logit bias, fixed per workload (copy-independent)."""
    rng = _rng(wl, STREAM_BIAS, 0)
    if wl.bias == "none":
        return np.zeros(wl.n_experts)
    if wl.bias == "normal":
        return 0.5 * rng.standard_normal(wl.n_experts)
    if wl.bias == "zipf":
        rank = rng.permutation(wl.n_experts) + 1
        return -1.1 * 0.3 * np.log(rank)
    raise ValueError(wl.bias)


def selection_bias(wl: Workload, std: float = 0.5) -> torch.Tensor:
    """A per-expert fp32 bias for selection-only use, N(0, std^2), fixed per
    workload (input data: the router adds it to its selection keys)."""
    b = std * _rng(wl, STREAM_SEL_BIAS, 0).standard_normal(wl.n_experts)
    return torch.from_numpy(b.astype(np.float32))


def spaced_logits(rng: np.random.Generator, n: int, bias: np.ndarray,
                  min_gap: float) -> np.ndarray:
    """fp32 N(0,1)+bias logits in which any two of a row differ by at least
    ``min_gap``: values too close to a neighbour are drawn again."""
    e = bias.shape[0]
    lg = (rng.standard_normal((n, e)) + bias[None, :]).astype(np.float32)
    for _ in range(10000):
        order = np.argsort(lg, axis=1, kind="stable")
        srt = np.take_along_axis(lg, order, axis=1).astype(np.float64)
        close = np.diff(srt, axis=1) < min_gap
        if not close.any():
            return lg
        r, c = np.nonzero(close)
        idx = order[r, c + 1]
        lg[r, idx] = (rng.standard_normal(len(r)) + bias[idx]).astype(np.float32)
    raise RuntimeError("could not space logits")


def router_logits(wl: Workload, copy: int = 0, n_tokens=None) -> torch.Tensor:
    n = wl.n_tokens if n_tokens is None else n_tokens
    lg = spaced_logits(_rng(wl, STREAM_LOGITS, copy), n, expert_bias(wl), wl.min_gap)
    return torch.from_numpy(lg)


def hash_table(wl: Workload):
    """tid2eid [vocab][k] int32 (distinct experts per row, partial
    Fisher-Yates) and tid2w [vocab][k] fp32 = routed_scale / k."""
    rng = _rng(wl, STREAM_TABLE, 0)
    v, e, k = wl.vocab, wl.n_experts, wl.top_k
    perm = np.tile(np.arange(e, dtype=np.int32), (v, 1))
    ar = np.arange(v)
    for i in range(k):
        j = i + rng.integers(0, e - i, size=v)
        a = perm[ar, i].copy()
        perm[ar, i] = perm[ar, j]
        perm[ar, j] = a
    tid2eid = np.ascontiguousarray(perm[:, :k])
    tid2w = np.full((v, k), wl.routed_scale / k, dtype=np.float32)
    return torch.from_numpy(tid2eid), torch.from_numpy(tid2w)


def token_ids(wl: Workload, copy: int = 0, n_tokens=None) -> torch.Tensor:
    n = wl.n_tokens if n_tokens is None else n_tokens
    t = _rng(wl, STREAM_TOKENS, copy).integers(0, wl.vocab, size=n).astype(np.int32)
    return torch.from_numpy(t)


def routing_inputs(wl: Workload, copy: int = 0, n_tokens=None) -> dict:
    """Inputs of the router for one batch (CPU tensors)."""
    if wl.routing == "learned":
        return {"kind": "learned", "logits": router_logits(wl, copy, n_tokens)}
    tid2eid, tid2w = hash_table(wl)
    return {"kind": "hash", "token_ids": token_ids(wl, copy, n_tokens),
            "tid2eid": tid2eid, "tid2w": tid2w}


def routing_to_numpy(routing: dict) -> dict:
    return {k: (v.numpy() if isinstance(v, torch.Tensor) else v) for k, v in routing.items()}


def activations_to_numpy(x: torch.Tensor) -> np.ndarray:
    """fp32 values, or bf16 bit patterns as uint16."""
    if x.dtype == torch.bfloat16:
        return x.cpu().view(torch.int16).numpy().view(np.uint16)
    return x.cpu().numpy()

"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
the oracle on the same seeded inputs, and compare."""

from __future__ import annotations

import numpy as np
import torch

from block_quantized_expert_amd import binding as B
from block_quantized_expert_amd import inputs as I
from oracle import moe_oracle as O

# tolerance on max|y - y_ref| / rms(y_ref) for fp32 outputs from bf16 (or fp32) activations
Y_TOL = 2e-3


def gpu_inputs(wl: I.Workload, copy: int = 0, with_shared: bool = True, n_tokens=None):
    """Device layer + activations + routing inputs of a workload."""
    dev = torch.device("cuda:0")
    weights = I.make_layer(wl, device=dev, copy=copy, with_shared=with_shared)
    x = I.activations(wl, copy, n_tokens)
    routing = I.routing_inputs(wl, copy, n_tokens)
    x_d = x.to(dev)
    routing_d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in routing.items()}
    return B.Layer(weights, wl.top_k), x, x_d, routing, routing_d


def oracle_routing(wl: I.Workload, routing: dict):
    r = I.routing_to_numpy(routing)
    if r["kind"] == "learned":
        return O.route_topk(r["logits"], wl.top_k, wl.routed_scale)
    return O.route_hash(r["token_ids"], r["tid2eid"], r["tid2w"])


def oracle_y(wl: I.Workload, x: torch.Tensor, ids, w, tokens=None, rows=None,
             with_shared=True, copy=0):
    """Oracle output for the sampled tokens/rows; only the experts those
    tokens use are generated (on the CPU, same bytes as on the GPU)."""
    tok = range(ids.shape[0]) if tokens is None else tokens
    needed = sorted({int(e) for t in tok for e in ids[t]})
    layer = I.layer_to_numpy(I.make_layer(wl, device="cpu", experts=needed,
                                          with_shared=with_shared, copy=copy))
    return O.ffn(layer, I.activations_to_numpy(x), wl.act, ids, w, tokens=tokens,
                 out_rows=rows, with_shared=with_shared)


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(y.astype(np.float64) - ref))) / rms


def assert_y_close(y: np.ndarray, ref: np.ndarray, tol: float = Y_TOL):
    assert y.shape == ref.shape
    assert np.all(np.isfinite(y))
    r = rel_err(y, ref)
    print("max|err|/rms = %.3e (bound %.1e)" % (r, tol))
    assert r <= tol, r


def assert_w_close(w_gpu: np.ndarray, w_ref: np.ndarray):
    """Both sides round an fp64 value to fp32 once: at most one ulp apart."""
    assert np.all(np.abs(w_gpu - w_ref) <= np.spacing(np.abs(w_ref).astype(np.float32)))


def host_layer(weights: dict, experts) -> dict:
    """The listed routed experts (and the shared expert) of a device layer
    made by ``inputs.make_layer``, copied to host NumPy for the oracle.  The
    bytes are the generator's, as on the GPU; copying them is faster than
    drawing them again on the CPU for layers with many experts."""
    out = {"hidden": weights["hidden"], "inter": weights["inter"],
           "n_experts": weights["n_experts"]}
    for proj in ("gate", "up", "down"):
        p = weights[proj]
        out[proj] = {"type": p["type"],
                     "codes": {int(e): p["codes"][int(e)].cpu().numpy() for e in experts},
                     "scales": {int(e): p["scales"][int(e)].cpu().numpy() for e in experts}}
    sh = weights.get("shared")
    if sh is None:
        out["shared"] = None
    else:
        out["shared"] = {"inter": sh["inter"]}
        for proj in ("gate", "up", "down"):
            out["shared"][proj] = {"type": sh[proj]["type"], "codes": sh[proj]["codes"].cpu().numpy(),
                                   "scales": sh[proj]["scales"].cpu().numpy()}
    return out


def oracle_y_host(weights: dict, act: str, x: torch.Tensor, ids, w, tokens=None, rows=None,
                  with_shared=True, lazy_tau=0.0):
    """oracle_y with the weights copied from the device layer."""
    tok = range(ids.shape[0]) if tokens is None else tokens
    needed = sorted({int(e) for t in tok for e in ids[t] if e >= 0})
    layer = host_layer(weights, needed)
    return O.ffn(layer, I.activations_to_numpy(x), act, ids, w, tokens=tokens, out_rows=rows,
                 with_shared=with_shared, lazy_tau=lazy_tau)


def assert_w_near(w_gpu: np.ndarray, w_ref: np.ndarray, tol: float = 1e-5):
    """Weights after options (pruning rescales): within 1e-5 absolute."""
    assert w_gpu.shape == w_ref.shape
    assert np.all(np.abs(w_gpu.astype(np.float64) - w_ref.astype(np.float64)) <= tol)


def assert_grouping(grouping, ids_ref, n_experts):
    """counts, offsets, perm, inv_perm bit-exact against the oracle's grouping."""
    counts, offsets, perm, inv = O.group(ids_ref, n_experts)
    g = [t.cpu().numpy() for t in grouping]
    assert np.array_equal(g[0], counts)
    assert np.array_equal(g[1], offsets)
    assert np.array_equal(g[2][: offsets[-1]], perm)
    assert np.array_equal(g[3], inv)


def block_tokens(ids: np.ndarray, n_experts: int, block: int = 16):
    """Tokens that put a slot in every `block`-slot block of every expert's
    group (and of the shared expert's, whose slot order is the token order):
    the first slot of each block.  Grouped slots are in expert order, stably
    by flat index, so this hits every token tile and every 16-token block
    the grouped kernels form."""
    counts, offsets, perm, _ = O.group(ids, n_experts)
    k = ids.shape[1]
    toks = set()
    for e in range(n_experts):
        for s in range(offsets[e], offsets[e + 1], block):
            toks.add(int(perm[s]) // k)
    toks.update(range(0, ids.shape[0], block))
    return sorted(toks)

#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN hot path on one MI355X.

One step = route -> group -> gate/up (+SwiGLU) -> down (+combine) over one
batch of synthetic input, every kernel launched through the C ABI of
libmoe.so on one HIP stream.  Default workload: the DeepSeek-V4-Flash-shaped
layer at single-token decode (hidden 4096, 256 routed experts + 1 shared,
intermediate 2048, top-6, MXFP4 experts, bf16 activations).

Cold caches: the weights live in --copies independent layer copies (3.44 GB
each) used round-robin, and every step takes a fresh batch from a seeded
pool, so no expert is served from the 256 MB last-level cache or the L2s.

Prints ONE JSON line.  `value` is tokens/s over the K timed steps
(wall clock, synchronised on both sides).  `roofline` is for the dominant
kernel (gate/up): algorithmic bytes per launch over its average duration
measured with HIP events on the launch stream inside the timed region (at
one token the whole layer is one kernel, and that kernel is the one
reported).  The
kernels record those events from their own dispatch packets; recording them
costs the host several microseconds per step, so at decode sizes (where the
host would otherwise fall behind the GPU) only every --event-every-th timed
step carries them.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-FFN tokens/s + % HBM peak (decode) / % MFMA peak (prefill), 1 GPU"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published

DEFAULTS = {  # workload: (steps, warmup, copies, pool, event_every)
    "decode1": (2000, 100, 8, 64, 8),
    "decode32": (400, 20, 8, 16, 1),
    "prefill512": (50, 5, 8, 4, 1),
    "hash4096": (20, 3, 2, 2, 1),
    "tiny": (2000, 100, 1, 8, 8),
}

# HBM traffic of the roofline kernel per launch, from two rocprofv3 --pmc
# passes over this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch,
# averaged over the timed dispatches), each scaled by what the same counter
# reads for a plain 256 MiB device copy run in the same process
# (--copy-mib 256): FETCH_SIZE read 131083.5 KiB for 262144 KiB read,
# WRITE_SIZE read 262144 KiB for 262144 KiB written.  Only workloads whose
# roofline kernel is unchanged since the counters were taken are listed.
FETCH_SCALE = 262144.0 / 131083.5
WRITE_SCALE = 1.0
KERNEL_TRAFFIC_KIB = {  # workload: (FETCH_SIZE, WRITE_SIZE) per step of the roofline stage
    "decode1": (46176.4, 82.2),           # decode_fused_kernel<8>
    "decode32": (474862.2, 1669.1),       # quant_x_kernel + gemm_gate_up_kernel<0, 112, true, true>
    "prefill512": (1184148.4, 27735.4),   # quant_x_kernel + gemm_gate_up_kernel<0, 112, true, true>
    "hash4096": (2321829.8, 231717.5),    # quant_x_kernel + MXFP4 routed and fp8 shared gate/up
}


def kernel_traffic(name):
    kib = KERNEL_TRAFFIC_KIB.get(name)
    if kib is None:
        return None
    return (kib[0] * FETCH_SCALE + kib[1] * WRITE_SCALE) * 1024.0


def proj_bytes(wtype: str, rows: int, cols: int) -> int:
    """Stored bytes of one expert matrix (codes + scales)."""
    if wtype == "mxfp4":
        return rows * cols // 2 + rows * cols // 32
    return rows * cols + rows * cols // 128


def workload_costs(wl, counts_list):
    """Algorithmic bytes and flops of each launch, averaged over steps.

    Gate/up launch: gate and up matrices of every routed expert with at
    least one token, plus the shared expert, plus the activations read.
    Down launch: the down matrices of the same experts plus y written.
    Whole path adds router input and ids/weights.  Flops: 2*3*I*H per
    (token, expert) pair including the shared expert.  Implementation
    traffic (h, per-slot outputs, permutation) is not counted.
    """
    h, i = wl.hidden, wl.inter
    si = wl.shared_inter or wl.inter
    act = 4 if wl.act == "f32" else 2
    per_routed_gu = 2 * proj_bytes("mxfp4", i, h)
    per_routed_dn = proj_bytes("mxfp4", h, i)
    sh_gu = 2 * proj_bytes(wl.shared, si, h)
    sh_dn = proj_bytes(wl.shared, h, si)
    n = wl.n_tokens
    gu, dn, path, flops = 0.0, 0.0, 0.0, 0.0
    for counts in counts_list:
        d = int((counts > 0).sum())
        g = d * per_routed_gu + sh_gu + n * h * act
        dd = d * per_routed_dn + sh_dn + n * h * 4
        route_in = n * wl.n_experts * 4 if wl.routing == "learned" else n * 4 + n * wl.top_k * 8
        gu += g
        dn += dd
        path += g + dd + route_in + n * wl.top_k * 8
        flops += 2.0 * (3 * i * h) * (n * wl.top_k) + 2.0 * (3 * si * h) * n
    k = len(counts_list)
    gu_flops = 2.0 * (2 * i * h) * (n * wl.top_k) + 2.0 * (2 * si * h) * n
    return {"gate_up_bytes": gu / k, "down_bytes": dn / k, "path_bytes": path / k,
            "path_flops": flops / k, "gate_up_flops": gu_flops,
            "per_routed_gate_up_bytes": per_routed_gu, "shared_gate_up_bytes": sh_gu}


class Runner:
    """Pre-built ctypes arguments for every (layer copy, input) pair so a
    step costs four direct library calls."""

    def __init__(self, wl, layers, pool, dev):
        import torch

        from block_quantized_expert_amd import binding as B

        self.B = B
        self.L = B.lib()
        self.wl = wl
        self.layers = layers
        self.pool = pool
        n, k, e = wl.n_tokens, wl.top_k, wl.n_experts
        self.ids = torch.empty((n, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((n, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(e, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(e + 1, dtype=torch.int32, device=dev)
        self.perm = torch.empty(n * k, dtype=torch.int32, device=dev)
        self.inv = torch.empty(n * k, dtype=torch.int32, device=dev)
        self.y = torch.empty((n, wl.hidden), dtype=torch.float32, device=dev)
        self.ws_bytes = layers[0].workspace_bytes(n)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        P = ctypes.c_void_p
        s = P(self.stream.cuda_stream)
        x_type = B.MOE_ACT_F32 if wl.act == "f32" else B.MOE_ACT_BF16
        grouping = (P(self.counts.data_ptr()), P(self.offsets.data_ptr()),
                    P(self.perm.data_ptr()), P(self.inv.data_ptr()))
        self.group_args = (P(self.ids.data_ptr()), n, k, e) + grouping + (None, None, 0, s)
        # learned routing: one fused route+group call; hash routing: the
        # table lookup, then the grouping
        self.route_args = []
        for item in pool:
            if wl.routing == "learned":
                self.route_args.append([("moe_route_group", (
                    P(item["logits"].data_ptr()), n, e, k, ctypes.c_float(wl.routed_scale),
                    P(self.ids.data_ptr()), P(self.w.data_ptr())) + grouping + (None, s))])
            else:
                self.route_args.append([("moe_route_hash", (
                    P(item["token_ids"].data_ptr()), n, P(item["tid2eid"].data_ptr()),
                    P(item["tid2w"].data_ptr()), item["tid2eid"].shape[0], e, k,
                    P(self.ids.data_ptr()), P(self.w.data_ptr()), None, s)),
                    ("moe_group", self.group_args)])
        # single-token learned routing: the whole layer is one moe_forward call
        # (one fused kernel); its outputs land in one set of buffers
        x_type_c = B.MOE_ACT_F32 if wl.act == "f32" else B.MOE_ACT_BF16
        self.fused = (wl.routing == "learned" and
                      self.L.moe_forward_single_kernel(ctypes.byref(layers[0].c), n,
                                                       x_type_c) == 1)
        self.fwd_args = {}
        if self.fused:
            self.fwd = B.ForwardBuffers(layers[0], n, dev)
            for c, layer in enumerate(layers):
                for r, item in enumerate(pool):
                    self.fwd_args[(c, r)] = (
                        [ctypes.byref(layer.c), P(item["logits"].data_ptr()),
                         ctypes.c_float(wl.routed_scale), P(item["x"].data_ptr()), x_type, n]
                        + self.fwd.args() + [s])
        self.ffn_args = {}
        for c, layer in enumerate(layers):
            for r, item in enumerate(pool):
                self.ffn_args[(c, r)] = (
                    ctypes.byref(layer.c), P(item["x"].data_ptr()), x_type, n,
                    P(self.w.data_ptr()), P(self.counts.data_ptr()), P(self.offsets.data_ptr()),
                    P(self.perm.data_ptr()), P(self.inv.data_ptr()), P(self.y.data_ptr()),
                    P(self.ws.data_ptr()), self.ws_bytes, s)

    def step(self, s, ev=None):
        """One pass of the path; ``ev`` = four events that the library
        records from the kernel dispatches themselves: gate/up start and stop,
        down start and stop, or (single fused kernel) its start and stop."""
        c = s % len(self.layers)
        r = s % len(self.pool)
        L = self.L
        if self.fused:
            evs = (None, None) if ev is None else ev[:2]
            if L.moe_forward_timed(*self.fwd_args[(c, r)], *evs):
                raise RuntimeError("moe_forward failed in step %d" % s)
            return
        st = 0
        for name, args in self.route_args[r]:
            st |= getattr(L, name)(*args)
        evs = (None, None, None, None) if ev is None else ev
        st |= L.moe_ffn_forward_timed(*self.ffn_args[(c, r)], *evs)
        if st:
            raise RuntimeError("a moe_* call failed in step %d" % s)


def make_pool(wl, n_items, dev):
    import torch

    from block_quantized_expert_amd import inputs as I

    pool = []
    table = None
    for r in range(n_items):
        item = {"x": I.activations(wl, copy=r).to(dev)}
        if wl.routing == "learned":
            item["logits"] = I.router_logits(wl, copy=r).to(dev)
        else:
            if table is None:
                t2e, t2w = I.hash_table(wl)
                table = (t2e.to(dev), t2w.to(dev))
            item["token_ids"] = I.token_ids(wl, copy=r).to(dev)
            item["tid2eid"], item["tid2w"] = table
        pool.append(item)
    torch.cuda.synchronize()
    return pool


def routed_counts(runner, n_items):
    """Per-input expert counts (route + group again, outside any timing)."""
    import numpy as np
    import torch

    out = []
    for r in range(n_items):
        for name, args in runner.route_args[r]:
            getattr(runner.L, name)(*args)
        torch.cuda.synchronize()
        out.append(runner.counts.cpu().numpy().astype(np.int64))
    return out


def cpu_baseline(wl, seconds_hint: float):
    """The oracle, as it is, on a bounded sample of the same workload: a few
    tokens of fresh inputs through route -> group -> FFN on the host cores.
    Regenerating the sampled experts' weight bytes is input preparation and
    is left out of the time."""
    from threadpoolctl import threadpool_info

    from block_quantized_expert_amd import inputs as I
    from oracle import moe_oracle as O

    n_sample = {"decode1": 1, "decode32": 2, "prefill512": 2, "hash4096": 2}.get(wl.name, 8)
    t_oracle, done, rounds = 0.0, 0, 0
    while (t_oracle < seconds_hint or rounds == 0) and rounds < 48:
        tokens = list(range(min(n_sample, wl.n_tokens)))
        x = I.activations_to_numpy(I.activations(wl, copy=rounds))[tokens]
        r = I.routing_to_numpy(I.routing_inputs(wl, copy=rounds))
        t0 = time.perf_counter()
        if r["kind"] == "learned":
            ids, w = O.route_topk(r["logits"][tokens], wl.top_k, wl.routed_scale)
        else:
            ids, w = O.route_hash(r["token_ids"][tokens], r["tid2eid"], r["tid2w"])
        O.group(ids, wl.n_experts)
        t1 = time.perf_counter()
        needed = sorted({int(e) for e in ids.reshape(-1)})
        layer = I.layer_to_numpy(I.make_layer(wl, device="cpu", experts=needed))
        t2 = time.perf_counter()
        O.ffn(layer, x, wl.act, ids, w)
        t3 = time.perf_counter()
        t_oracle += (t1 - t0) + (t3 - t2)
        done += len(tokens)
        rounds += 1
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    return {"value": done / t_oracle, "unit": "tokens/s",
            "cores": threads or (os.cpu_count() or 1), "kind": "oracle",
            "sample": "%d token(s) of %s from %d fresh input(s), all %d outputs each, "
                      "through the fp64 NumPy oracle (route, group, FFN); %.1f s"
                      % (done, wl.name, rounds, wl.hidden, t_oracle)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode1")
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--pool", type=int, default=None)
    ap.add_argument("--event-every", type=int, default=None,
                    help="record the per-kernel events on every n-th timed step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the warm-up, copy this many MiB once with a plain device "
                         "copy kernel (a known byte count for calibrating memory counters)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: this path runs on a single GPU and has no "
              "multi-GPU mode (asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_quantized_expert_amd import build as _build

    if not os.path.exists(_build.LIB):
        _build.build()
    from block_quantized_expert_amd import binding as B
    from block_quantized_expert_amd import inputs as I

    wl = I.WORKLOADS[args.workload]
    d_steps, d_warm, d_copies, d_pool, d_every = DEFAULTS[wl.name]
    steps = args.steps if args.steps is not None else d_steps
    warmup = args.warmup if args.warmup is not None else d_warm
    copies = args.copies if args.copies is not None else d_copies
    n_pool = args.pool if args.pool is not None else d_pool
    every = max(1, args.event_every if args.event_every is not None else d_every)

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    layers = [B.Layer(I.make_layer(wl, device=dev, copy=c), wl.top_k) for c in range(copies)]
    pool = make_pool(wl, n_pool, dev)
    runner = Runner(wl, layers, pool, dev)
    torch.cuda.synchronize()
    print("setup %.1f s: %d layer copies, %d inputs" % (time.perf_counter() - t0, copies, n_pool),
          file=sys.stderr, flush=True)

    if args.copy_mib > 0:
        # one read and one write of exactly copy_mib MiB, outside the timed region
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for s in range(warmup):
        runner.step(s)
    torch.cuda.synchronize()

    sampled = list(range(0, steps, every))
    evs = [tuple(B.HipEvent() for _ in range(4)) for _ in sampled]
    ev_handles = [None] * steps
    for i, j in enumerate(sampled):
        ev_handles[j] = tuple(e.handle for e in evs[i])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for j in range(steps):
        runner.step(warmup + j, ev_handles[j])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    gate_up_ms = [e[0].elapsed_ms(e[1]) for e in evs]
    gu_avg_s = float(np.mean(gate_up_ms)) / 1e3
    dn_avg_s = float("nan") if runner.fused else float(np.mean(
        [e[2].elapsed_ms(e[3]) for e in evs])) / 1e3
    counts_list = routed_counts(runner, n_pool)
    used = [counts_list[(warmup + j) % n_pool] for j in range(steps)]
    costs = workload_costs(wl, used)

    ms_per_step = elapsed / steps * 1e3
    tokens_per_s = wl.n_tokens * steps / elapsed
    if runner.fused:
        # one kernel does the whole layer: its roof is HBM for all the
        # layer's bytes
        kernel_name = "decode_fused_kernel (moe_forward: route + group + FFN)"
        k_bytes, k_flops = costs["path_bytes"], costs["path_flops"]
    else:
        kernel_name = "gate/up + SwiGLU stage (moe_ffn_gate_up)"
        k_bytes, k_flops = costs["gate_up_bytes"], costs["gate_up_flops"]
    # HBM below the ridge point, the bf16 MFMA peak above it (the
    # contractions run in bf16)
    intensity = k_flops / k_bytes
    mfma_bound = intensity > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    achieved = k_bytes / gu_avg_s / 1e9
    gu_tflops = k_flops / gu_avg_s / 1e12
    path_gbps = costs["path_bytes"] / (elapsed / steps) / 1e9
    path_tflops = costs["path_flops"] / (elapsed / steps) / 1e12
    traffic = kernel_traffic(wl.name)
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "%s: %d token(s), hidden %d, %d routed experts + %s shared, "
                        "intermediate %d, top-%d, %s routing, MXFP4 routed experts, %s "
                        "activations, %d cold layer copies"
                        % (wl.name, wl.n_tokens, wl.hidden, wl.n_experts,
                           "1 " + wl.shared, wl.inter, wl.top_k, wl.routing, wl.act, copies),
            "n_tokens": wl.n_tokens,
        },
        "roofline": {
            "kernel": kernel_name,
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": gu_tflops if mfma_bound else achieved,
            "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": gu_tflops / MFMA_BF16_PEAK_TFLOPS if mfma_bound else achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "bytes_per_launch": k_bytes,
            "flops_per_launch": k_flops,
            "flop_per_byte": intensity,
            "avg_launch_us": gu_avg_s * 1e6,
            "timed_launches": len(sampled),
        },
        "down_kernel": None if runner.fused else {
            "bytes_per_launch": costs["down_bytes"],
            "avg_launch_us": dn_avg_s * 1e6,
            "achieved_GBps": costs["down_bytes"] / dn_avg_s / 1e9,
        },
        "path": {
            "bytes_per_step": costs["path_bytes"],
            "achieved_GBps": path_gbps,
            "hbm_frac": path_gbps / HBM_PEAK_GBPS,
            "flops_per_step": costs["path_flops"],
            "achieved_TFLOPs": path_tflops,
            "mfma_bf16_frac": path_tflops / MFMA_BF16_PEAK_TFLOPS,
        },
    }
    if runner.fused:
        print("timed %d steps in %.3f s: %.2f us/step, fused kernel %.2f us (%.0f GB/s), "
              "path %.0f GB/s" % (steps, elapsed, ms_per_step * 1e3, gu_avg_s * 1e6, achieved,
                                  path_gbps), file=sys.stderr, flush=True)
    else:
        print("timed %d steps in %.3f s: %.2f us/step, gate/up %.2f us (%.0f GB/s), down %.2f us "
              "(%.0f GB/s), path %.0f GB/s"
              % (steps, elapsed, ms_per_step * 1e3, gu_avg_s * 1e6, achieved, dn_avg_s * 1e6,
                 costs["down_bytes"] / dn_avg_s / 1e9, path_gbps), file=sys.stderr, flush=True)
    del runner, layers, pool
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

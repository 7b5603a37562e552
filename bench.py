#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN hot path on one MI355X.

One step = route -> group -> gate/up (+SwiGLU) -> down (+combine) over one
batch of synthetic input, every kernel launched through the C ABI of
libmoe.so on one HIP stream.

The headline line is the largest workload that fits one GPU: the hash-routed
prefill of 4096 tokens on the DeepSeek-V4-Flash-shaped layer (hidden 4096,
256 routed MXFP4 experts + 1 fp8-e4m3 shared, intermediate 2048, top-6).
Its K timed steps follow W warm-up steps.  The other workloads (tiny,
single-token decode, batched decode of 32, prefill of 512) are measured in
the same run, each with its own step count, and reported as nested records
under "configs", together with records of the routing and FFN options
(VARIANTS: tail pruning, group-limited top-k, the gate-first lazy skip) on
those workloads (``--workload NAME`` measures only that one as the line).

Cold caches: the weights live in several independent layer copies (3.44 GB
each) used round-robin, and every step takes a fresh batch from a seeded
pool, so no expert is served from the 256 MB last-level cache or the L2s.

Every record holds:
- ``value``: tokens/s over its timed steps (wall clock, synchronised on both
  sides) and ``ms_per_step``;
- ``step_stats``: the timed steps split into five consecutive repetitions,
  each timed with stream events: median, min and max of the per-step time,
  and ``spread_over_15pct`` when (max - min) / median > 0.15;
- ``roofline``: the kernel that runs the routed experts' gate/up (at one
  token, the single kernel that does the whole layer), its algorithmic bytes
  or flops per launch over its average duration from HIP events that its own
  dispatch records (on the stream it runs on).  Those events are taken in a
  pass of at least 20 more steps right after the timed steps (the same
  rotation of layer copies and inputs, so still cold): a dispatch that
  records events leaves the GPU idle for several microseconds, which at
  single-token decode (a ~29 us step) would inflate the timed steps;
- ``cpu_baseline``: the fp64 oracle on a bounded sample of the same workload
  on the host cores.
The line also carries ``hbm_read_ceiling``: the rate of a plain streaming
read over 4 GiB (moe_stream_read), the measured ceiling beside the 8 TB/s
published figure; and ``mfma_issue_ceiling``: the rate at which independent
scaled matrix instructions issue (moe_mfma_rate), for the instruction the
grouped GEMMs use and for the 32x32x64 shape with E2M1 x E2M3 operands.
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
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8, published
HEADLINE = "hash4096"
PACK = True  # --no-pack: the batched GEMMs read the row-major weights
NESTED = ["tiny", "decode1", "decode32", "prefill512"]
REPS = 5

# Routing and FFN options (moe_opts) measured on top of a workload, as nested
# records: name -> (workload, options).  "sel_bias" draws the per-expert
# selection bias of the inputs module (N(0, 0.5^2)).
VARIANTS = {
    # tail pruning with L2 rescaling: at most 4 or 5 of the 6 routed experts
    # ("Deep-Dive Mathematical & Kernel Guide", section 3.2 configuration table)
    "decode1_top4": ("decode1", dict(keep_max=4)),
    "decode1_top5": ("decode1", dict(keep_max=5)),
    "decode32_top4": ("decode32", dict(keep_max=4)),
    # group-limited top-k (8 groups, 4 kept) with a selection-only bias
    "decode1_groups": ("decode1", dict(n_group=8, topk_group=4, sel_bias=True)),
    "decode32_groups": ("decode32", dict(n_group=8, topk_group=4, sel_bias=True)),
    # gate-first lazy skip at the RFC's threshold: the gate rows first, then the
    # up rows of the experts some token keeps (on these inputs every expert is
    # kept, so this is the cost of the gate-first order)
    "decode1_lazy": ("decode1", dict(lazy_tau=1e-3)),
}

# workload: (steps, warmup, copies, pool) when it is measured as a nested
# record or as the line without --steps/--warmup
DEFAULTS = {
    "tiny": (2000, 100, 1, 8),
    "decode1": (2000, 100, 8, 64),
    "decode32": (400, 20, 8, 16),
    "prefill512": (100, 10, 8, 4),
    "hash4096": (20, 5, 2, 2),
}
MIN_EVENT_SAMPLES = 20

# HBM traffic of the roofline kernel per launch, from two rocprofv3 --pmc
# passes over this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch of
# that kernel, averaged over the dispatches after the first fifth), each
# scaled by what the same counter reads for a plain 256 MiB device copy run
# in the same process (--copy-mib 256): FETCH_SIZE read 131093.3 KiB for
# 262144 KiB read (it counts a 128-byte request as 64 bytes; a third pass by
# request size showed these kernels issue 128-byte reads only), WRITE_SIZE
# 262144 KiB for 262144 KiB written.  Only kernels unchanged since their
# counters were taken are listed.
FETCH_SCALE = 262144.0 / 131093.3
WRITE_SCALE = 1.0
KERNEL_TRAFFIC_KIB = {  # (workload, packed copy used): (FETCH_SIZE, WRITE_SIZE) per dispatch
    ("decode1", False): (46204.5, 82.2),        # decode_fused_kernel<8, false>
    ("decode32", False): (475411.1, 5502.4),    # gemm_gate_up_kernel<0, 112, true, true, false, false, false>
    ("prefill512", False): (1180630.5, 27385.2),
    ("hash4096", False): (2131057.8, 176253.2),
    ("decode1", True): (46191.4, 82.2),         # decode_fused_kernel<8, true>
    ("decode32", True): (478980.2, 3448.8),     # gemm_gate_up_kernel<0, 112, true, true, false, true, false>
    ("prefill512", True): (1168681.3, 24638.4),
    ("hash4096", True): (1549354.8, 147249.9),  # gemm_gate_up_mix_kernel<false>
}


def kernel_traffic(name, packed):
    kib = KERNEL_TRAFFIC_KIB.get((name, packed))
    if kib is None:
        return None
    return (kib[0] * FETCH_SCALE + kib[1] * WRITE_SCALE) * 1024.0


def proj_bytes(wtype: str, rows: int, cols: int) -> int:
    """Stored bytes of one expert matrix (codes + scales)."""
    if wtype == "mxfp4":
        return rows * cols // 2 + rows * cols // 32
    return rows * cols + rows * cols // 128


def shared_in_routed_launch(wl, packed):
    """Whether the shared expert's gate/up and down run in the routed
    experts' launches: when it is stored like them, and for an fp8 shared
    expert next to packed MXFP4 routed experts on the E2M3 down path (at
    least 16 routed slots per expert, intermediate sizes up to 2048)."""
    if wl.shared == wl.routed:
        return True
    si = wl.shared_inter or wl.inter
    return (packed and wl.routed == "mxfp4" and wl.shared == "fp8_e4m3_b128"
            and wl.n_tokens * wl.top_k >= 16 * wl.n_experts
            and wl.inter <= 2048 and si <= 2048)


def workload_costs(wl, counts_list, same=None):
    """Algorithmic bytes and flops, averaged over the steps' routings.

    Routed gate/up kernel: the gate and up matrices of every routed expert
    with at least one token (plus the shared expert when it runs in the same
    launch: ``same``, by default when it is stored like the routed ones) and
    the activations.
    Routed down kernel: the down matrices of the same experts and y.  Whole
    path: every expert touched + shared + x + router input + ids/weights + y.
    Flops: 2*2*I*H per (token, expert) for gate/up, 2*I*H for down, the
    shared expert counted with weight 1.  Implementation traffic (h,
    per-slot outputs, quantized activations, the permutation) is not counted.
    """
    h, i = wl.hidden, wl.inter
    si = wl.shared_inter or wl.inter
    act = 4 if wl.act == "f32" else 2
    per_gu = 2 * proj_bytes(wl.routed, i, h)
    per_dn = proj_bytes(wl.routed, h, i)
    sh_gu = 2 * proj_bytes(wl.shared, si, h)
    sh_dn = proj_bytes(wl.shared, h, si)
    if same is None:
        same = wl.shared == wl.routed
    n, k = wl.n_tokens, wl.top_k
    gu = dn = path = slots = 0.0
    for counts in counts_list:
        d = int((counts > 0).sum())
        gu += d * per_gu + (sh_gu if same else 0) + n * h * act
        dn += d * per_dn + (sh_dn if same else 0) + n * h * 4
        route_in = n * wl.n_experts * 4 if wl.routing == "learned" else n * 4 + n * k * 8
        path += (d * (per_gu + per_dn) + sh_gu + sh_dn + n * h * act + n * h * 4 + route_in
                 + n * k * 8)
        slots += int(counts.sum())  # n*k, or fewer after tail pruning
    c = len(counts_list)
    slots /= c
    sh_tok = n if same else 0
    return {
        "gate_up_bytes": gu / c, "down_bytes": dn / c, "path_bytes": path / c,
        "gate_up_flops": 4.0 * i * h * slots + 4.0 * si * h * sh_tok,
        "down_flops": 2.0 * i * h * slots + 2.0 * si * h * sh_tok,
        "path_flops": 6.0 * i * h * slots + 6.0 * si * h * n,
        "routed_slots": slots,
    }


class Runner:
    """Pre-built ctypes arguments for every (layer copy, input) pair so a
    step costs a few direct library calls."""

    def __init__(self, wl, layers, pool, dev, opts=None):
        import torch

        from block_quantized_expert_amd import binding as B

        self.B = B
        self.L = B.lib()
        self.wl = wl
        self.layers = layers
        self.pool = pool
        self.opts = opts
        o = None if opts is None else ctypes.byref(opts)
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
                self.route_args.append([("moe_route_group_ex", (
                    P(item["logits"].data_ptr()), n, e, k, ctypes.c_float(wl.routed_scale), o,
                    P(self.ids.data_ptr()), P(self.w.data_ptr())) + grouping + (None, s))])
            else:
                self.route_args.append([("moe_route_hash", (
                    P(item["token_ids"].data_ptr()), n, P(item["tid2eid"].data_ptr()),
                    P(item["tid2w"].data_ptr()), item["tid2eid"].shape[0], e, k,
                    P(self.ids.data_ptr()), P(self.w.data_ptr()), None, s)),
                    ("moe_group", self.group_args)])
        # single-token learned routing: the whole layer is one moe_forward call
        # (one fused kernel); its outputs land in one set of buffers
        self.fused = (wl.routing == "learned" and
                      self.L.moe_forward_single_kernel(ctypes.byref(layers[0].c), n,
                                                       x_type) == 1 and
                      (opts is None or opts.lazy_tau == 0.0))
        self.fwd_args = {}
        if self.fused:
            self.fwd = B.ForwardBuffers(layers[0], n, dev)
            for c, layer in enumerate(layers):
                for r, item in enumerate(pool):
                    self.fwd_args[(c, r)] = (
                        [ctypes.byref(layer.c), P(item["logits"].data_ptr()),
                         ctypes.c_float(wl.routed_scale), o, P(item["x"].data_ptr()), x_type, n]
                        + self.fwd.args() + [s])
        self.ffn_args = {}
        for c, layer in enumerate(layers):
            for r, item in enumerate(pool):
                self.ffn_args[(c, r)] = (
                    ctypes.byref(layer.c), P(item["x"].data_ptr()), x_type, n,
                    P(self.w.data_ptr()), P(self.counts.data_ptr()), P(self.offsets.data_ptr()),
                    P(self.perm.data_ptr()), P(self.inv.data_ptr()), P(self.y.data_ptr()), o,
                    P(self.ws.data_ptr()), self.ws_bytes, s)

    def step(self, s, ev=None):
        """One pass of the path; ``ev`` = four events that the library
        records from the kernel dispatches themselves: routed gate/up kernel
        start and stop, routed down kernel start and stop, or (single fused
        kernel) its start and stop."""
        c = s % len(self.layers)
        r = s % len(self.pool)
        L = self.L
        if self.fused:
            evs = (None, None) if ev is None else ev[:2]
            if L.moe_forward_ex(*self.fwd_args[(c, r)], *evs):
                raise RuntimeError("moe_forward_ex failed in step %d" % s)
            return
        st = 0
        for name, args in self.route_args[r]:
            st |= getattr(L, name)(*args)
        evs = (None, None, None, None) if ev is None else ev
        st |= L.moe_ffn_forward_ex(*self.ffn_args[(c, r)], *evs)
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


def describe(wl, copies):
    return ("%s: %d token(s), hidden %d, %d routed experts (%s) + 1 shared (%s), "
            "intermediate %d, top-%d, %s routing, %s activations, %d cold layer copies"
            % (wl.name, wl.n_tokens, wl.hidden, wl.n_experts, wl.routed, wl.shared, wl.inter,
               wl.top_k, wl.routing, wl.act, copies))


def step_stats(rep_ms, rep_steps):
    import numpy as np

    per = np.array(rep_ms) / np.array(rep_steps) * 1e3  # us per step in each repetition
    med = float(np.median(per))
    return {"reps": len(per), "steps_per_rep": list(rep_steps),
            "us_per_step_median": med, "us_per_step_min": float(per.min()),
            "us_per_step_max": float(per.max()),
            "spread_over_15pct": bool((per.max() - per.min()) / med > 0.15)}


def run_workload(name, steps, warmup, copies, n_pool, cpu_seconds, dev, variant=None):
    """Measure one workload (with the options of `variant`, a key of
    VARIANTS); returns its record (without the top-level contract keys)."""
    import numpy as np
    import torch

    from block_quantized_expert_amd import binding as B
    from block_quantized_expert_amd import inputs as I

    wl = I.WORKLOADS[name]
    opts, opts_desc = None, None
    if variant is not None:
        kw = dict(VARIANTS[variant][1])
        if kw.pop("sel_bias", False):
            kw["sel_bias"] = I.selection_bias(wl).to(dev)
        opts = B.make_opts(**kw)
        opts_desc = {k: (v if k != "sel_bias" else "N(0, 0.5^2) per expert")
                     for k, v in kw.items()}
    t0 = time.perf_counter()
    layers = [B.Layer(I.make_layer(wl, device=dev, copy=c), wl.top_k) for c in range(copies)]
    # the packed copy of the MXFP4 matrices (moe_pack_experts, once per layer
    # like loading the weights): read by the batched gate/up and down and by
    # the single-token fused kernel
    pool = make_pool(wl, n_pool, dev)
    runner = Runner(wl, layers, pool, dev, opts)
    packed = (PACK and wl.act == "bf16" and (wl.n_tokens > 16 or runner.fused)
              and all(l.pack() for l in layers))
    name = variant or name
    torch.cuda.synchronize()
    print("%s setup %.1f s: %d layer copies, %d inputs" % (name, time.perf_counter() - t0,
                                                            copies, n_pool),
          file=sys.stderr, flush=True)

    for s in range(warmup):
        runner.step(s)
    torch.cuda.synchronize()

    # repetition boundaries: stream events between steps
    reps = min(REPS, steps)
    bounds = [round(r * steps / reps) for r in range(reps + 1)]
    rep_ev = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    stream = runner.stream
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    b = 0
    for j in range(steps):
        if j == bounds[b]:
            rep_ev[b].record(stream)
            b += 1
        runner.step(warmup + j)
    rep_ev[b].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    rep_ms = [rep_ev[r].elapsed_time(rep_ev[r + 1]) for r in range(reps)]
    rep_steps = [bounds[r + 1] - bounds[r] for r in range(reps)]

    # kernel durations: events recorded by the kernels' own dispatches, on
    # every step of a further pass that continues the same rotation
    n_samp = max(MIN_EVENT_SAMPLES, min(steps // 4, 250))
    evs = [tuple(B.HipEvent() for _ in range(4)) for _ in range(n_samp)]
    first = warmup + steps
    for i in range(n_samp):
        runner.step(first + i, tuple(e.handle for e in evs[i]))
    torch.cuda.synchronize()
    gu_avg_s = float(np.mean([e[0].elapsed_ms(e[1]) for e in evs])) / 1e3
    dn_avg_s = None if runner.fused else float(np.mean([e[2].elapsed_ms(e[3]) for e in evs])) / 1e3
    counts_list = routed_counts(runner, n_pool)
    used = [counts_list[(warmup + j) % n_pool] for j in range(steps)]
    used_samp = [counts_list[(first + i) % n_pool] for i in range(n_samp)]
    same = shared_in_routed_launch(wl, packed)
    costs = workload_costs(wl, used, same)
    kcosts = workload_costs(wl, used_samp, same)

    ms_per_step = elapsed / steps * 1e3
    if runner.fused:
        kernel_name = "decode_fused_kernel<%d> (moe_forward: route + group + FFN)" % (wl.hidden // 512)
        k_bytes, k_flops, issue = kcosts["path_bytes"], kcosts["path_flops"], 1.0
    else:
        kernel_name = ("routed gate/up kernel of moe_ffn_forward (+ SwiGLU)"
                       + (", with the shared expert's items" if same else ""))
        k_bytes, k_flops = kcosts["gate_up_bytes"], kcosts["gate_up_flops"]
        # bf16 x on the grouped GEMMs: each product issued once per E4M3 part
        # of x (two) on the scaled fp8 instruction
        issue = 2.0 if (wl.act == "bf16" and wl.n_tokens > 16) else 1.0
    intensity = k_flops / k_bytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    mfma_bound = intensity > ridge
    gbps = k_bytes / gu_avg_s / 1e9
    tflops = k_flops / gu_avg_s / 1e12
    roof = {
        "kernel": kernel_name,
        "bound": "mfma" if mfma_bound else "hbm",
        "achieved": tflops if mfma_bound else gbps,
        "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "frac": tflops / MFMA_BF16_PEAK_TFLOPS if mfma_bound else gbps / HBM_PEAK_GBPS,
        "traffic": kernel_traffic(name, packed),
        "bytes_per_launch": k_bytes,
        "flops_per_launch": k_flops,
        "flop_per_byte": intensity,
        "avg_launch_us": gu_avg_s * 1e6,
        "timed_launches": n_samp,
        "timing": "dispatch-recorded HIP events on every step of a %d-step pass right "
                  "after the timed steps (same rotation, cold)" % n_samp,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "mfma_bf16_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
    }
    if issue > 1.0:
        roof["peak_note"] = ("bf16-equivalent: algorithmic flops against the dense bf16 peak; "
                             "the kernel issues each product %d times (once per E4M3 part of x) "
                             "on v_mfma_scale_f32_16x16x128_f8f6f4 at the fp8 rate" % issue)
        roof["issued_flops_per_launch"] = issue * k_flops
        roof["issued_frac_of_fp8_peak"] = issue * tflops / MFMA_FP8_PEAK_TFLOPS
    rec = {
        "workload": name,
        "config": {"workload": describe(wl, copies), "n_tokens": wl.n_tokens,
                   "packed_experts": packed},
        "routed_slots_per_step": costs["routed_slots"],
        "value": wl.n_tokens * steps / elapsed,
        "unit": "tokens/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "step_stats": step_stats(rep_ms, rep_steps),
        "roofline": roof,
        "path": {
            "bytes_per_step": costs["path_bytes"],
            "achieved_GBps": costs["path_bytes"] / (elapsed / steps) / 1e9,
            "hbm_frac": costs["path_bytes"] / (elapsed / steps) / 1e9 / HBM_PEAK_GBPS,
            "flops_per_step": costs["path_flops"],
            "achieved_TFLOPs": costs["path_flops"] / (elapsed / steps) / 1e12,
            "mfma_bf16_frac": costs["path_flops"] / (elapsed / steps) / 1e12
                              / MFMA_BF16_PEAK_TFLOPS,
        },
    }
    if dn_avg_s is not None:
        dissue = 3.0 if issue > 1.0 else 1.0  # h as three E4M3 parts
        rec["down_kernel"] = {
            "kernel": "routed down kernel of moe_ffn_forward" + (", with the shared expert's items" if same else ""),
            "bytes_per_launch": kcosts["down_bytes"],
            "flops_per_launch": kcosts["down_flops"],
            "avg_launch_us": dn_avg_s * 1e6,
            "achieved_GBps": kcosts["down_bytes"] / dn_avg_s / 1e9,
            "achieved_TFLOPs": kcosts["down_flops"] / dn_avg_s / 1e12,
            "mfma_bf16_frac": kcosts["down_flops"] / dn_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "issued_frac_of_fp8_peak": dissue * kcosts["down_flops"] / dn_avg_s / 1e12
                                       / MFMA_FP8_PEAK_TFLOPS,
        }
    if opts_desc is not None:
        rec["config"]["options"] = opts_desc
        rec["config"]["path"] = ("single fused kernel" if runner.fused else
                                 "route+group kernel(s), gate/up, down")
    st = rec["step_stats"]
    print("%s: %d steps %.2f us/step (reps median %.2f, min %.2f, max %.2f), roofline kernel "
          "%.2f us (%.0f GB/s, %.0f TFLOP/s)%s" % (
              name, steps, ms_per_step * 1e3, st["us_per_step_median"], st["us_per_step_min"],
              st["us_per_step_max"], gu_avg_s * 1e6, gbps, tflops,
              "" if dn_avg_s is None else ", down %.2f us" % (dn_avg_s * 1e6)),
          file=sys.stderr, flush=True)
    del runner, layers, pool
    torch.cuda.empty_cache()
    if cpu_seconds > 0 and variant is None:
        rec["cpu_baseline"] = cpu_baseline(wl, cpu_seconds)
    return rec


def read_ceiling(dev, gib=4, reps=5):
    """GB/s of moe_stream_read over a cold buffer of `gib` GiB (median and
    best of `reps` runs after one warm-up)."""
    import numpy as np
    import torch

    from block_quantized_expert_amd import binding as B

    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    L = B.lib()
    args = (ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
            ctypes.c_void_p(s.cuda_stream))
    if L.moe_stream_read(*args):
        raise RuntimeError("moe_stream_read failed")
    rates = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        L.moe_stream_read(*args)
        b.record(s)
        torch.cuda.synchronize()
        rates.append(n / (a.elapsed_time(b) / 1e3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return {"kernel": "moe_stream_read (16 B per lane and load, 4 loads in flight per lane)",
            "bytes": n, "GBps_median": float(np.median(rates)), "GBps_max": float(max(rates)),
            "frac_of_published": float(np.median(rates)) / HBM_PEAK_GBPS}


def mfma_ceiling(dev, iters=8000, reps=5):
    """TFLOP/s that moe_mfma_rate issues (median and best of `reps` runs of
    a few milliseconds after one warm-up) for the instruction the grouped
    GEMMs use (16x16x128, E2M1 weights x E4M3 activations) and for the
    32x32x64 shape with E2M1 x E2M3 operands."""
    import numpy as np
    import torch

    from block_quantized_expert_amd import binding as B

    L = B.lib()
    n = L.moe_mfma_rate_out_floats()
    out = torch.empty(max(int(n), 1), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()
    waves = n // 64
    res = {}
    for label, shape, fa, fb in (("16x16x128 E2M1 x E4M3 (the kernels' instruction)", 16, 4, 0),
                                 ("32x32x64 E2M1 x E2M3", 32, 4, 2)):
        args = (shape, fa, fb, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
        if L.moe_mfma_rate(*args):
            raise RuntimeError("moe_mfma_rate failed")
        flops = waves * iters * (8 * 2 * 16 * 16 * 128 if shape == 16 else 4 * 2 * 32 * 32 * 64)
        rates = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            L.moe_mfma_rate(*args)
            b.record(s)
            torch.cuda.synchronize()
            rates.append(flops / (a.elapsed_time(b) / 1e3) / 1e12)
        res[label] = {"median": float(np.median(rates)), "max": float(max(rates))}
    return {"kernel": "moe_mfma_rate (independent scaled MFMAs, operands in registers)",
            "TFLOPs": res, "fp8_peak_TFLOPs": 5000.0}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    help="measure only this workload (default: %s as the line, the others "
                         "as nested records)" % HEADLINE)
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--pool", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-pack", action="store_true",
                    help="batched workloads without the packed copy of the weights")
    ap.add_argument("--no-variants", action="store_true",
                    help="leave out the nested records of the routing/FFN options")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the warm-up, copy this many MiB once with a plain device "
                         "copy kernel (a known byte count for calibrating memory counters)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--nested-cpu-seconds", type=float, default=4.0)
    args = ap.parse_args()
    global PACK
    PACK = not args.no_pack

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: this path runs on a single GPU and has no "
              "multi-GPU mode (asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_quantized_expert_amd import build as _build

    if not os.path.exists(_build.LIB):
        _build.build()

    dev = torch.device("cuda:0")
    if args.copy_mib > 0:
        # one read and one write of exactly copy_mib MiB, outside the timed regions
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    line_name = args.workload or HEADLINE
    nested = [] if args.workload else NESTED
    cpu = not args.no_cpu_baseline
    configs = {}
    for name in nested:
        st, wu, cp, po = DEFAULTS[name]
        configs[name] = run_workload(name, st, wu, cp, po,
                                     args.nested_cpu_seconds if cpu else 0.0, dev)
    if not args.workload and not args.no_variants:
        for var, (name, _) in VARIANTS.items():
            st, wu, cp, po = DEFAULTS[name]
            configs[var] = run_workload(name, st, wu, cp, po, 0.0, dev, variant=var)
    variant = None
    if line_name in VARIANTS:  # a workload with options, measured alone
        variant, line_name = line_name, VARIANTS[line_name][0]
    st, wu, cp, po = DEFAULTS[line_name]
    steps = args.steps if args.steps is not None else st
    warmup = args.warmup if args.warmup is not None else wu
    rec = run_workload(line_name, steps, warmup,
                       args.copies if args.copies is not None else cp,
                       args.pool if args.pool is not None else po,
                       args.cpu_seconds if cpu else 0.0, dev, variant=variant)

    result = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "compute": "E2M1 expert weights with UE8M0 block scales on the matrix cores "
                   "(batched: gate/up with exact E4M3 parts of the bf16 activations on "
                   "v_mfma_scale_f32_16x16x128_f8f6f4, down with h as three E4M3 parts on "
                   "the same instruction or, packed with >= 16 slots per expert, as three "
                   "E2M3 parts on v_mfma_scale_f32_32x32x64_f8f6f4; one token: decoded "
                   "exactly to bf16); fp32 accumulation",
        "data": "synthetic",
        "config": rec["config"],
        "step_stats": rec["step_stats"],
        "roofline": rec["roofline"],
        "path": rec["path"],
    }
    if "down_kernel" in rec:
        result["down_kernel"] = rec["down_kernel"]
    if "cpu_baseline" in rec:
        result["cpu_baseline"] = rec["cpu_baseline"]
    if not args.no_ceiling:
        result["hbm_read_ceiling"] = read_ceiling(dev)
        result["mfma_issue_ceiling"] = mfma_ceiling(dev)
    if configs:
        result["configs"] = configs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

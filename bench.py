#!/usr/bin/env python3
"""Paged-decode benchmark on one MI355X.

Headline workload: single-user long-context split-KV decode.  One step is one
decoded token through 32 layers; per layer, one append-form split-KV call
stores the new token's K/V into that layer's block-paged cache and attends
over the 32768-token context (partition 512: the partition kernel, which also
does the store, then the log-sum-exp merge kernel).  Batch 1, q_len 1, 32
query / 8 KV heads, head_dim 128, fp16, 2048 blocks of 16 per layer in a
randomly permuted pool, one block table shared by the layers.  32 distinct
layer caches (4 GiB) keep the working set far beyond the 256 MB Infinity
Cache.  The step's 64 launches are captured once in a HIP graph and replayed,
as a decode loop runs them; the same step launched eagerly, and the unfused
two-call step (kv_cache_write, then split-KV decode), are reported beside it.

value = KV bytes streamed per step (32 x 128 MiB) / step time, with all inputs
resident in HBM.  The dominant kernel's roofline entry uses HIP events around
32 back-to-back launches of the partition kernel on its launch stream, in a
second pass of the same work (the headline pass carries no extra events).

python bench.py [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]
python bench.py --ceiling      # read ceiling of the 32K layer (probe library) + the kernel
python bench.py --ceiling-k8v4 # the same for the K8/V4 batch
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-decode KV-stream GB/s (% of 8 TB/s HBM) + us/layer at 32K ctx"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_partition_long32k.json")
KERNEL_SOURCES = ["paged_kv_cache_181_amd/csrc/attn_kernels.hip",
                  "paged_kv_cache_181_amd/csrc/pkv_common.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--partition", type=int, default=512)
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="skip the other four workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (scale for rocprofv3 byte counters)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the read ceiling of the 32K layer with the probe library, "
                         "next to the partition kernel")
    ap.add_argument("--ceiling-k8v4", action="store_true",
                    help="only measure the read ceiling of the K8/V4 batch with the probe library, "
                         "next to its partition kernel")
    ap.add_argument("--only", default=None,
                    help="time only this one of the other workloads (for profiling), e.g. k8v4")
    ap.add_argument("--only-partition", default=None,
                    help="with --only: the split to time instead of the workload's own "
                         "(direct, 0 for the balanced split, or a partition size)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------

class Long32K:
    """Headline: batch 1, 32K context, 32 layers, split-KV decode."""
    name = "long32k"

    def __init__(self, P, W, torch, layers, partition, seed):
        import numpy as np
        self.P, self.torch, self.layers, self.partition = P, torch, layers, partition
        dev = torch.device("cuda:0")
        case = W.long32k(seed)
        self.case = case
        self.L = int(case.context_lens[0])
        self.hq, self.hkv, self.d = case.num_q_heads, case.num_kv_heads, case.head_dim
        self.nb = case.num_blocks
        up = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.float16)  # noqa: E731
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed * 1000)
        shape = (self.nb, 16, self.hkv, self.d)
        self.K, self.V, self.q, self.nk, self.nv = [], [], [], [], []
        for l in range(layers):
            if l == 0:          # the parity-tested seeded case, byte for byte
                self.K.append(up(case.key_cache))
                self.V.append(up(case.value_cache))
                self.q.append(up(case.query))
                self.nk.append(up(case.new_key))
                self.nv.append(up(case.new_value))
            else:
                self.K.append(torch.randn(shape, generator=gen, device=dev, dtype=torch.float16))
                self.V.append(torch.randn(shape, generator=gen, device=dev, dtype=torch.float16))
                self.q.append(torch.randn(case.query.shape, generator=gen, device=dev,
                                          dtype=torch.float16))
                self.nk.append(torch.randn(case.new_key.shape, generator=gen, device=dev,
                                           dtype=torch.float16))
                self.nv.append(torch.randn(case.new_value.shape, generator=gen, device=dev,
                                           dtype=torch.float16))
        self.bt = torch.from_numpy(case.block_tables).to(dev)
        self.cl = torch.from_numpy(case.context_lens).to(dev)
        self.slots = torch.from_numpy(case.slot_mapping).to(dev)
        self.out = [torch.empty(case.query.shape, dtype=torch.float16, device=dev)
                    for _ in range(layers)]
        nbytes = P.splitkv_workspace_size(1, 1, self.hq, self.d, self.L, partition)
        self.ws = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)
        # algorithmic KV bytes one layer must read: K and V rows of every position
        self.layer_bytes = self.L * self.hkv * self.d * 2 * 2
        self.step_bytes = self.layer_bytes * layers

    def step(self):
        """Per layer: store the new token and attend (append form)."""
        P, c = self.P, self.case
        for l in range(self.layers):
            P.paged_attention_decode_splitkv_append(self.out[l], self.q[l], self.nk[l], self.nv[l],
                                                    self.K[l], self.V[l], self.bt, self.cl,
                                                    c.scale, c.gqa_factor, self.L,
                                                    self.partition, self.ws)

    def step_two_call(self):
        """The same step as two calls per layer: kv_cache_write, then split-KV
        decode over a length that includes the new token."""
        P, c = self.P, self.case
        for l in range(self.layers):
            P.kv_cache_write(self.nk[l], self.nv[l], self.K[l], self.V[l], self.slots)
            P.paged_attention_decode_splitkv(self.out[l], self.q[l], self.K[l], self.V[l], self.bt,
                                             self.cl, c.scale, c.gqa_factor, self.L,
                                             self.partition, self.ws)

    def step_write_only(self):
        """Only the slot scatter of a step: one kv_cache_write per layer (the
        new token's K and V rows into that layer's cache)."""
        P = self.P
        for l in range(self.layers):
            P.kv_cache_write(self.nk[l], self.nv[l], self.K[l], self.V[l], self.slots)

    def step_timed_kernels(self):
        """The same work as a step, reordered so that the 32 partition-kernel
        launches run back to back between two events: the partition kernels
        (append form, one workspace per layer), then the merges."""
        P, c, torch = self.P, self.case, self.torch
        if not hasattr(self, "wss"):
            self.wss = [torch.zeros_like(self.ws) for _ in range(self.layers)]
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for l in range(self.layers):
            P.paged_attention_decode_splitkv_append_partials(
                self.q[l], self.nk[l], self.nv[l], self.K[l], self.V[l], self.bt, self.cl,
                c.scale, c.gqa_factor, self.L, self.partition, self.wss[l])
        e.record()
        for l in range(self.layers):
            P.paged_attention_decode_splitkv_merge(self.out[l], self.L, self.partition, self.wss[l])
        return s, e


def long32k_other_partition(wl, P, torch, part, steps, warmup):
    """The headline step (append form, same 32 layer caches) at another
    partition size; reported beside the headline, which keeps 512."""
    c = wl.case
    n = P.splitkv_workspace_size(1, 1, wl.hq, wl.d, wl.L, part)
    ws = torch.zeros(n // 4 + 4, dtype=torch.float32, device="cuda")

    def step():
        for l in range(wl.layers):
            P.paged_attention_decode_splitkv_append(wl.out[l], wl.q[l], wl.nk[l], wl.nv[l], wl.K[l],
                                                    wl.V[l], wl.bt, wl.cl, c.scale, c.gqa_factor,
                                                    wl.L, part, ws)
    ms, med = time_steps(torch, graph_of(torch, step).replay, steps, warmup, median=True)
    us = ms * 1e3 / wl.layers
    return {"us_per_layer": round(us, 3), "median_us_per_layer": round(med * 1e3 / wl.layers, 3),
            "kv_bytes_per_layer": wl.layer_bytes,
            "kv_stream_gbs": round(wl.layer_bytes / (us * 1e-6) / 1e9, 2),
            "pct_of_hbm_peak": round(100 * wl.layer_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "layers": wl.layers, "partition_size": part,
            "form": f"split-KV partition {part} (eight KV heads per workgroup, one wave per head), "
                    "append form, HIP graph; finer partials than the 512-token headline"}


def graph_of(torch, fn):
    """Capture one call of ``fn`` (a whole step's launches, stream-ordered on
    the current stream) into a HIP graph.  Nothing is allocated or cleared by
    the launches, so replays redo exactly the captured work."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_steps(torch, fn, steps, warmup, median=False):
    """ms per step over `steps` steps after `warmup` untimed ones: the mean
    (first to last event), and with `median` also the median of the per-step
    intervals (an event between consecutive steps)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[-1]) / steps
    if not median:
        return mean
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    med = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return mean, med


def kernel_average_ms(torch, wl, steps):
    """Average partition-kernel duration from HIP events on its launch stream:
    one event pair around the 32 back-to-back partition launches of a step (the
    merges follow after the closing event), averaged over ``steps`` steps."""
    total, n = 0.0, 0
    for _ in range(steps):
        ev = wl.step_timed_kernels()
        torch.cuda.synchronize()
        total += ev[0].elapsed_time(ev[1])
        n += wl.layers
    return total / n, n


def source_digest():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel source as it is now; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline_tiny_one_thread(W, seconds=2.0):
    """The oracle on the tiny workload (one sequence of 256 tokens, 8/2
    heads, D 64) with BLAS held to one thread: microseconds per call."""
    import oracle
    c = W.tiny()
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except Exception:
        limit = None
    try:
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.paged_attention(c.query, c.key_cache, c.value_cache, c.block_tables,
                                   c.context_lens, c.scale, c.gqa_factor, "f16")
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 2000:
                break
    finally:
        if limit is not None:
            limit.unregister()
    return {"us_per_call": round(el / reps * 1e6, 1), "cores": 1, "kind": "oracle",
            "calls": reps, "threads_limited": limit is not None}


def cpu_baseline(wl, seconds):
    """The oracle as it stands on layer 0 of the same workload, repeated until
    about ``seconds`` of host time; reported in the metric's unit (GB/s)."""
    import numpy as np
    import oracle
    c = wl.case
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [i.get("num_threads", 1) for i in threadpool_info()
                             if i.get("user_api") == "blas"])
    except Exception:
        pass
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.paged_attention(c.query, c.key_cache, c.value_cache, c.block_tables,
                               c.context_lens, c.scale, c.gqa_factor, "f16")
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 200:
            break
    return {"value": round(reps * wl.layer_bytes / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layer 0 of the 32K workload (128 MiB of K/V), {reps} oracle runs in "
                      f"{el:.1f} s; numpy float64 with {threads} BLAS thread(s), "
                      f"host has {os.cpu_count()} logical CPUs"}


# ----------------------------------------------------------------------------
# The other four workloads (timing only: K/V drawn on the GPU, tables, lengths
# and slots from the seeded generator).  Reported beside the headline.

OTHER = {
    # name: (seed, layers, split partition: None for the direct form, 0 for
    # the balanced split); the partition is the caller's choice for these
    # batches: the fastest of a sweep over direct, balanced, 256, 512, 1024
    # and 2048 on MI355X
    "tiny": (1, 32, None),
    "llama8b_batch": (2, 32, 0),
    "spec_verify": (4, 32, 0),
    "k8v4": (5, 32, 512),
    "long32k_window2048": (3, 32, 128),
}
WINDOW = {"long32k_window2048": 2048}       # sliding window of the windowed workloads


def k8v4_pools(P, torch, rnd, NB, Hkv, D, layers):
    """One K8/V4 pool per layer, every slot written by the quantize-on-write
    path from normal draws."""
    dev = torch.device("cuda:0")
    pools = []
    all_slots = torch.arange(NB * 16, dtype=torch.int64, device=dev)
    for _ in range(layers):
        pool = dict(k=torch.empty(NB, 16, Hkv, D, dtype=torch.int8, device=dev),
                    ks=torch.empty(NB, 16, Hkv, dtype=torch.float16, device=dev),
                    v=torch.empty(NB, 16, Hkv, D // 2, dtype=torch.uint8, device=dev),
                    vs=torch.empty(NB, 16, Hkv, D // 32, dtype=torch.float16, device=dev),
                    vz=torch.empty(NB, 16, Hkv, D // 32, dtype=torch.float16, device=dev))
        for c0 in range(0, NB * 16, 65536):
            sl = all_slots[c0:c0 + 65536]
            P.kv_cache_write_k8v4(rnd(len(sl), Hkv, D), rnd(len(sl), Hkv, D), pool["k"],
                                  pool["ks"], pool["v"], pool["vs"], pool["vz"], sl)
        pools.append(pool)
    return pools


def other_workload(name, P, W, torch, steps, warmup):
    seed, layers, part = OTHER[name]
    window = WINDOW.get(name, 0)
    lay, B, Q, Hq, Hkv, D, fmt = W.layout_of(name.split("_window")[0], seed)
    dev = torch.device("cuda:0")
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1000 + 7)
    NB, G = lay.num_blocks, Hq // Hkv
    scale = float(1.0 / D ** 0.5)
    T = len(lay.slot_mapping)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    cl = torch.from_numpy(lay.context_lens).to(dev)
    slots = torch.from_numpy(lay.slot_mapping).to(dev)
    mcl = int(lay.context_lens.max())
    rnd = lambda *sh: torch.randn(sh, generator=gen, device=dev, dtype=dt)  # noqa: E731
    q = [rnd(B, Q, Hq, D) for _ in range(layers)]
    nk = [rnd(T, Hkv, D) for _ in range(layers)]
    nv = [rnd(T, Hkv, D) for _ in range(layers)]
    out = [torch.empty(B, Q, Hq, D, dtype=dt, device=dev) for _ in range(layers)]
    ws = None
    split = part is not None
    if split:
        span = min(mcl, window + Q + 15) if window else mcl   # a window's grid spans the window
        ws = torch.zeros(P.splitkv_workspace_size(B, Q, Hq, D, span, part) // 4 + 4,
                         dtype=torch.float32, device=dev)
    sum_len = int(lay.context_lens.astype("int64").sum())
    if window:          # positions any row sees (q_len 1: the last `window` of each sequence)
        sum_len = int(sum(min(int(n), window + Q - 1) for n in lay.context_lens))
    if name == "k8v4":
        pools = k8v4_pools(P, torch, rnd, NB, Hkv, D, layers)
        per_tok_head = D + 2 + D // 2 + 4 * (D // 32)

        def step():             # append form: quantize the new rows and attend, one call
            for l in range(layers):
                p = pools[l]
                P.paged_attention_decode_splitkv_k8v4_append(
                    out[l], q[l], nk[l], nv[l], p["k"], p["ks"], p["v"], p["vs"], p["vz"], bt, cl,
                    scale, G, mcl, part, ws)

        def step_two_call():    # the same step as quantize-on-write, then decode
            for l in range(layers):
                p = pools[l]
                P.kv_cache_write_k8v4(nk[l], nv[l], p["k"], p["ks"], p["v"], p["vs"], p["vz"], slots)
                P.paged_attention_decode_splitkv_k8v4(out[l], q[l], p["k"], p["ks"], p["v"], p["vs"],
                                                      p["vz"], bt, cl, scale, G, mcl, part, ws)
    else:
        K = [rnd(NB, 16, Hkv, D) for _ in range(layers)]
        V = [rnd(NB, 16, Hkv, D) for _ in range(layers)]
        per_tok_head = 4 * D

        def step_two_call():    # the windowed step as write, then windowed split-KV decode
            for l in range(layers):
                P.kv_cache_write(nk[l], nv[l], K[l], V[l], slots)
                P.paged_attention_decode_splitkv_window(out[l], q[l], K[l], V[l], bt, cl, scale,
                                                        G, window, mcl, part, ws)

        def step():             # append form: store the new rows and attend, one call
            for l in range(layers):
                if window:
                    P.paged_attention_decode_splitkv_window_append(out[l], q[l], nk[l], nv[l],
                                                                   K[l], V[l], bt, cl, scale, G,
                                                                   window, mcl, part, ws)
                elif split:
                    P.paged_attention_decode_splitkv_append(out[l], q[l], nk[l], nv[l], K[l], V[l],
                                                            bt, cl, scale, G, mcl, part, ws)
                else:
                    P.paged_attention_decode_append(out[l], q[l], nk[l], nv[l], K[l], V[l], bt,
                                                    cl, scale, G)
    ms, med = time_steps(torch, graph_of(torch, step).replay, steps, warmup, median=True)
    extra = {"median_us_per_layer": round(med * 1e3 / layers, 3)}
    if name == "k8v4" or window:
        ms2 = time_steps(torch, graph_of(torch, step_two_call).replay, steps, warmup)
        extra["two_call_us_per_layer"] = round(ms2 * 1e3 / layers, 3)
    layer_bytes = sum_len * Hkv * per_tok_head
    us = ms * 1e3 / layers
    return {"us_per_layer": round(us, 3), **extra, "kv_bytes_per_layer": layer_bytes,
            "kv_stream_gbs": round(layer_bytes / (us * 1e-6) / 1e9, 2),
            "pct_of_hbm_peak": round(100 * layer_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "decode_rows_per_s": round(B * Q / (ms * 1e-3), 1),
            "layers": layers,
            "form": ("direct" if not split else "balanced split" if part == 0
                     else f"split-KV partition {part}")
            + (", append form (quantize-on-write in the decode launch)" if name == "k8v4"
               else f", append form, sliding window {window}" if window else ", append form")
            + ", HIP graph",
            "writes_per_layer": T, "kv_format": "k8v4" if name == "k8v4" else fmt}


def gather_workload(P, W, torch, steps, warmup, layers=8):
    """gather_kv_cache of every sequence of the Llama-3-8B-shaped batch
    (bf16, 32 sequences of 512..4096 tokens) into packed rows, per layer."""
    import numpy as np
    lay, B, Q, Hq, Hkv, D, fmt = W.layout_of("llama8b_batch", 2)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(2 * 1000 + 11)
    NB = lay.num_blocks
    lens = lay.context_lens.astype(np.int64)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    total = int(lens.sum())
    bt = torch.from_numpy(lay.block_tables).to(dev)
    K = [torch.randn(NB, 16, Hkv, D, generator=gen, device=dev, dtype=torch.bfloat16)
         for _ in range(layers)]
    V = [torch.randn(NB, 16, Hkv, D, generator=gen, device=dev, dtype=torch.bfloat16)
         for _ in range(layers)]
    ko = [torch.empty(total, Hkv, D, device=dev, dtype=torch.bfloat16) for _ in range(layers)]
    vo = [torch.empty_like(x) for x in ko]
    mx = int(lens.max())

    def step():
        for l in range(layers):
            P.gather_kv_cache(K[l], V[l], bt, cu, mx, ko[l], vo[l])
    ms = time_steps(torch, graph_of(torch, step).replay, steps, warmup)
    us = ms * 1e3 / layers
    read = total * Hkv * D * 2 * 2
    return {"us_per_layer": round(us, 3), "kv_bytes_read_per_layer": read,
            "kv_stream_gbs": round(read / (us * 1e-6) / 1e9, 2),
            "hbm_gbs_read_plus_write": round(2 * read / (us * 1e-6) / 1e9, 2),
            "pct_of_hbm_peak": round(100 * 2 * read / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "layers": layers, "form": "gather_kv_cache of all 32 sequences (K and V), HIP graph",
            "kv_format": "bf16"}


def cascade_workload(P, W, torch, steps, warmup, layers=8):
    """Shared system prompt: 8 groups of 4 sequences share a 4096-token
    prefix, each with its own 64..1024-token suffix (bf16, 32/8 heads, D 128).
    Cascade (prefix read once per group) against plain split-KV (read once
    per sequence); both partition 1024 (the cascade's prefix pass; its suffix
    pass is a balanced split), the fastest of 256..4096 for both."""
    import numpy as np
    lens, tables, NB, _, members, pre = W.shared_prefix_layout(W.rng_for(6), 8, 4, 4096, 64, 1024)
    B, Q, Hq, Hkv, D, part = 32, 1, 32, 8, 128, 1024
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(6 * 1000 + 13)
    rnd = lambda *sh: torch.randn(sh, generator=gen, device=dev, dtype=torch.bfloat16)  # noqa: E731
    K = [rnd(NB, 16, Hkv, D) for _ in range(layers)]
    V = [rnd(NB, 16, Hkv, D) for _ in range(layers)]
    q = [rnd(B, Q, Hq, D) for _ in range(layers)]
    out = [torch.empty(B, Q, Hq, D, device=dev, dtype=torch.bfloat16) for _ in range(layers)]
    bt = torch.from_numpy(tables).to(dev)
    cl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    mem = torch.from_numpy(members).to(dev)
    pb = torch.from_numpy(pre).to(dev)
    mcl, mpl = int(lens.max()), 4096
    ws_c = torch.zeros(P.cascade_workspace_size(B, Q, Hq, D, mcl, mpl, part) // 4, device=dev)
    ws_p = torch.zeros(P.splitkv_workspace_size(B, Q, Hq, D, mcl, part) // 4, device=dev)
    scale = float(1.0 / D ** 0.5)

    def cascade():
        for l in range(layers):
            P.paged_attention_decode_cascade(out[l], q[l], K[l], V[l], bt, cl, scale, 4, mem, pb,
                                             mpl, mcl, part, ws_c)

    def plain():
        for l in range(layers):
            P.paged_attention_decode_splitkv(out[l], q[l], K[l], V[l], bt, cl, scale, 4, mcl,
                                             part, ws_p)
    ms_c = time_steps(torch, graph_of(torch, cascade).replay, steps, warmup)
    ms_p = time_steps(torch, graph_of(torch, plain).replay, steps, warmup)
    logical = int(lens.sum()) * Hkv * D * 4                      # K+V bytes attended
    read = (8 * 4096 + int((lens - 4096).sum())) * Hkv * D * 4   # each shared block once
    us_c, us_p = ms_c * 1e3 / layers, ms_p * 1e3 / layers
    return {"us_per_layer": round(us_c, 3), "plain_splitkv_us_per_layer": round(us_p, 3),
            "speedup_vs_plain": round(us_p / us_c, 3),
            "kv_bytes_attended_per_layer": logical, "kv_bytes_read_per_layer": read,
            "kv_stream_gbs": round(read / (us_c * 1e-6) / 1e9, 2),
            "pct_of_hbm_peak": round(100 * read / (us_c * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "attended_gbs": round(logical / (us_c * 1e-6) / 1e9, 2),
            "layers": layers, "kv_format": "bf16",
            "form": "cascade (prefix pass at 1024-token partitions + balanced suffix pass + merge) "
                    "vs plain split-KV at 1024, HIP graph"}


def sparse_v_workload(P, W, torch, steps, warmup, layers=32, tau=1e-3, sharpen=8.0):
    """Approximate sparse-V decode at 32K: the long32k shape with queries drawn
    N(0, 8^2) instead of N(0, 1), a stand-in for sharply peaked attention rows
    (random unit-variance queries give nearly flat rows, where nothing can be
    skipped).  V rows weighing < tau of their row's running maximum are not
    read.  Against dense split-KV on the same inputs, partition 512."""
    import numpy as np
    lay, B, Q, Hq, Hkv, D, fmt = W.layout_of("long32k", 3)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(3 * 1000 + 17)
    NB, L, part = lay.num_blocks, int(lay.context_lens[0]), 512
    K = [torch.randn(NB, 16, Hkv, D, generator=gen, device=dev, dtype=torch.float16)
         for _ in range(layers)]
    V = [torch.randn(NB, 16, Hkv, D, generator=gen, device=dev, dtype=torch.float16)
         for _ in range(layers)]
    q = [torch.randn(B, Q, Hq, D, generator=gen, device=dev, dtype=torch.float16) * sharpen
         for _ in range(layers)]
    out = [torch.empty(B, Q, Hq, D, device=dev, dtype=torch.float16) for _ in range(layers)]
    bt = torch.from_numpy(lay.block_tables).to(dev)
    cl = torch.from_numpy(lay.context_lens).to(dev)
    ws = torch.zeros(P.splitkv_workspace_size(B, Q, Hq, D, L, part) // 4, device=dev)
    rows = torch.zeros(1, dtype=torch.int64, device=dev)
    scale = float(1.0 / D ** 0.5)

    def sparse():
        for l in range(layers):
            P.paged_attention_decode_splitkv_sparse_v(out[l], q[l], K[l], V[l], bt, cl, scale, 4,
                                                      tau, L, part, ws, v_rows_read=rows)

    def dense():
        for l in range(layers):
            P.paged_attention_decode_splitkv(out[l], q[l], K[l], V[l], bt, cl, scale, 4, L, part,
                                             ws)
    rows.zero_()
    sparse()
    torch.cuda.synchronize()
    frac = int(rows.item()) / (layers * L * Hkv)
    ms_s = time_steps(torch, graph_of(torch, sparse).replay, steps, warmup)
    ms_d = time_steps(torch, graph_of(torch, dense).replay, steps, warmup)
    us_s, us_d = ms_s * 1e3 / layers, ms_d * 1e3 / layers
    dense_bytes = L * Hkv * D * 4
    read = int(L * Hkv * D * 2 * (1 + frac))           # all of K, the V rows read
    return {"us_per_layer": round(us_s, 3), "dense_splitkv_us_per_layer": round(us_d, 3),
            "speedup_vs_dense": round(us_d / us_s, 3), "v_rows_read_fraction": round(frac, 4),
            "kv_bytes_read_per_layer": read, "dense_kv_bytes_per_layer": dense_bytes,
            "kv_stream_gbs": round(read / (us_s * 1e-6) / 1e9, 2),
            "layers": layers, "kv_format": "f16", "approximate": True,
            "form": f"sparse-V split-KV (threshold {tau:g}, queries x{sharpen:g}) vs dense "
                    "split-KV on the same inputs, partition 512, HIP graph"}


# ----------------------------------------------------------------------------
# Streaming ceiling of the 32K layer (--ceiling): how fast the same 32 x 128 MiB
# can be read at all, by read-only probes (libpagedkv_probe.so) timed exactly
# like the partition kernel (HIP events around 32 back-to-back launches, one
# per layer cache), next to the partition kernel itself.

# (label, heads per workgroup, waves, blocks per partition, depth, LDS bytes)
PAGED_SHAPES = [
    ("one head per workgroup, 8 waves x 4 blocks, 2 workgroups per CU (one-head kernel's shape)",
     1, 8, 32, 2, 60 * 1024),
    ("head pairs, 8 waves x 8 blocks, 1 workgroup per CU (the shipped kernel's shape)",
     2, 8, 32, 2, 82 * 1024),
    ("head pairs, depth 3", 2, 8, 32, 3, 82 * 1024),
    ("head pairs, depth 4", 2, 8, 32, 4, 82 * 1024),
    ("head pairs, 16 waves x 4 blocks, depth 3", 2, 16, 32, 3, 82 * 1024),
    ("head quads, 8 waves x 8 blocks, 256-token partitions", 4, 8, 16, 2, 82 * 1024),
    ("head quads, depth 4", 4, 8, 16, 4, 82 * 1024),
    ("all 8 heads, 8 waves x 8 blocks, 128-token partitions", 8, 8, 8, 2, 82 * 1024),
    ("all 8 heads, depth 4", 8, 8, 8, 4, 82 * 1024),
    ("all 8 heads, 16 waves x 4 blocks, depth 3", 8, 16, 8, 3, 82 * 1024),
    ("head pairs, depth 1 (each block's loads issued after the last is folded)", 2, 8, 32, 1,
     82 * 1024),
    ("all 8 heads, depth 1", 8, 8, 8, 1, 82 * 1024),
]
# (workgroups, waves, depth)
STREAM_SHAPES = [(256, 8, 4), (256, 16, 4), (512, 8, 2), (512, 8, 4), (1024, 8, 2), (1024, 4, 4),
                 (2048, 4, 2), (2048, 8, 1)]


def ceiling_mode(P, W, torch, args):
    import statistics
    from paged_kv_cache_181_amd import probe
    log("building the 32K workload")
    wl = Long32K(P, W, torch, args.layers, args.partition, args.seed)
    dev = torch.device("cuda:0")
    sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
    reps = max(args.steps, 5)

    def timed(launch):
        """median over `reps` of the per-launch time of 32 back-to-back launches"""
        for l in range(wl.layers):          # warm-up pass
            launch(l)
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for l in range(wl.layers):
                launch(l)
            e.record()
            torch.cuda.synchronize()
            per.append(s.elapsed_time(e) * 1e3 / wl.layers)
        return statistics.median(per), min(per), max(per)

    def row(us, lo, hi, **kw):
        return {**kw, "us_per_launch": round(us, 3), "us_min": round(lo, 3), "us_max": round(hi, 3),
                "tb_per_s": round(wl.layer_bytes / (us * 1e-6) / 1e12, 3),
                "pct_of_hbm_peak": round(100 * wl.layer_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}

    out = {"workload": "long32k layer caches (32 x 128 MiB of K and V, fp16)",
           "bytes_per_launch": wl.layer_bytes, "launches_per_timing": wl.layers,
           "timings": reps, "stream": [], "paged": []}
    for wgs, waves, depth in STREAM_SHAPES:
        log(f"stream read {wgs} x {waves} waves, depth {depth}")
        r = timed(lambda l: probe.stream_read(wl.K[l], wl.V[l], wgs, waves, depth, sink))
        out["stream"].append(row(*r, workgroups=wgs, waves=waves, depth=depth))
    for label, hp, waves, part, depth, lds in PAGED_SHAPES:
        log(f"paged read: {label}")
        r = timed(lambda l: probe.paged_read(wl.K[l], wl.V[l], wl.bt, hp, waves, part, depth, lds,
                                             sink))
        out["paged"].append(row(*r, shape=label, heads_per_workgroup=hp, waves=waves,
                                blocks_per_partition=part, depth=depth))
    c = wl.case
    log("partition kernel (append form, as the headline step)")
    if not hasattr(wl, "wss"):
        wl.wss = [torch.zeros_like(wl.ws) for _ in range(wl.layers)]
    r = timed(lambda l: P.paged_attention_decode_splitkv_append_partials(
        wl.q[l], wl.nk[l], wl.nv[l], wl.K[l], wl.V[l], wl.bt, wl.cl, c.scale, c.gqa_factor, wl.L,
        wl.partition, wl.wss[l]))
    out["partition_kernel"] = row(*r, kernel="attn_partition_kernel<F16,F16,128,4> head-pair form")
    r = timed(lambda l: P.paged_attention_decode_splitkv_merge(wl.out[l], wl.L, wl.partition,
                                                                wl.wss[l]))
    out["merge_kernel_us_per_launch"] = round(r[0], 3)
    best_stream = min(out["stream"], key=lambda x: x["us_per_launch"])
    best_paged = min(out["paged"], key=lambda x: x["us_per_launch"])
    shipped = out["paged"][1]
    k_us = out["partition_kernel"]["us_per_launch"]
    out["summary"] = {
        "best_stream_us": best_stream["us_per_launch"],
        "best_paged_us": best_paged["us_per_launch"], "best_paged_shape": best_paged["shape"],
        "shipped_shape_read_us": shipped["us_per_launch"],
        "partition_kernel_us": k_us,
        "kernel_frac_of_best_stream": round(best_stream["us_per_launch"] / k_us, 4),
        "kernel_frac_of_shipped_shape_read": round(shipped["us_per_launch"] / k_us, 4),
        "us_per_layer_at_70pct_of_peak": round(wl.layer_bytes / (0.7 * HBM_PEAK_GBS * 1e9) * 1e6, 3),
    }
    print(json.dumps({"ceiling": out}), flush=True)


def ceiling_k8v4_mode(P, W, torch, args):
    """Read ceiling of the K8/V4 batch (16 x 8192 tokens, 32 layers): the
    probe library reads the same 32 layer pools with the head-group form's
    lane addressing (one wave per KV head over a 512-token partition, the six
    loads per block of the attention kernel), timed like the partition kernel
    beside it (median of 32 back-to-back launches)."""
    import statistics
    from paged_kv_cache_181_amd import probe
    seed, layers, part = OTHER["k8v4"]
    lay, B, Q, Hq, Hkv, D, fmt = W.layout_of("k8v4", seed)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1000 + 7)
    rnd = lambda *sh: torch.randn(sh, generator=gen, device=dev, dtype=torch.float16)  # noqa: E731
    NB, G = lay.num_blocks, Hq // Hkv
    log("building the K8/V4 pools")
    pools = k8v4_pools(P, torch, rnd, NB, Hkv, D, layers)
    lens = lay.context_lens.astype("int64")
    nblk = (lens + 15) // 16
    flat = torch.from_numpy(__import__("numpy").concatenate(
        [lay.block_tables[b, :nblk[b]] for b in range(B)]).astype("int32")).to(dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    cl = torch.from_numpy(lay.context_lens).to(dev)
    mcl = int(lens.max())
    q = [rnd(B, Q, Hq, D) for _ in range(layers)]
    nbytes = P.splitkv_workspace_size(B, Q, Hq, D, mcl, part)
    wss = [torch.zeros(nbytes // 4 + 4, dtype=torch.float32, device=dev) for _ in range(layers)]
    out = [torch.empty(B, Q, Hq, D, dtype=torch.float16, device=dev) for _ in range(layers)]
    sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)
    layer_bytes = int(lens.sum()) * Hkv * (D + 2 + D // 2 + 4 * (D // 32))
    reps = max(args.steps, 5)
    scale = float(1.0 / D ** 0.5)

    def timed(launch):
        for l in range(layers):
            launch(l)
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for l in range(layers):
                launch(l)
            e.record()
            torch.cuda.synchronize()
            per.append(s.elapsed_time(e) * 1e3 / layers)
        return statistics.median(per), min(per), max(per)

    def row(us, lo, hi, **kw):
        return {**kw, "us_per_launch": round(us, 3), "us_min": round(lo, 3), "us_max": round(hi, 3),
                "tb_per_s": round(layer_bytes / (us * 1e-6) / 1e12, 3),
                "pct_of_hbm_peak": round(100 * layer_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}

    res = {"workload": f"k8v4 layer pools ({B} x {mcl} tokens, {Hkv} KV heads, D {D}, "
                       f"{layers} layers)", "bytes_per_launch": layer_bytes,
           "launches_per_timing": layers, "timings": reps, "probe": []}
    pblk = part // 16
    for lds in (0, 96 * 1024):
        for depth in (1, 2, 3, 4):
            log(f"K8/V4 read probe: depth {depth}, LDS {lds}")
            r = timed(lambda l: probe.k8v4_read(pools[l]["k"], pools[l]["ks"], pools[l]["v"],
                                                pools[l]["vs"], pools[l]["vz"], flat, pblk, depth,
                                                lds, sink))
            res["probe"].append(row(*r, depth=depth, lds_bytes=lds,
                                    workgroups=flat.numel() // pblk))
    log("K8/V4 partition kernel (head groups, partition 512)")
    r = timed(lambda l: P.paged_attention_decode_splitkv_k8v4_partials(
        q[l], pools[l]["k"], pools[l]["ks"], pools[l]["v"], pools[l]["vs"], pools[l]["vz"], bt, cl,
        scale, G, mcl, part, wss[l]))
    res["partition_kernel"] = row(*r, kernel="attn_partition_kernel<K8V4,F16,128,4> head groups",
                                  partition_size=part)
    r = timed(lambda l: P.paged_attention_decode_splitkv_merge(out[l], mcl, part, wss[l]))
    res["merge_kernel_us_per_launch"] = round(r[0], 3)
    best = min(res["probe"], key=lambda x: x["us_per_launch"])
    same = [x for x in res["probe"] if x["depth"] == 2 and x["lds_bytes"] == 96 * 1024][0]
    k_us = res["partition_kernel"]["us_per_launch"]
    res["summary"] = {"best_probe_us": best["us_per_launch"], "best_probe_depth": best["depth"],
                      "best_probe_lds_bytes": best["lds_bytes"],
                      "kernel_shape_probe_us": same["us_per_launch"],
                      "partition_kernel_us": k_us,
                      "kernel_frac_of_best_probe": round(best["us_per_launch"] / k_us, 4),
                      "kernel_frac_of_its_shape": round(same["us_per_launch"] / k_us, 4)}
    print(json.dumps({"ceiling_k8v4": res}), flush=True)


def copy_calibration(torch):
    """A plain device copy of known size: 1 GiB read + 1 GiB written per launch.
    rocprofv3's FETCH_SIZE / WRITE_SIZE for these launches give the scale
    from counter units to bytes for the same counters on our kernels."""
    n = 1 << 30
    src = torch.empty(n // 2, dtype=torch.float16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import paged_kv_cache_181_amd as P
    from paged_kv_cache_181_amd import workloads as W
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.ceiling_k8v4:
        ceiling_k8v4_mode(P, W, torch, args)
        return
    if args.ceiling:
        ceiling_mode(P, W, torch, args)
        return
    if args.only:
        runners = {n: (lambda n=n: other_workload(n, P, W, torch, args.steps, args.warmup))
                   for n in OTHER}
        runners["cascade_system_prompt"] = lambda: cascade_workload(P, W, torch, args.steps,
                                                                    args.warmup)
        runners["sparse_v_long32k_peaked"] = lambda: sparse_v_workload(P, W, torch, args.steps,
                                                                       args.warmup)
        runners["gather_llama8b_batch"] = lambda: gather_workload(P, W, torch, args.steps,
                                                                  args.warmup)
        if args.only not in runners:
            print(json.dumps({"error": f"unknown workload {args.only}; one of {sorted(runners)}"}))
            sys.exit(2)
        if args.only_partition is not None and args.only in OTHER:
            seed, layers, _ = OTHER[args.only]
            part = None if args.only_partition == "direct" else int(args.only_partition)
            OTHER[args.only] = (seed, layers, part)
        log(f"timing {args.only}")
        print(json.dumps({"workload": args.only, "library": os.path.basename(P.lib._name),
                          **runners[args.only]()}), flush=True)
        return

    log("building the 32K workload")
    wl = Long32K(P, W, torch, args.layers, args.partition, args.seed)
    log("timing steps")
    eager_ms = time_steps(torch, wl.step, args.steps, args.warmup)
    graph = graph_of(torch, wl.step)
    ms, med_ms = time_steps(torch, graph.replay, args.steps, args.warmup, median=True)
    two_call_ms = time_steps(torch, graph_of(torch, wl.step_two_call).replay, args.steps,
                             args.warmup)
    write_ms = time_steps(torch, graph_of(torch, wl.step_write_only).replay, args.steps,
                          args.warmup)
    gbs = wl.step_bytes / (ms * 1e-3) / 1e9
    log(f"{ms:.3f} ms/step (median {med_ms:.3f}; {eager_ms:.3f} eager, {two_call_ms:.3f} two-call, "
        f"{write_ms:.3f} the writes alone), {gbs:.1f} GB/s")
    kern_ms, launches = kernel_average_ms(torch, wl, args.steps)
    achieved = wl.layer_bytes / (kern_ms * 1e-3) / 1e9
    log(f"partition kernel {kern_ms * 1e3:.2f} us avg over {launches} launches, {achieved:.1f} GB/s")

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "library": os.path.basename(P.lib._name),
        "config": {
            "workload": "long32k: single-user split-KV decode, batch 1, q_len 1, 32 query / 8 KV "
                        "heads, head_dim 128, fp16 K/V, context 32768 (2048 blocks of 16, "
                        "permuted pool), 32 layers, partition 512; per layer the new token's "
                        "store + partition kernel + LSE merge kernel (append form), the "
                        "step replayed as one HIP graph",
            "batch": 1, "context": wl.L, "layers": args.layers, "partition_size": args.partition,
            "kv_bytes_per_step": wl.step_bytes,
        },
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_layer": round(ms * 1e3 / args.layers, 3),
        "median_ms_per_step": round(med_ms, 4),
        "median_us_per_layer": round(med_ms * 1e3 / args.layers, 3),
        "median_pct_of_hbm_peak": round(100 * wl.step_bytes / (med_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        2),
        "eager_ms_per_step": round(eager_ms, 4),
        "two_call_ms_per_step": round(two_call_ms, 4),
        "kv_cache_write_us_per_layer": round(write_ms * 1e3 / args.layers, 3),
        "decode_tokens_per_s": round(1e3 / ms, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "attn_partition_kernel<F16,F16,128,4> (head-pair form)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "avg_launch_us": round(kern_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": wl.layer_bytes,
        },
    }
    if not args.no_extra:
        log("timing long32k at 128-token partitions")
        finer = long32k_other_partition(wl, P, torch, 128, args.steps, args.warmup)
        del wl.K, wl.V
        torch.cuda.empty_cache()
        result["other_workloads"] = {"long32k_partition128": finer}
        for name in ("tiny", "llama8b_batch", "spec_verify", "k8v4", "long32k_window2048"):
            log(f"timing {name}")
            result["other_workloads"][name] = other_workload(name, P, W, torch, args.steps,
                                                             args.warmup)
            torch.cuda.empty_cache()
        log("timing cascade")
        result["other_workloads"]["cascade_system_prompt"] = cascade_workload(
            P, W, torch, args.steps, args.warmup)
        torch.cuda.empty_cache()
        log("timing sparse-V")
        result["other_workloads"]["sparse_v_long32k_peaked"] = sparse_v_workload(
            P, W, torch, args.steps, args.warmup)
        torch.cuda.empty_cache()
        log("timing gather_kv_cache")
        result["other_workloads"]["gather_llama8b_batch"] = gather_workload(P, W, torch,
                                                                            args.steps, args.warmup)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        if "other_workloads" in result:
            result["other_workloads"]["tiny"]["cpu_oracle_one_thread"] = \
                cpu_baseline_tiny_one_thread(W)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

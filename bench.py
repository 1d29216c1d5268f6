"""Benchmark of the int4 KV-cache path on one MI355X.

One step is the whole hot path over one batch of the OPT-175B layer shape
(b=144, a=96, d=128, h=12288, prompt s=512, n=32 generated tokens, 96 layers
whose int4 caches stay resident in HBM):

  * prefill: kv_quantize_prefill of every layer's prompt K and V;
  * decode:  for j = 1..32, for every layer: the new token's K/V quantised into
             slot s+j-1 and attention over s+j tokens -- kv_append_quant then
             decode_attention_q4 (or, with --fused, one kv_append_attend_q4 launch).

value = algorithmic HBM bytes of the step / step time (GB/s).  Algorithmic
bytes: quantise 2 B in + 0.5 B codes + 0.125 B metadata per element; decode
attention 160 B per (batch row, head, token) (64 B K codes + 64 B V codes +
32 B fp32 min/scale) plus q and out; append as quantise on one token.  The
decode attention kernel is timed live with HIP events on the stream it runs
on; its achieved bandwidth against the 8 TB/s HBM peak is the `roofline`
entry.  The sparse top-10% variant is timed on its own workload (b=32, a=96,
context 2048) and the split-context reduce path on one long sequence (b=1,
a=96, context 65536); both are reported beside it.  `cpu_baseline` times the CPU oracle
on a bounded sample of the same job.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention int4-KV HBM GB/s (% of peak) + layer-tokens/s, OPT-175B shape"
HBM_PEAK_GBS = 8000.0
PROFILE_PMC = os.path.join(ROOT, "profiles", "k_decode_opt175b_pmc.md")
KERNEL_SRC = (os.path.join(ROOT, "quantized_kv_cache_prefill_amd", "csrc", "kvq4_kernels.hip"),
              os.path.join(ROOT, "quantized_kv_cache_prefill_amd", "csrc", "kvq4_device.h"))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic bytes
def bytes_quantize(rows: int, d: int, mb: int = 4) -> int:
    """fp16 in (2 B/elem) + codes (0.5 B/elem) + min and scale (mb bytes each) per 64 elements."""
    return rows * d * 2 + rows * d // 2 + rows * (d // 64) * 2 * mb


def bytes_decode(pairs: int, T: int, d: int, mb: int = 4) -> int:
    """K and V codes + min/scale (mb bytes each) for T tokens, plus q and out (fp16)."""
    per_token = d + 4 * mb * (d // 64)         # 2 * d/2 code bytes + 4 metadata values per group
    return pairs * (T * per_token + 2 * d * 2)


def bytes_topk(pairs: int, T: int, k: int, d: int, mb: int = 4) -> int:
    """All K (codes + metadata), the k kept V rows, q, out and the kept indices."""
    half = d // 2 + 2 * mb * (d // 64)
    return pairs * ((T + k) * half + 2 * d * 2 + 4 * k)


META_BYTES = {"f32": 4, "f16": 2}


def kernel_source_hash() -> str:
    """Hash of the decode kernel's source files (the kernels and their shared device header)."""
    hsh = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()[:16]


def stored_traffic():
    """Measured HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None when absent or taken on a different kernel source."""
    try:
        with open(PROFILE_PMC) as f:
            for line in f:
                if line.startswith("<!-- traffic "):
                    rec = json.loads(line[len("<!-- traffic "):].rsplit("-->", 1)[0])
                    if rec.get("kernel_source_sha256_16") == kernel_source_hash():
                        return rec
    except OSError:
        pass
    return None


# ------------------------------------------------------------------- GPU job
class Job:
    """One layer stack of workload `w`: L int4 caches resident in HBM, the prompt of every
    layer quantised, then n decode steps, each appending the new token's K/V and attending
    over s+j tokens in every layer (append + decode_attention_q4, or the fused launch)."""

    def __init__(self, w, L, n, meta="f32", fused=False):
        import torch

        import quantized_kv_cache_prefill_amd as kvq
        import workloads as W

        self.torch, self.kvq, self.W = torch, kvq, W
        self.w, self.L, self.n, self.meta, self.fused = w, L, n, meta, fused
        mb = META_BYTES[meta]
        dev = self.dev = "cuda"
        torch.cuda.set_device(0)
        log(f"[bench] {w.name}: allocating {L} int4 caches of b={w.b} a={w.a} d={w.d} S={w.S}, {meta} min/scale")
        self.caches = [kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device=dev, meta=meta) for _ in range(L)]
        # prompt K/V: a few distinct seeded buffers used in rotation (an OPT-175B layer's prompt is 3.6 GB)
        self.n_prompt = min(4, L)
        self.prompts = [W.prefill_kv(w, l, dev) for l in range(self.n_prompt)]
        log(f"[bench] {w.name}: generating decode inputs for {L} layers x {n} steps")
        self.dec = [[W.decode_inputs(w, l, j, dev) for j in range(1, n + 1)] for l in range(L)]
        self.out = torch.empty((L, w.b, 1, w.a, w.d), dtype=torch.float16, device=dev)
        self.stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        pairs = w.b * w.a
        self.b_prefill = 2 * L * bytes_quantize(w.b * w.a * w.s, w.d, mb)
        self.b_append = 0 if fused else 2 * L * n * bytes_quantize(pairs, w.d, mb)
        self.b_decode_per_launch = [bytes_decode(pairs, w.s + j, w.d, mb) for j in range(1, n + 1)]
        if fused:  # the timed launch also quantises and writes the new K/V rows
            self.b_decode_per_launch = [x + 2 * bytes_quantize(pairs, w.d, mb) for x in self.b_decode_per_launch]
        self.b_decode = L * sum(self.b_decode_per_launch)
        self.b_step = self.b_prefill + self.b_append + self.b_decode

    def step(self, events=None):
        kvq, w = self.kvq, self.w
        for l in range(self.L):
            k, v = self.prompts[l % self.n_prompt]
            kvq.kv_quantize_prefill(self.caches[l], k, v)
        for j in range(1, self.n + 1):
            for l in range(self.L):
                q, kn, vn = self.dec[l][j - 1]
                if not self.fused:
                    kvq.kv_append_quant(self.caches[l], kn, vn, w.s + j - 1)
                if events is not None:
                    e0, e1 = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
                    e0.record(self.stream)
                if self.fused:
                    kvq.kv_append_attend_q4(self.caches[l], q, kn, vn, w.s + j - 1, out=self.out[l])
                else:
                    kvq.decode_attention_q4(self.caches[l], q, w.s + j, out=self.out[l])
                if events is not None:
                    e1.record(self.stream)
                    events.append((e0, e1, self.b_decode_per_launch[j - 1]))

    def run(self, steps, warmup):
        """warmup untimed steps, then `steps` timed ones; returns (wall ms per step, decode events)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        events = []
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(events)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps, events

    def summary(self, ms_step, events, steps):
        w = self.w
        dec_ms = [a.elapsed_time(b) for a, b, _ in events]
        dec_bytes = [nb for _, _, nb in events]
        avg_ms = sum(dec_ms) / len(dec_ms)
        achieved = (sum(dec_bytes) / len(dec_bytes)) / avg_ms / 1e6
        srt = sorted(dec_ms)
        return {"ms_per_step": round(ms_step, 2), "step_gbs": round(self.b_step / (ms_step / 1e3) / 1e9, 1),
                "decode_attention": {
                    "gbs": round(achieved, 1), "pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
                    "layer_tokens_per_s": round(w.b / (avg_ms / 1e3), 1),
                    "stack_tokens_per_s": round(w.b * self.n / (sum(dec_ms) / steps / 1e3), 1),
                    "launch_ms": {"min": round(srt[0], 5), "median": round(srt[len(srt) // 2], 5),
                                  "p90": round(srt[int(0.9 * (len(srt) - 1))], 5), "max": round(srt[-1], 5),
                                  "mean": round(avg_ms, 5), "launches": len(srt)}},
                "avg_launch_ms": avg_ms, "achieved_gbs": achieved,
                "algorithmic_bytes_per_launch": int(sum(dec_bytes) / len(dec_bytes))}


def time_stack(w, steps=2, warmup=1):
    """The whole stack job of workload `w` (all its layers resident), as the headline job."""
    import torch
    job = Job(w, w.layers, w.n)
    ms, ev = job.run(steps, warmup)
    res = job.summary(ms, ev, steps)
    res.pop("avg_launch_ms"), res.pop("achieved_gbs")
    res["workload"] = (f"{w.name} layer stack: b={w.b} a={w.a} d={w.d} h={w.h}, prompt {w.s}, {w.n} decode steps, "
                       f"{w.layers} int4 caches resident ({job.L * job.caches[0].nbytes() / 1e9:.1f} GB)")
    res["steps"], res["warmup"] = steps, warmup
    del job
    torch.cuda.empty_cache()
    return res


def time_cache_warm_layer(w, reps=60):
    """One layer of workload `w` at its final context, attended `reps` times in a row: the
    layer's cache (89 MB for OPT-6.7B) stays in the 256 MB Infinity Cache, so this is a
    cache-warm rate, not an HBM one."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    T = w.S
    cache = kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device="cuda")
    k, v = W.prefill_kv(w, 0, "cuda", s_len=T)
    kvq.kv_quantize_prefill(cache, k, v)
    del k, v
    q = W.decode_inputs(w, 0, 1, "cuda")[0]
    out = torch.empty_like(q)
    st = torch.cuda.current_stream()
    ev = []
    for _ in range(reps + 5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        kvq.decode_attention_q4(cache, q, T, out=out)
        e1.record(st)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev[5:])
    med = ms[len(ms) // 2]
    nb = bytes_decode(w.b * w.a, T, w.d)
    return {"workload": f"{w.name} single layer: b={w.b} a={w.a} d={w.d} context {T}, the same cache {reps} times "
                        f"(cache-warm: it fits the Infinity Cache)",
            "ms_per_call_median": round(med, 5), "algorithmic_bytes": nb, "gbs": round(nb / med / 1e6, 1),
            "layer_tokens_per_s": round(w.b / (med / 1e3), 1)}


def time_tiny_latency(reps=200):
    """Latency of one decode layer-step on the tiny configuration (b=2, a=2, d=64, prompt 16,
    context 17..20): append + attention (two launches), attention alone, and the fused launch;
    then the two-launch and the fused step as HIP graph replays; medians of HIP events around
    each, launch overhead included."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    w = W.TINY
    cache = kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device="cuda")
    k, v = W.prefill_kv(w, 0, "cuda")
    kvq.kv_quantize_prefill(cache, k, v)
    inputs = [W.decode_inputs(w, 0, j, "cuda") for j in range(1, w.n + 1)]
    out = torch.empty_like(inputs[0][0])
    st = torch.cuda.current_stream()
    res = {}
    for label in ("append_then_attend", "attend_only", "fused"):
        ev = []
        for r in range(reps + 10):
            j = r % w.n + 1
            q, kn, vn = inputs[j - 1]
            pos = w.s + j - 1
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            if label == "fused":
                kvq.kv_append_attend_q4(cache, q, kn, vn, pos, out=out)
            else:
                if label == "append_then_attend":
                    kvq.kv_append_quant(cache, kn, vn, pos)
                kvq.decode_attention_q4(cache, q, pos + 1, out=out)
            e1.record(st)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev[10:])
        res[label] = {"us_median": round(us[len(us) // 2], 2), "us_min": round(us[0], 2)}
    # The steps captured as HIP graphs and replayed (the library enqueues kernels only, so
    # every call is capturable): one graph per step, and one graph holding all n steps of the
    # layer, reported per step.
    for label in ("graph_append_then_attend", "graph_fused"):
        def one_step(j):
            q, kn, vn = inputs[j - 1]
            pos = w.s + j - 1
            if label == "graph_fused":
                kvq.kv_append_attend_q4(cache, q, kn, vn, pos, out=out)
            else:
                kvq.kv_append_quant(cache, kn, vn, pos)
                kvq.decode_attention_q4(cache, q, pos + 1, out=out)
        graphs = []
        for j in range(1, w.n + 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_step(j)
            graphs.append(g)
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for j in range(1, w.n + 1):
                one_step(j)
        for key, run, per in ((label, lambda r: graphs[r % w.n].replay(), 1),
                              (label + f"_{w.n}_steps_per_graph", lambda r: g_all.replay(), w.n)):
            ev = []
            for r in range(reps + 10):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                run(r)
                e1.record(st)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            us = sorted(a.elapsed_time(b) * 1e3 / per for a, b in ev[10:])
            res[key] = {"us_median": round(us[len(us) // 2], 2), "us_min": round(us[0], 2)}
        del graphs, g_all
    res["workload"] = f"tiny: b={w.b} a={w.a} d={w.d}, prompt {w.s}, contexts {w.s + 1}..{w.S}, one layer"
    res["bytes_per_step"] = bytes_decode(w.b * w.a, w.S, w.d)
    return res


def time_topk(reps: int = 12, copies: int = 4):
    """Sparse top-10% decode attention on b=32, a=96, context 2048 (k = 205).  The layer is
    held in `copies` separate caches (1 GB each) used in rotation, so the 256 MB Infinity
    Cache cannot serve a repeat."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    w = W.SPARSE
    T = w.s + w.n
    k_top = w.k_top(T)
    caches = [kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device="cuda") for _ in range(copies)]
    k, v = W.prefill_kv(w, 0, "cuda")
    q, kn, vn = W.decode_inputs(w, 0, 1, "cuda")
    for c in caches:
        kvq.kv_quantize_prefill(c, k, v)
        kvq.kv_append_quant(c, kn, vn, w.s)
    del k, v
    out = torch.empty_like(q)
    sel = torch.empty((w.b, w.a, k_top), dtype=torch.int32, device="cuda")
    # up to KVQ_TOPK_FUSED_MAX_CTX tokens the call is one launch that keeps the scores on chip
    need = kvq.kvq_workspace_bytes(caches[0], T, 0, k_top)
    ws = torch.empty(need // 4, dtype=torch.float32, device="cuda") if need else None
    for r in range(4 * copies):           # untimed: the clock settles after the cache set-up
        kvq.decode_attention_q4_topk(caches[r % copies], q, T, k_top, out=out, sel_idx=sel, ws=ws)
    times = []
    st = torch.cuda.current_stream()
    for r in range((reps + 1) * copies):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        kvq.decode_attention_q4_topk(caches[r % copies], q, T, k_top, out=out, sel_idx=sel, ws=ws)
        e1.record(st)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in times[copies:]]
    ms.sort()
    med = ms[len(ms) // 2]
    nbytes = bytes_topk(w.b * w.a, T, k_top, w.d)
    dense_bytes = bytes_decode(w.b * w.a, T, w.d)
    return {"workload": f"sparse top-10%: b={w.b} a={w.a} d={w.d} context {T}, k={k_top}",
            "ms_per_call_median": round(med, 4), "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / med / 1e6, 1), "frac_of_hbm_peak": round(nbytes / med / 1e6 / HBM_PEAK_GBS, 4),
            "dense_equivalent_bytes": dense_bytes,
            "launches": 1 if T <= kvq.KVQ_TOPK_FUSED_MAX_CTX else 2}


def time_split_context(T: int = 65536, copies: int = 3, reps: int = 5):
    """The split-context path (decode_attention_q4 with its automatic split count and the
    log-sum-exp reduce pass) on one long sequence: b=1, a=96, d=128, context T.  With only
    96 (batch row, head) pairs the heuristic splits every context across workgroups; the
    same call with num_splits=1 is timed beside it."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    b, a, d = 1, 96, 128
    caches = [kvq.QuantKVCache(b, a, a * d, T, 0, device="cuda") for _ in range(copies)]
    k = W.random_fp16((b, T, a, d), 777, "cuda")
    v = W.random_fp16((b, T, a, d), 778, "cuda")
    for c in caches:
        kvq.kv_quantize_prefill(c, k, v)
    del k, v
    q = W.random_fp16((b, 1, a, d), 779, "cuda")
    out = torch.empty_like(q)
    st = torch.cuda.current_stream()
    res = {}
    for label, ns in (("auto", 0), ("one_split", 1)):
        need = kvq.kvq_workspace_bytes(caches[0], T, ns)
        ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda")
        times = []
        for r in range((reps + 1) * copies):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            kvq.decode_attention_q4(caches[r % copies], q, T, out=out, num_splits=ns, ws=ws)
            e1.record(st)
            times.append((e0, e1))
        torch.cuda.synchronize()
        ms = sorted(x.elapsed_time(y) for x, y in times[copies:])
        med = ms[len(ms) // 2]
        res[label] = {"ms_per_call_median": round(med, 4), "workspace_bytes": need,
                      "gbs": round(bytes_decode(b * a, T, d) / med / 1e6, 1)}
    res["workload"] = f"one long sequence: b={b} a={a} d={d} context {T}"
    res["algorithmic_bytes"] = bytes_decode(b * a, T, d)
    return res


def time_meta_f16(copies: int = 6, reps: int = 8):
    """Dense decode attention on the OPT-175B layer (b=144, a=96, d=128, context 544) with
    binary16 min/scale planes (144 B per (batch row, head, token)) beside the same call on
    binary32 planes (160 B).  `copies` caches of each kind are used in rotation so the
    Infinity Cache cannot serve a repeat, and the two kinds' launches alternate so that
    both see the same conditions; medians of per-launch HIP events."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    w = W.OPT_175B
    T = w.S
    k, v = W.prefill_kv(w, 0, "cuda", s_len=T)
    q, _, _ = W.decode_inputs(w, 0, 1, "cuda")
    out = torch.empty_like(q)
    st = torch.cuda.current_stream()
    metas = ("f32", "f16")
    caches = {m: [kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device="cuda", meta=m) for _ in range(copies)]
              for m in metas}
    for m in metas:
        for c in caches[m]:
            kvq.kv_quantize_prefill(c, k, v)
    del k, v
    times = {m: [] for m in metas}
    for r in range((reps + 1) * copies):
        for m in metas:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            kvq.decode_attention_q4(caches[m][r % copies], q, T, out=out)
            e1.record(st)
            times[m].append((e0, e1))
    torch.cuda.synchronize()
    res = {"workload": f"OPT-175B layer: b={w.b} a={w.a} d={w.d} context {T}, {copies} caches per kind in rotation, "
                       f"launches of the two kinds alternating"}
    for m in metas:
        ms = sorted(x.elapsed_time(y) for x, y in times[m][copies:])
        med = ms[len(ms) // 2]
        nb = bytes_decode(w.b * w.a, T, w.d, META_BYTES[m])
        res[m] = {"ms_per_call_median": round(med, 4), "algorithmic_bytes": nb,
                  "gbs": round(nb / med / 1e6, 1), "frac_of_hbm_peak": round(nb / med / 1e6 / HBM_PEAK_GBS, 4),
                  "layer_tokens_per_s": round(w.b / (med / 1e3), 1)}
    del caches
    res["f16_speedup"] = round(res["f32"]["ms_per_call_median"] / res["f16"]["ms_per_call_median"], 4)
    return res


MFMA_F16_PEAK_TFLOPS = 2500.0


def time_projections(copies: int = 3, reps: int = 8):
    """The decode projections of one OPT-175B layer with int4 weights (gemm_w4a16): the
    fused Q/K/V projection (N = 3h = 36864, K = h = 12288) and the output projection
    (N = K = 12288), M = 144 tokens (the effective batch).  Synthetic weights N(0, 0.02^2),
    activations N(0, 1); `copies` weight sets in rotation so the Infinity Cache cannot
    serve a repeat; medians of per-launch HIP events, timed two ways:
      * back to back: one projection launched repeatedly (matrix-core load without a
        break, the clock settles at the chip's sustained power limit);
      * in decode-layer order: attention over the layer's int4 cache (b=144, a=96,
        context 544) -> QKV projection -> output projection, repeated, as one decode
        step runs them."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    M, h = 144, 12288
    st = torch.cuda.current_stream()
    res = {"workload": f"OPT-175B decode projections, M={M} tokens, int4 weights (group 64, binary16 min/scale), "
                       f"{copies} weight sets in rotation"}

    def rec(lst, fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        lst.append((e0, e1))

    def med_of(lst):
        ms = sorted(a.elapsed_time(b) for a, b in lst)
        return ms[len(ms) // 2]

    x = W.random_fp16((M, h), 9100, "cuda")
    sets, ys, wss = {}, {}, {}
    for label, N in (("qkv", 3 * h), ("out", h)):
        sets[label] = []
        for c in range(copies):
            w = W.random_fp16((N, h), 9000 + 10 * c + (N == h), "cuda", 0.02)
            sets[label].append(kvq.kvq_w4_quantize(w))
            del w
        ys[label] = torch.empty((M, N), dtype=torch.float16, device="cuda")
        need = kvq.kvq_gemm_w4_workspace_bytes(M, N, h)
        wss[label] = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda")
        times = []
        for r in range((reps + 1) * copies):
            rec(times, lambda: kvq.gemm_w4a16(x, *sets[label][r % copies], y=ys[label], ws=wss[label]))
        torch.cuda.synchronize()
        med = med_of(times[copies:])
        flops = 2 * M * N * h
        wbytes = N * h // 2 + 2 * 2 * N * (h // 64)
        res[label] = {"N": N, "K": h, "ms_per_call_median": round(med, 4),
                      "tflops": round(flops / med / 1e9, 1),
                      "frac_of_mfma_f16_peak": round(flops / med / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                      "weight_gbs": round(wbytes / med / 1e6, 1), "workspace_bytes": need,
                      "form": "stream" if need == kvq.kvq_gemm_w4_workspace_bytes(M, N, h, kvq.KVQ_GEMM_STREAM)
                      else "split"}
    # decode-layer order
    wl = W.OPT_175B
    cache = kvq.QuantKVCache(wl.b, wl.a, wl.h, wl.s, wl.n, device="cuda", meta="f32")
    k, v = W.prefill_kv(wl, 0, "cuda")
    kvq.kv_quantize_prefill(cache, k, v)
    del k, v
    q, kn, vn = W.decode_inputs(wl, 0, 1, "cuda")
    for j in range(wl.n):
        kvq.kv_append_quant(cache, kn, vn, wl.s + j)
    out = torch.empty((wl.b, 1, wl.a, wl.d), dtype=torch.float16, device="cuda")
    ev = {"attention": [], "qkv": [], "out": []}
    for r in range((reps + 1) * copies):
        rec(ev["attention"], lambda: kvq.decode_attention_q4(cache, q, wl.s + wl.n, out=out))
        for label in ("qkv", "out"):
            rec(ev[label], lambda: kvq.gemm_w4a16(x, *sets[label][r % copies], y=ys[label], ws=wss[label]))
    torch.cuda.synchronize()
    res["decode_layer_order"] = {lab: {"ms_per_call_median": round(med_of(lst[copies:]), 4)} for lab, lst in ev.items()}
    for label, N in (("qkv", 3 * h), ("out", h)):
        med = res["decode_layer_order"][label]["ms_per_call_median"]
        res["decode_layer_order"][label]["frac_of_mfma_f16_peak"] = round(
            2 * M * N * h / med / 1e9 / MFMA_F16_PEAK_TFLOPS, 4)
    del sets, cache
    torch.cuda.empty_cache()
    return res


def time_projection_sustained(calls: int = 6000):
    """The OPT-175B QKV projection (M = 144, N = 36864, K = 12288) launched `calls` times
    back to back, automatic form (stream) and 3 K splits, with the shader clock sampled
    by rocm-smi every ~0.1 s meanwhile: the matrix-core load without a break settles the
    clock at the chip's sustained power limit."""
    import re
    import subprocess
    import threading

    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    M, h = 144, 12288
    N = 3 * h
    sets = [kvq.kvq_w4_quantize(W.random_fp16((N, h), 9000 + 10 * c, "cuda", 0.02)) for c in range(3)]
    x = W.random_fp16((M, h), 9100, "cuda")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(kvq.kvq_gemm_w4_workspace_bytes(M, N, h, s) for s in (0, 3)) // 4 + 4,
                     dtype=torch.float32, device="cuda")
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                                     timeout=10).stdout
                m = re.search(r'"sclk clock speed:": "\((\d+)Mhz\)"', out)
                if m:
                    samples.append((time.time(), int(m.group(1))))
            except (OSError, subprocess.SubprocessError):
                return
            time.sleep(0.05)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    torch.cuda.synchronize()
    time.sleep(1.0)
    res = {"workload": f"OPT-175B QKV projection, M={M}, N={N}, K={h}, {calls} calls back to back, "
                       f"3 weight sets in rotation"}
    t_first = time.time()
    for label, splits in (("auto", 0), ("split3", 3)):
        t0 = time.time()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(calls):
            kvq.gemm_w4a16(x, *sets[r % 3], y=y, ws=ws, num_splits=splits)
        e1.record()
        torch.cuda.synchronize()
        t1 = time.time()
        clk = sorted(c for t, c in samples if t0 + 0.3 <= t <= t1)
        res[label] = {"us_per_call": round(e0.elapsed_time(e1) / calls * 1e3, 1),
                      "sclk_mhz_median": clk[len(clk) // 2] if clk else None, "clock_samples": len(clk)}
        time.sleep(1.0)
    idle = sorted(c for t, c in samples if t < t_first - 0.2)
    res["sclk_mhz_idle_median"] = idle[len(idle) // 2] if idle else None
    stop.set()
    th.join(timeout=15)
    del sets
    torch.cuda.empty_cache()
    return res


def bytes_prefill(b: int, a: int, s: int, d: int, mb: int = 4) -> int:
    """Algorithmic HBM bytes of kv_quantize_prefill_attend: q, k, v read once, out written
    once (fp16 [b][s][a][d] each), plus the K and V planes of s slots (codes d/2 bytes,
    min and scale (d/64) * mb bytes each, per (batch row, head, token))."""
    rows = b * a * s
    return 4 * rows * d * 2 + 2 * rows * (d // 2 + 2 * (d // 64) * mb)


def flops_prefill(b: int, a: int, s: int, d: int) -> int:
    """Causal prefill attention: query i meets keys 0..i; 2d flops for q.k and 2d for p.v."""
    return 4 * d * b * a * (s * (s + 1) // 2)


def time_prefill(reps: int = 12, warm: int = 8):
    """The prompt phase of one OPT-175B layer (b=144, a=96, d=128, prompt 512): the fused
    kv_quantize_prefill_attend (causal attention on the matrix cores + the cache planes)
    against kv_quantize_prefill alone; two caches in rotation; after `warm` untimed calls,
    medians of `reps` per-launch HIP events."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    w = W.OPT_175B
    st = torch.cuda.current_stream()
    q = W.prefill_q(w, 0, "cuda")
    k, v = W.prefill_kv(w, 0, "cuda")
    out = torch.empty_like(q)
    caches = [kvq.QuantKVCache(w.b, w.a, w.h, w.s, w.n, device="cuda") for _ in range(2)]

    def med(fn):
        for r in range(warm):  # the clock settles under the load before the timed calls
            fn(caches[r % 2])
        ms = []
        for r in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn(caches[r % 2])
            e1.record(st)
            ms.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ms)
        return t[len(t) // 2], t
    fused, all_ms = med(lambda c: kvq.kv_quantize_prefill_attend(c, q, k, v, out=out))
    quant, _ = med(lambda c: kvq.kv_quantize_prefill(c, k, v))
    nb = bytes_prefill(w.b, w.a, w.s, w.d)
    fl = flops_prefill(w.b, w.a, w.s, w.d)
    gbs = nb / fused / 1e6
    tfl = fl / fused / 1e9
    return {"workload": f"OPT-175B layer prompt: b={w.b} a={w.a} d={w.d} prompt {w.s}, causal, binary32 min/scale",
            "kernel": "k_prefill_pp<f32> (kv_quantize_prefill_attend, head_dim 128)",
            "ms_per_call_median": round(fused, 4), "ms_per_call_min": round(all_ms[0], 4),
            "algorithmic_bytes": nb, "flops": fl,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "hbm_floor_ms": round(nb / HBM_PEAK_GBS / 1e6, 4),
                         "mfma_floor_ms": round(fl / MFMA_F16_PEAK_TFLOPS / 1e9, 4)},
            "tflops": round(tfl, 1), "frac_of_mfma_f16_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
            "quantise_only_ms_median": round(quant, 4),
            "prompt_tokens_per_s": round(w.b * w.s / (fused / 1e3), 1)}


def time_host_attention(reps: int = 5):
    """Decode attention delegated to the CPU (decode_attention_q4_host) on one OPT-6.7B layer
    (b=32, a=32, d=128, context 544) with the int4 cache in host memory, on the host's cores,
    beside the two GPU alternatives for a cache that lives in host memory: copy its planes to
    HBM over PCIe (pinned, one transfer) and attend there, or keep a resident copy in HBM
    (decode_attention_q4 alone).  Medians over `reps` calls."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    import workloads as W
    w = W.OPT_6_7B
    T = w.s + w.n
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    k, v = W.prefill_kv(w, 0, "cpu", s_len=T)
    q = W.decode_inputs(w, 0, 1, "cpu")[0]
    hc = kvq.QuantKVCache(w.b, w.a, w.h, T, 0, device="cpu", meta="f32")
    kvq.kv_quantize_prefill_host(hc, k, v, n_threads=threads)
    out = torch.empty_like(q)
    host_ms = []
    for _ in range(reps + 1):
        t0 = time.perf_counter()
        kvq.decode_attention_q4_host(hc, q, T, out=out, n_threads=threads)
        host_ms.append((time.perf_counter() - t0) * 1e3)
    host_ms = sorted(host_ms[1:])
    pinned = [p.pin_memory() for p in hc.planes()]
    gc = kvq.QuantKVCache(w.b, w.a, w.h, T, 0, device="cuda", meta="f32")
    qd = q.cuda()
    st = torch.cuda.current_stream()
    copy_ms, attend_ms = [], []
    for _ in range(reps + 1):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(st)
        for dst, src in zip(gc.planes(), pinned):
            dst.copy_(src, non_blocking=True)
        e1.record(st)
        kvq.decode_attention_q4(gc, qd, T)
        e2.record(st)
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
        attend_ms.append(e1.elapsed_time(e2))
    copy_ms, attend_ms = sorted(copy_ms[1:]), sorted(attend_ms[1:])
    nb = bytes_decode(w.b * w.a, T, w.d)
    plane_bytes = sum(p.numel() * p.element_size() for p in pinned)
    hm, cm, am = host_ms[len(host_ms) // 2], copy_ms[len(copy_ms) // 2], attend_ms[len(attend_ms) // 2]
    return {"workload": f"OPT-6.7B layer: b={w.b} a={w.a} d={w.d} context {T}, binary32 min/scale planes",
            "threads": threads, "avx512": kvq.kvq_host_simd(), "cpu_model": cpu_model(),
            "algorithmic_bytes": nb, "cache_plane_bytes": plane_bytes,
            "host_attention": {"ms_per_call_median": round(hm, 3), "gbs": round(nb / hm / 1e6, 2),
                               "layer_tokens_per_s": round(w.b / (hm / 1e3), 1)},
            "copy_to_hbm_then_gpu": {"copy_ms_median": round(cm, 3), "attend_ms_median": round(am, 4),
                                     "pcie_gbs": round(plane_bytes / cm / 1e6, 2),
                                     "layer_tokens_per_s": round(w.b / ((cm + am) / 1e3), 1)},
            "gpu_resident": {"ms_per_call_median": round(am, 4), "gbs": round(nb / am / 1e6, 1)}}


def hbm_copy_ceiling():
    """Practical HBM ceiling for mixed read/write streams: a plain 4 GiB device copy
    (torch), read + write bytes / time."""
    import torch
    n = 4 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    ms = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del a, b
    return round(2 * n / min(ms[1:]) / 1e6, 1)


def hbm_read_ceiling(gib: int = 4, reps: int = 8):
    """Read-only HBM ceiling measured in the same run: kvq_stream_read over a `gib` GiB buffer
    (16-byte nontemporal loads, the cache streams' load form), best and median of `reps`."""
    import torch

    import quantized_kv_cache_prefill_amd as kvq
    n = gib << 30
    a = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros((n + 65535) // 65536, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    ev = []
    for _ in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        kvq.kvq_stream_read(a, sink)
        e1.record(st)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in ev[2:])
    del a, sink
    return {"bytes": n, "gbs_best": round(n / ms[0] / 1e6, 1), "gbs_median": round(n / ms[len(ms) // 2] / 1e6, 1),
            "kernel": "k_stream_read (kvq_stream_read)"}


# ------------------------------------------------------------- CPU baseline
def _oracle_pair_seconds(w, seed):
    """The oracle's work for one (batch row, head) of one layer of workload `w`: quantise the
    s-token prompt, then n decode steps of append + attention (dense, or top-k with
    k = ceil(topk_frac * T) for the sparse workload).  Returns (seconds, algorithmic bytes)."""
    import numpy as np

    import oracle
    G = w.d // 64
    rr = np.random.default_rng(seed)
    K = (rr.standard_normal((w.S, w.d)) * w.std).astype(np.float16)
    V = (rr.standard_normal((w.S, w.d)) * w.std).astype(np.float16)
    Q = (rr.standard_normal((w.n, w.d)) * w.std).astype(np.float16)
    t0 = time.perf_counter()
    planes = []
    for X in (K, V):
        c, m, sc = (np.zeros((w.S, w.d // 2), np.uint8), np.zeros((w.S, G), np.float32),
                    np.zeros((w.S, G), np.float32))
        c[:w.s], m[:w.s], sc[:w.s] = oracle.quantize_rows(X[:w.s])
        planes.append((c, m, sc))
    nbytes = 2 * bytes_quantize(w.s, w.d)
    for j in range(1, w.n + 1):
        pos = w.s + j - 1
        for X, (c, m, sc) in zip((K, V), planes):
            c[pos:pos + 1], m[pos:pos + 1], sc[pos:pos + 1] = oracle.quantize_rows(X[pos:pos + 1])
        hc = oracle.HeadCache(*planes[0], *planes[1])
        nbytes += 2 * bytes_quantize(1, w.d)
        if w.topk_frac > 0:
            oracle.attend_topk(Q[j - 1], hc, w.k_top(pos + 1), pos + 1)
            nbytes += bytes_topk(1, pos + 1, w.k_top(pos + 1), w.d)
        else:
            oracle.attend(Q[j - 1], hc, pos + 1)
            nbytes += bytes_decode(1, pos + 1, w.d)
    return time.perf_counter() - t0, nbytes


def oracle_layer_rate(w, cores, budget_s, seed0=1234):
    """The oracle on a bounded sample of (batch row, head) pairs of one layer of `w`, spread
    over `cores` threads (ctypes releases the GIL): GB/s over the same algorithmic bytes as
    the GPU, and the layer-tokens/s the sampled rate implies."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    oracle.lib()
    r = np.random.default_rng(seed0 + w.idx)
    pairs_total = w.b * w.a
    with cf.ThreadPoolExecutor(cores) as ex:
        # one untimed round (first calls), then one pair per thread timed to size the sample
        list(ex.map(lambda sd: _oracle_pair_seconds(w, int(sd)), r.integers(0, 2**31, min(cores, pairs_total))))
        tb = time.perf_counter()
        list(ex.map(lambda sd: _oracle_pair_seconds(w, int(sd)), r.integers(0, 2**31, min(cores, pairs_total))))
        batch = time.perf_counter() - tb
        n_pairs = int(min(pairs_total, max(1, budget_s / max(batch, 1e-3)) * cores))
        t0 = time.perf_counter()
        res = list(ex.map(lambda sd: _oracle_pair_seconds(w, int(sd)), r.integers(0, 2**31, n_pairs)))
        wall = time.perf_counter() - t0
    nbytes = sum(b for _, b in res)
    return {"gbs": round(nbytes / wall / 1e9, 4), "pairs": n_pairs, "of_pairs": pairs_total, "wall_s": round(wall, 2),
            "layer_tokens_per_s": round(n_pairs / w.a * w.n / wall, 3),
            "sample": (f"{n_pairs} of the {pairs_total} (batch row, head) pairs of one {w.name} layer: prompt quantise "
                       f"({w.s} tokens) + {w.n} x (append + {'top-k' if w.topk_frac > 0 else 'dense'} attention)")}


def cpu_baseline(budget_s: float = 12.0, per_config_budget_s: float = 3.0):
    """The oracle on a sample of the headline job (OPT-175B layer, `budget_s` of work) and on
    a sample of one layer of every other configuration (`per_config_budget_s` each)."""
    import workloads as W

    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(16, affinity))
    main = oracle_layer_rate(W.OPT_175B, cores, budget_s)
    t1 = sum(_oracle_pair_seconds(W.OPT_175B, 77 + i)[0] for i in range(3))
    per_pair_bytes = _oracle_pair_seconds(W.OPT_175B, 80)[1]
    per_config = {}
    for w in (W.TINY, W.OPT_6_7B, W.OPT_30B, W.SPARSE):
        per_config[w.name] = oracle_layer_rate(w, cores, per_config_budget_s)
    return {"value": main["gbs"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": main["sample"] + f"; {main['wall_s']} s wall on {cores} threads",
            "layer_tokens_per_s": main["layer_tokens_per_s"],
            "single_thread_gbs": round(3 * per_pair_bytes / t1 / 1e9, 4),
            "host_cpus_in_affinity": affinity, "os_cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(), "per_config": per_config}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------------------- main
LEGS = {"prefill": lambda: time_prefill(), "proj": lambda: time_projections(), "topk": lambda: time_topk(),
        "proj_sustained": lambda: time_projection_sustained(),
        "split": lambda: time_split_context(), "meta16": lambda: time_meta_f16(),
        "host": lambda: time_host_attention(), "read_ceiling": lambda: hbm_read_ceiling(),
        "tiny": lambda: time_tiny_latency()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=0, help="layers in the stack (default: the workload's 96)")
    ap.add_argument("--decode-steps", type=int, default=0, help="decode steps per job (default 32)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-topk", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the C1/C2/C3 configuration legs")
    ap.add_argument("--no-meta16", action="store_true", help="skip the binary16-metadata leg")
    ap.add_argument("--no-proj", action="store_true", help="skip the int4-weight projection leg")
    ap.add_argument("--no-host", action="store_true", help="skip the CPU-delegated attention leg")
    ap.add_argument("--no-prefill", action="store_true", help="skip the fused prefill attention leg")
    ap.add_argument("--meta", choices=("f32", "f16"), default="f32",
                    help="min/scale plane type of the timed stack (default binary32)")
    ap.add_argument("--fused", action="store_true",
                    help="append and attend in one kv_append_attend_q4 launch per layer-step")
    ap.add_argument("--leg", choices=tuple(LEGS), default=None,
                    help="run this one leg alone and print its JSON (for profiling one kernel)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU step and this build runs on "
              "a single MI355X.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import workloads as W

    if args.leg:
        log(f"[bench] leg {args.leg} alone")
        print(json.dumps({args.leg: LEGS[args.leg]()}), flush=True)
        return

    w = W.OPT_175B
    job = Job(w, args.layers or w.layers, args.decode_steps or w.n, args.meta, args.fused)
    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    ms_step, events = job.run(args.steps, args.warmup)
    sm = job.summary(ms_step, events, args.steps)
    avg_ms, achieved = sm["avg_launch_ms"], sm["achieved_gbs"]
    value = job.b_step / (ms_step / 1e3) / 1e9

    traffic = stored_traffic() if job.meta == "f32" else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": (("k_decode<128,4,2> (kv_append_attend_q4: append + attention)" if job.fused
                            else "k_decode<128,4,2> (decode_attention_q4)") + f", {job.meta} min/scale planes"),
                "algorithmic_bytes_per_launch": sm["algorithmic_bytes_per_launch"],
                "avg_launch_ms": round(avg_ms, 5), "launches_timed": len(events)}

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"OPT-175B layer stack: b={w.b} a={w.a} d={w.d} h={w.h}, prompt {w.s}, "
                               f"{job.n} decode steps, {job.L} int4 caches resident",
                   "b": w.b, "a": w.a, "d": w.d, "h": w.h, "s": w.s, "n": job.n, "layers": job.L,
                   "meta": job.meta,
                   "step": ("prefill quantise all layers + n x (append + decode attention) all layers"
                            + (", append fused into the attention launch" if job.fused else ", two launches")),
                   "parallelism": "1 GPU"},
        "roofline": roofline,
        "decode_attention": sm["decode_attention"],
        "step_bytes": {"prefill": job.b_prefill, "append": job.b_append, "decode": job.b_decode},
    }
    log(f"[bench] step {ms_step:.1f} ms, decode kernel {achieved:.0f} GB/s")
    del job
    torch.cuda.empty_cache()
    log("[bench] read-only HBM ceiling")
    res["hbm_read_ceiling"] = hbm_read_ceiling()
    if not args.no_configs:
        log("[bench] configuration legs: tiny latency, OPT-6.7B (cache-warm layer, 32-layer stack), "
            "OPT-30B 48-layer stack")
        res["configs"] = {"tiny": time_tiny_latency(),
                          "opt-6.7b": {"single_layer_cache_warm": time_cache_warm_layer(W.OPT_6_7B),
                                       "stack": time_stack(W.OPT_6_7B)},
                          "opt-30b": {"stack": time_stack(W.OPT_30B)}}
        torch.cuda.empty_cache()
    if not args.no_topk:
        log("[bench] sparse top-k leg")
        res["sparse_topk"] = time_topk()
        log("[bench] split-context leg")
        res["split_context"] = time_split_context()
    torch.cuda.empty_cache()
    if not args.no_meta16:
        log("[bench] binary16 metadata leg")
        res["meta_f16"] = time_meta_f16()
        torch.cuda.empty_cache()
    if not args.no_proj:
        log("[bench] int4-weight projection leg")
        res["projections_w4"] = time_projections()
        torch.cuda.empty_cache()
    if not args.no_prefill:
        log("[bench] fused prefill attention leg")
        res["prefill_attention"] = time_prefill()
        torch.cuda.empty_cache()
    if not args.no_host:
        log("[bench] CPU-delegated attention leg")
        res["host_attention"] = time_host_attention()
        torch.cuda.empty_cache()
    res["hbm_copy_ceiling_gbs"] = hbm_copy_ceiling()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

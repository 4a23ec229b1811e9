"""Benchmark of the TokenGate gated-prefill hot path on one MI355X.

A step is one pass of the whole path over one prompt of the workload:
gate MLP over all N tokens and top-K select (question tail kept) in one
kernel -> gather of the kept rows, gate values and positions -> for each upper
layer: RoPE + the compact KV cache, then token-gated causal GQA attention.
Inputs are resident in HBM before timing starts; four copies of the hidden
states rotate between steps so that the 256 MB last-level cache cannot serve
the gate's input.

    python bench.py [--steps K] [--warmup W] [--workload qwen1p7b_32k]

Prints one JSON line.  `value` is tokens/s (prompt tokens N per step time).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gated-prefill tokens/s (gate+topK+gated attn) @N=32k,K=4k; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ATTN_KERNEL_SOURCE = os.path.join(ROOT, "learned_token_pruning_03_amd", "csrc", "attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_qwen1p7b_32k_traffic.json")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="qwen1p7b_32k", choices=["qwen1p7b_32k", "qwen1p7b_128k", "stack19"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-full-context", action="store_true",
                   help="skip the comparison of one upper layer on the K kept tokens with one on all N tokens")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the 28-layer prefill comparison (gated at layer 9 of 28 against all layers full)")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the decode attention figure over compact KV caches")
    p.add_argument("--stage-reps", type=int, default=30, help="repetitions of the per-stage timing loop")
    p.add_argument("--select", default="auto", choices=["auto", "one", "ws"],
                   help="stand-alone top-K entry point timed for reference (and used by the 128k workload): "
                        "tg_select_topk (one workgroup per prompt), tg_select_topk_ws (several workgroups, caller "
                        "workspace), or auto: ws from %d tokens" % SELECT_WS_FROM)
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the run, launch a plain 1 GiB -> 1 GiB streaming kernel (torch.neg on fp32) "
                        "three times; its PMC byte counters calibrate FETCH_SIZE / WRITE_SIZE")
    p.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU run: reduce two rocprofv3 --pmc output folders (FETCH_SIZE, then WRITE_SIZE, "
                        "each from a --copy-calibration run) to HBM bytes per attention launch")
    return p.parse_args(argv)


def _file_sha(path):
    """SHA-256 prefix of a C++/HIP source's code: comments, trailing spaces and
    blank lines are dropped first, so that a comment edit does not void the
    counters taken on the same code."""
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


# The stand-alone multi-workgroup select (a clearing kernel, a histogram kernel
# whose last workgroup ranks, a compaction) costs ~27-34 us per call at any
# length, where the one-workgroup kernel grows with the prompt: 21 us at 16k
# tokens, 32 us at 32k, 114 us at 128k (events, one MI355X).
SELECT_WS_FROM = 24576


H_COPIES = 4  # copies of h: a gate input is reused only after 3 x 134 MB of other gate traffic


class Path:
    """Device buffers and the launch sequence of one workload."""

    def __init__(self, tg, W, name, dev, select="auto"):
        import torch
        sh = W.SHAPES[name]
        seed = W.SEEDS[name]
        self.tg, self.sh, self.dev = tg, sh, dev
        self.h = [W.hidden_states(sh.n, sh.d, sh.dtype, seed + 100 * c, planted_frac=sh.planted_frac).to(dev)
                  for c in range(H_COPIES)]
        w1, b1, w2, b2 = W.gate_weights(sh.d, sh.hidden, sh.dtype, seed)
        self.w1, self.b1, self.w2, self.b2 = w1.to(dev), b1.to(dev), w2.to(dev), b2
        self.layers = []
        for layer in range(sh.layers):
            q, k, v = W.qkv(sh.k, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, seed * 1000 + layer)
            self.layers.append((q.to(dev), k.to(dev), v.to(dev), torch.empty_like(k, device=dev),
                                torch.empty_like(v, device=dev), torch.empty_like(q, device=dev)))
        self.table = tg.tg_rope_table(sh.n, sh.dh, sh.rope_base, dev)
        kept = min(sh.k, sh.n)
        f32, i32 = torch.float32, torch.int32
        self.g = torch.empty(sh.n, dtype=f32, device=dev)
        self.idx = torch.empty(kept, dtype=i32, device=dev)
        # Zero-filled once; every call of the gate + select leaves it zero-filled.
        self.sel_workspace = tg.select_workspace(sh.n, dev)
        self.ref_workspace = tg.select_workspace(sh.n, dev)  # for the stand-alone select timings
        self.ref_idx = torch.empty(kept, dtype=i32, device=dev)
        self.hk = torch.empty(kept, sh.d, dtype=sh.dtype, device=dev)
        self.gk = torch.empty(kept, dtype=f32, device=dev)
        self.pos = torch.empty(kept, dtype=i32, device=dev)
        self.lse = torch.empty(sh.hq, kept, dtype=f32, device=dev)
        self.wide_g = None
        if name == "qwen1p7b_128k":  # select/attention use a widely spread gate vector
            self.wide_g = W.gate_values_wide(sh.n, seed).to(dev)
        self.fused = self.wide_g is None
        self.select_ws = select == "ws" or (select == "auto" and sh.n >= SELECT_WS_FROM)
        self.step_no = 0

    def cur_h(self):
        return self.h[self.step_no % len(self.h)]

    # The path: gate + select + gather, then per upper layer RoPE + KV and attention.
    def prune(self):
        """Gate, top-K select and gather.  Two kernels (tg_gate_select_gather)
        where the selection ranks the gate's own scores; the 128k workload
        ranks a drawn, widely spread gate vector instead, so there the gate,
        the select and the gather are three calls."""
        if self.fused:
            self.tg.tg_gate_select_gather(self.cur_h(), self.w1, self.b1, self.w2, self.b2, self.sh.k,
                                          self.sh.q_len, g=self.g, idx=self.idx, h_out=self.hk, g_out=self.gk,
                                          pos_out=self.pos, workspace=self.sel_workspace)
        else:
            self.gate()
            self.select(self.wide_g, self.idx)
            self.gather()

    def gate_select(self):
        """Gate + select without the gather (reference timing)."""
        self.tg.tg_gate_select(self.cur_h(), self.w1, self.b1, self.w2, self.b2, self.sh.k, self.sh.q_len,
                               g=self.g, idx=self.idx, workspace=self.sel_workspace)

    # Stand-alone stages, timed for reference next to the fused call.
    def gate(self):
        self.tg.tg_gate_score(self.cur_h(), self.w1, self.b1, self.w2, self.b2, g=self.g)

    def select(self, g=None, idx=None):
        g = self.g if g is None else g
        idx = self.ref_idx if idx is None else idx
        if self.select_ws:
            self.tg.tg_select_topk_ws(g, self.sh.k, self.sh.q_len, idx=idx, workspace=self.ref_workspace)
        else:
            self.tg.tg_select_topk(g, self.sh.k, self.sh.q_len, idx=idx)

    def gather(self):
        g = self.g if self.wide_g is None else self.wide_g
        self.tg.tg_gather(self.cur_h(), g, self.idx, h_out=self.hk, g_out=self.gk, pos_out=self.pos)

    def rope(self, layer):
        q, k, v, kc, vc, _ = self.layers[layer]
        self.tg.tg_rope_kv(q, k, v, self.pos, self.table, k_cache=kc, v_cache=vc)

    def attn(self, layer, events=None):
        q, _, _, kc, vc, o = self.layers[layer]
        if events is not None:  # start/end pair on the stream the kernel runs on
            events[0].record()
        self.tg.tg_gated_attn(q, kc, vc, self.gk, self.pos, o=o, lse=self.lse)
        if events is not None:
            events[1].record()

    def step(self, attn_events=None):
        self.prune()
        for layer in range(self.sh.layers):
            self.rope(layer)
            self.attn(layer, None if attn_events is None else attn_events[layer])
        self.step_no += 1


def attn_flops(sh):
    """Algorithmic flops of one causal attention launch: 2 products (QK^T and
    PV) x 2 flop per multiply-add x Dh x Hq x visible (query, key) pairs."""
    k = min(sh.k, sh.n)
    return 4.0 * sh.dh * sh.hq * k * (k + 1) / 2.0


def gate_flops(sh):
    return 2.0 * sh.n * sh.d * sh.hidden + 4.0 * sh.n * sh.hidden


def stage_bytes(sh):
    k = min(sh.k, sh.n)
    es = 2
    return {
        "gate": sh.n * sh.d * es + sh.hidden * sh.d * es + sh.n * 4,
        "select": sh.n * 4 + k * 4,
        "gate_select": sh.n * sh.d * es + sh.hidden * sh.d * es + sh.n * 4 + k * 4,
        "prune": sh.n * sh.d * es + sh.hidden * sh.d * es + sh.n * 4 + k * 4 + 2 * k * (sh.d * es + 8),
        "gather": 2 * k * (sh.d * es + 8),
        "rope_kv": k * (2 * (sh.hq + sh.hkv) * sh.dh * es + 2 * sh.hkv * sh.dh * es + sh.dh * 4),
        "attn": k * (sh.hq * sh.dh * es * 2 + 2 * sh.hkv * sh.dh * es + 8),
    }


def graph_steps(torch, path, steps, warmup):
    """The same step captured into one HIP graph per copy of h and replayed:
    the launch sequence without the host's per-call overhead.  The captured
    calls are the library's kernels only (no memset nodes)."""
    copies = len(path.h)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(copies):  # warm-up on the capture stream
            path.step_no = c
            path.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        path.step_no = c
        with torch.cuda.graph(g):
            path.step()
        graphs.append(g)
    for i in range(warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        graphs[i % copies].replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return {"ms_per_step": round(ms, 4), "tokens/s": round(path.sh.n / (ms * 1e-3), 1), "steps": steps}


SPIN_CYCLES = 100_000  # GPU clock cycles of the spin kernel queued ahead of a timed call


def queue_ahead(torch):
    """Keep the stream busy for a few tens of microseconds (torch's spin
    kernel) before a start event, so that the event is processed after the
    host has queued the work it times: an event pair around work launched onto
    an idle stream also measures the host's launch latency.  Skipped where
    torch has no spin kernel."""
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is not None:
        spin(SPIN_CYCLES)


def path_stage_fns(path):
    """(name, call) of the step's own stages, in path order (one upper layer)."""
    if path.fused:
        fns = [("prune", path.prune)]
    else:
        fns = [("gate", path.gate), ("select", lambda: path.select(path.wide_g, path.idx)), ("gather", path.gather)]
    return fns + [("rope_kv", lambda: path.rope(0)), ("attn", lambda: path.attn(0))]


def reference_fns(path):
    """Stand-alone calls timed for reference next to the step's own stages."""
    return [("gate", path.gate), ("gate_select", path.gate_select), ("select", lambda: path.select()),
            ("gather", path.gather)]


def time_stages(path, reps):
    """Per-stage medians (and means) in path order, each stage right after the
    one before it, as in the step: every input the previous stage touched may
    still sit in the last-level cache (cache-warm figures)."""
    import torch
    fns = path_stage_fns(path)
    samples = {n: [] for n, _ in fns}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(fns))]
    for _ in range(reps):
        queue_ahead(torch)
        for i, (_, fn) in enumerate(fns):
            ev[2 * i].record()
            fn()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        for i, (n, _) in enumerate(fns):
            samples[n].append(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3)  # us
        path.step_no += 1
    return {n: statistics.median(v) for n, v in samples.items()}, {n: sum(v) / len(v) for n, v in samples.items()}


FLUSH_BYTES = 1 << 30  # read between cold launches: 4x the 256 MB last-level cache


def flush_caches(flush):
    """Reads the whole flush buffer (a reduction, no writes: writing it would
    leave dirty lines whose write-back the next kernel would pay for)."""
    flush.amax()


def cold_stages(path, reps):
    """Per-launch event pairs of each stage after 1 GiB has been read from a
    scratch buffer (outside the pair), so that no input is served by the L2s or
    the 256 MB last-level cache.  The pair also holds the launch's dispatch
    latency (a few us), so these figures are upper bounds."""
    import torch
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=path.dev)
    fns = path_stage_fns(path) + reference_fns(path)
    seen = set()
    out = {}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for n, fn in fns:
        if n in seen:
            continue
        seen.add(n)
        ts = []
        for r in range(reps):
            flush_caches(flush)
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3)
            path.step_no += 1
        out[n] = statistics.median(ts)
    del flush
    return out


def back_to_back(path, reps=24):
    """Per-launch time of a stage launched `reps` times in a row between one
    event pair, so that the pair's own dispatch overhead (a few us against a
    gather of about 8) is spread over the launches; the gaps between the
    kernels stay in the figure.

    Cold (the HBM figures): every launch works on a footprint that was last
    touched more than 256 MB of traffic earlier, so neither the L2s nor the
    last-level cache can serve it:
      gate, gate_select, prune (gate + select + gather)
                         the four copies of h (134 MB each) in turn;
      gather             24 footprints: the four copies of h x six disjoint
                         ascending sets of kept rows, each written to one of
                         twelve output buffers in turn (16.8 MB read + 16.8 MB
                         written per launch);
      rope_kv            eight sets of q, k, v and caches (50 MB each) in turn.
    Warm (no HBM claim): attention (MFMA-bound; its 50 MB of q, k, v stay in the
    last-level cache) and the stand-alone select (128 KB of scores)."""
    import torch
    sh, dev, tg = path.sh, path.dev, path.tg
    kept = min(sh.k, sh.n)
    out = {}
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def timed(name, launches):
        flush_caches(flush)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for fn in launches:
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        out[name] = ev[0].elapsed_time(ev[1]) * 1e3 / len(launches)

    def at(i, fn):
        def run():
            path.step_no = i
            fn()
        return run

    timed("gate", [at(i, path.gate) for i in range(reps)])
    if path.fused:
        timed("prune", [at(i, path.prune) for i in range(reps)])
        timed("gate_select", [at(i, path.gate_select) for i in range(reps)])
    # gather: disjoint kept-row sets, each ascending, as select writes them
    perm = torch.randperm(sh.n, generator=torch.Generator().manual_seed(5))
    nsets = max(1, min(6, sh.n // kept))
    sets = [perm[j * kept:(j + 1) * kept].sort().values.to(torch.int32).to(dev) for j in range(nsets)]
    outs = [(torch.empty(kept, sh.d, dtype=sh.dtype, device=dev), torch.empty(kept, dtype=torch.float32, device=dev),
             torch.empty(kept, dtype=torch.int32, device=dev)) for _ in range(12)]
    g = path.g if path.wide_g is None else path.wide_g

    def gather_at(i):
        hk, gk, pos = outs[i % len(outs)]
        return lambda: tg.tg_gather(path.h[i % len(path.h)], g, sets[(i // len(path.h)) % nsets], h_out=hk,
                                    g_out=gk, pos_out=pos)

    timed("gather", [gather_at(i) for i in range(reps)])
    # rope + KV: eight independent sets of q, k, v and caches
    rsets = []
    for j in range(8):
        q, k, v = (torch.randn(kept, hh, sh.dh, device=dev).mul_(0.09).to(sh.dtype) for hh in (sh.hq, sh.hkv, sh.hkv))
        rsets.append((q, k, v, torch.empty_like(k), torch.empty_like(v)))
    pos = path.pos

    def rope_at(i):
        q, k, v, kc, vc = rsets[i % len(rsets)]
        return lambda: tg.tg_rope_kv(q, k, v, pos, path.table, k_cache=kc, v_cache=vc)

    timed("rope_kv", [rope_at(i) for i in range(reps)])
    timed("attn", [lambda: path.attn(0) for _ in range(reps)])
    timed("select", [lambda: path.select() for _ in range(reps)])
    del flush, rsets, outs
    return out


FFN = 6144  # SwiGLU width of the Qwen3-1.7B-shaped upper layer (d = 2048)


def upper_layer(tg, W, sh, dev, m, gated, reps=8):
    """One upper layer of the Qwen3-1.7B shape on m token rows, every stage in
    the library: fused QKV projection -> RoPE + KV cache -> attention (gated
    on the kept tokens, ungated over the full prompt) -> O projection onto the
    residual stream -> SwiGLU -> down projection onto the residual stream.
    Medians of event-timed repetitions per stage.  RMSNorms are not included."""
    import numpy as np
    import torch
    d, hq, hkv, dh = sh.d, sh.hq, sh.hkv, sh.dh
    x = W.hidden_states(m, d, sh.dtype, 21).to(dev)
    # The O and down projections add into x in place; every repetition starts
    # from the same x again (restored outside the timed stages), so each one
    # times one layer pass on the same input.
    x0 = x.clone()
    w_qkv = W.linear_weight((hq + 2 * hkv) * dh, d, sh.dtype, 22).to(dev)
    w_o = W.linear_weight(d, hq * dh, sh.dtype, 23).to(dev)
    w_g = W.linear_weight(FFN, d, sh.dtype, 24).to(dev)
    w_u = W.linear_weight(FFN, d, sh.dtype, 25).to(dev)
    w_d = W.linear_weight(d, FFN, sh.dtype, 26).to(dev)
    if gated:
        pos = np.sort(np.random.default_rng(27).choice(sh.n, m, replace=False)).astype(np.int32)
        g = W.random_scores(m, 28).to(dev)
    else:
        pos, g = np.arange(m, dtype=np.int32), None
    pos = torch.from_numpy(pos).to(dev)
    table = tg.tg_rope_table(sh.n, dh, sh.rope_base, dev)
    q = torch.empty(m, hq, dh, dtype=sh.dtype, device=dev)
    k, v = (torch.empty(m, hkv, dh, dtype=sh.dtype, device=dev) for _ in range(2))
    kc, vc = torch.empty_like(k), torch.empty_like(v)
    o = torch.empty_like(q)
    a = torch.empty(m, FFN, dtype=sh.dtype, device=dev)
    stages = [
        ("qkv_proj", lambda: tg.tg_qkv_proj(x, w_qkv, hq, hkv, dh, q=q, k=k, v=v)),
        ("rope_kv", lambda: tg.tg_rope_kv(q, k, v, pos, table, k_cache=kc, v_cache=vc)),
        ("attn", lambda: tg.tg_gated_attn(q, kc, vc, g, pos, o=o)),
        ("o_proj", lambda: tg.tg_linear(o.view(m, hq * dh), w_o, residual=x, y=x)),
        ("swiglu", lambda: tg.tg_swiglu(x, w_g, w_u, y=a)),
        ("down_proj", lambda: tg.tg_linear(a, w_d, residual=x, y=x)),
    ]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
    times = {n: [] for n, _ in stages}
    for r in range(reps + 1):
        x.copy_(x0)
        queue_ahead(torch)
        ev[0].record()
        for i, (_, fn) in enumerate(stages):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        if r:
            for i, (n, _) in enumerate(stages):
                times[n].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
    med = {n: round(statistics.median(t), 2) for n, t in times.items()}
    dense_flops = 2.0 * m * d * ((hq + 2 * hkv) * dh + hq * dh + 3 * FFN)
    dense_us = med["qkv_proj"] + med["o_proj"] + med["swiglu"] + med["down_proj"]
    attn_flops = 4.0 * dh * hq * m * (m + 1) / 2.0
    return {"rows": m, "gated": gated, "stage_us": med, "total_us": round(sum(med.values()), 2),
            "dense_us": round(dense_us, 2), "dense_TFLOP/s": round(dense_flops / (dense_us * 1e-6) / 1e12, 1),
            "attn_TFLOP/s": round(attn_flops / (med["attn"] * 1e-6) / 1e12, 1)}


STACK_LAYERS, STACK_SELECT_LAYER = 28, 9  # Qwen3-1.7B depth; the gate sits after layer 9


def prune_time(tg, W, sh, dev, reps=10):
    """Median event-timed gate + select (one call) plus gather on one prompt of
    sh.n tokens: the pruning overhead paid once per prompt at the selection
    layer."""
    import torch
    seed = W.SEEDS[sh.name]
    h = W.hidden_states(sh.n, sh.d, sh.dtype, seed, planted_frac=sh.planted_frac).to(dev)
    w1, b1, w2, b2 = (t.to(dev) if hasattr(t, "to") else t for t in W.gate_weights(sh.d, sh.hidden, sh.dtype, seed))
    kept = min(sh.k, sh.n)
    g = torch.empty(sh.n, dtype=torch.float32, device=dev)
    idx = torch.empty(kept, dtype=torch.int32, device=dev)
    ws = tg.select_workspace(sh.n, dev)
    hk = torch.empty(kept, sh.d, dtype=sh.dtype, device=dev)
    gk = torch.empty(kept, dtype=torch.float32, device=dev)
    pos = torch.empty(kept, dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts = []
    for r in range(reps + 2):
        queue_ahead(torch)
        ev[0].record()
        tg.tg_gate_select(h, w1, b1, w2, b2, sh.k, sh.q_len, g=g, idx=idx, workspace=ws)
        tg.tg_gather(h, g, idx, h_out=hk, g_out=gk, pos_out=pos)
        ev[1].record()
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3)
    return statistics.median(ts)


def stack_ratio(tg, W, dev):
    """Prefill of a whole Qwen3-1.7B-shaped stack (28 layers, random weights),
    with the gate after layer 9 and K = 4096 of N = 65536 tokens kept, against
    the same stack with every layer on all N tokens.  Composed from medians of
    one layer of each kind, timed separately, times the layer counts:
        full  = 28 x (one layer on N tokens, no gate)
        gated =  9 x (one layer on N tokens, no gate)
               + gate + select + gather on N tokens
               + 19 x (one gated layer on the K kept tokens)
    Each layer is every library stage (QKV, RoPE + KV, attention, O + residual,
    SwiGLU, down + residual); RMSNorms, embeddings and the LM head are left
    out of both stacks."""
    sh = W.SHAPES["stack19"]
    full = upper_layer(tg, W, sh, dev, sh.n, gated=False, reps=2)
    gated = upper_layer(tg, W, sh, dev, sh.k, gated=True, reps=8)
    prune_us = prune_time(tg, W, sh, dev)
    below = STACK_SELECT_LAYER
    above = STACK_LAYERS - STACK_SELECT_LAYER
    t_full = STACK_LAYERS * full["total_us"]
    t_gated = below * full["total_us"] + prune_us + above * gated["total_us"]
    return {"n": sh.n, "k": sh.k, "layers": STACK_LAYERS, "selection_layer": STACK_SELECT_LAYER,
            "full_layer_us": full["total_us"], "gated_layer_us": gated["total_us"], "pruning_us": round(prune_us, 2),
            "full_stack_ms": round(t_full / 1e3, 3), "gated_stack_ms": round(t_gated / 1e3, 3),
            "prefill_speedup": round(t_full / t_gated, 3),
            "composition": "per-layer medians x layer counts (9 full + pruning + 19 gated vs 28 full); "
                           "each layer timed as one unit of six library calls",
            "full_layer": full, "gated_layer": gated}


def decode_step(tg, W, sh, dev, batch=32, reps=20):
    """Decode attention of one upper layer after pruning: `batch` sequences,
    each one new query over its compact cache of K kept prompt tokens plus a
    ragged 0-255 generated tokens (gate 1), median of event-timed launches.
    Algorithmic bytes: the caches (K and V), the gate values, q and o."""
    import numpy as np
    import torch
    rng = np.random.default_rng(11)
    lens = [sh.k + int(x) for x in rng.integers(0, 256, batch)]
    total = int(sum(lens))
    q, _, _ = W.qkv(batch, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, 12)
    _, kc, vc = W.qkv(total, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, 13)
    g = torch.ones(total)
    for b in range(batch):  # the kept prompt tokens carry their gate values
        a = sum(lens[:b])
        g[a:a + sh.k] = W.random_scores(sh.k, 14 + b)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    q, kc, vc, g, cu = (t.to(dev) for t in (q, kc, vc, g, cu))
    o = torch.empty_like(q)
    lse = torch.empty(batch, sh.hq, dtype=torch.float32, device=dev)
    ws = torch.empty(tg.tg_decode_attn_workspace_size(batch, max(lens), sh.hq, sh.hkv, sh.dh), dtype=torch.uint8,
                     device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts = []
    for r in range(reps + 2):
        queue_ahead(torch)
        ev[0].record()
        tg.tg_decode_attn(q, kc, vc, g, cu, max(lens), o=o, lse=lse, workspace=ws)
        ev[1].record()
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3)
    esz = 2 if sh.dtype == torch.bfloat16 else 4
    byts = 2 * total * sh.hkv * sh.dh * esz + 4 * total + 2 * batch * sh.hq * sh.dh * esz + 4 * batch * sh.hq
    us = statistics.median(ts)
    return {"batch": batch, "cache_len_mean": round(total / batch, 1), "us": round(us, 2),
            "GB/s": round(byts / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
            "tokens/s": round(batch / (us * 1e-6), 1)}


ATTN_SAMPLE_ROWS = 4096  # query rows of the attention in the CPU baseline's sample (all, up to 4096 kept)


def cpu_baseline(W, name):
    """The oracle, untouched, on a bounded sample of the same workload (a few
    to some tens of seconds of host work), scaled to the whole prompt: the full
    gate, select, gather and RoPE, and up to 4096 random query rows of the
    attention (scaled by the exact count of visible query-key pairs); one warm
    pass, then per stage the median of three timed passes."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle as O
    sh = W.SHAPES[name]
    seed = W.SEEDS[name]
    h = W.hidden_states(sh.n, sh.d, sh.dtype, seed, planted_frac=sh.planted_frac)
    w1, b1, w2, b2 = W.gate_weights(sh.d, sh.hidden, sh.dtype, seed)
    q, k, v = W.qkv(sh.k, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, seed * 1000)
    rows_gate = sh.n

    def one_pass():
        t0 = time.perf_counter()
        g, _ = O.ref_gate(h[:rows_gate], w1, b1, w2, b2)
        t_gate = (time.perf_counter() - t0) * sh.n / rows_gate
        g_full = g.astype(np.float32)
        t0 = time.perf_counter()
        idx = O.ref_select(g_full, sh.k, sh.q_len)
        t_sel = time.perf_counter() - t0
        t0 = time.perf_counter()
        hk, gk, pos = O.ref_gather(h.view(torch.int16).numpy(), g_full, idx)
        t_gat = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.ref_rope_kv(q, k, v, pos, sh.rope_base)
        t_rope = time.perf_counter() - t0
        kk = len(idx)
        n_rows = min(ATTN_SAMPLE_ROWS, kk)
        rows = np.sort(np.random.default_rng(seed).choice(kk, n_rows, replace=False))
        t0 = time.perf_counter()
        O.ref_attn(q, k, v, gk, pos, rows=rows)
        t_attn = (time.perf_counter() - t0) * (kk * (kk + 1) / 2) / float(np.sum(rows + 1))
        return kk, n_rows, {"gate": t_gate, "select": t_sel, "gather": t_gat, "rope_kv": t_rope, "attn": t_attn}

    # One warm pass, then the median of three timed passes, stage by stage.
    one_pass()
    passes = [one_pass() for _ in range(3)]
    kk, n_rows = passes[0][0], passes[0][1]
    stage_s = {st: statistics.median(p[2][st] for p in passes) for st in passes[0][2]}
    t_gate, t_sel, t_gat, t_rope, t_attn = (stage_s[st] for st in ("gate", "select", "gather", "rope_kv", "attn"))
    total = t_gate + t_sel + t_gat + sh.layers * (t_rope + t_attn)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": sh.n / total,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"numpy fp64 oracle on the same seeded {name} inputs: gate on {rows_gate} of {sh.n} rows, "
                   f"full select/gather/RoPE, attention on {n_rows} of {kk} query rows (all heads); each stage "
                   f"scaled to the full prompt; median of 3 timed passes after a warm one"
                   + (f"; RoPE + attention timed for one upper layer, x{sh.layers} extrapolated" if sh.layers > 1
                      else "")),
        "stage_s": stage_s,
        "host_cpus": os.cpu_count(),
        "cpu_model": _cpu_model(),
        "next_rows": cpu_next_rows(W, sh),
    }


def _cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_next_rows(W, sh, batch=32):
    """The oracle on the two later rows the bench also times on the GPU, each on
    a bounded sample scaled to the full call: decode attention (16 of the 32
    sequences, caches of K keys) and one upper layer's dense work (QKV and O
    projections, SwiGLU, down projection on 1024 of the K kept rows)."""
    import numpy as np
    import torch

    import oracle as O
    nseq = 16
    q, _, _ = W.qkv(nseq, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, 12)
    _, kc, vc = W.qkv(nseq * sh.k, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, 13)
    g = W.random_scores(nseq * sh.k, 14)
    cu = np.arange(nseq + 1) * sh.k
    t0 = time.perf_counter()
    O.ref_decode(q, kc, vc, g, cu)
    t_dec = (time.perf_counter() - t0) * batch / nseq
    rows, d = 1024, sh.d
    x = W.hidden_states(rows, d, sh.dtype, 21)
    w_qkv = W.linear_weight((sh.hq + 2 * sh.hkv) * sh.dh, d, sh.dtype, 22)
    w_o = W.linear_weight(d, sh.hq * sh.dh, sh.dtype, 23)
    w_g = W.linear_weight(FFN, d, sh.dtype, 24)
    w_u = W.linear_weight(FFN, d, sh.dtype, 25)
    w_d = W.linear_weight(d, FFN, sh.dtype, 26)
    o = torch.zeros(rows, sh.hq * sh.dh, dtype=sh.dtype)
    t0 = time.perf_counter()
    O.ref_linear(x, w_qkv)
    O.ref_linear(o, w_o, x)
    O.ref_mlp(x, w_g, w_u, w_d, x)
    t_dense = (time.perf_counter() - t0) * sh.k / rows
    return {"decode_s": t_dec, "decode_tokens/s": batch / t_dec,
            "upper_dense_s": t_dense, "upper_dense_rows": sh.k,
            "sample": f"decode: {nseq} of {batch} sequences with {sh.k}-key caches, scaled by {batch // nseq}; "
                      f"dense: {rows} of {sh.k} kept rows, scaled by {sh.k // rows}"}


def load_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary,
    valid only for the workload it was taken on and while the attention kernel
    source is the one it was taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("kernel_source_sha256_16") != _file_sha(ATTN_KERNEL_SOURCE):
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_CAL_ELEMS = 1 << 28  # fp32 elements: 1 GiB read + 1 GiB written per launch


def copy_calibration(torch, dev):
    """Three launches of a plain streaming kernel of known size (torch.neg on a
    1 GiB fp32 tensor into another): reads and writes exactly 2^30 bytes each."""
    src = torch.ones(COPY_CAL_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _pmc_per_dispatch(folder, counter, match):
    """Mean over dispatches of `counter` (summed over its rows) for kernels whose
    name contains `match`, from rocprofv3 csv counter-collection output."""
    import csv
    import glob
    per = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter or match not in r.get("Kernel_Name", ""):
                    continue
                key = (fn, r.get("Dispatch_Id"))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {match!r} under {folder}")
    return sum(per.values()) / len(per), len(per)


def _pmc_all_kernels(folder, counter):
    """{kernel name: (mean of `counter` per dispatch, dispatches)} over every
    kernel in rocprofv3 csv counter-collection output."""
    import csv
    import glob
    per = {}
    for fn in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                name = r.get("Kernel_Name", "").replace("(anonymous namespace)::", "").replace("void ", "")
                name = name.split("(")[0]
                key = (name, fn, r.get("Dispatch_Id"))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _, _), v in per.items():
        tot, cnt = out.get(name, (0.0, 0))
        out[name] = (tot + v, cnt + 1)
    return {k: (tot / cnt, cnt) for k, (tot, cnt) in out.items()}


def traffic_table(fetch_dir, write_dir, f_scale, w_scale):
    """Markdown rows: calibrated HBM read and write bytes per launch of every
    kernel seen by both counter passes."""
    fe = _pmc_all_kernels(fetch_dir, "FETCH_SIZE")
    wr = _pmc_all_kernels(write_dir, "WRITE_SIZE")
    rows = ["| Kernel | Launches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | Read (MB) | Write (MB) |",
            "|---|---|---|---|---|---|"]
    for name in sorted(set(fe) & set(wr), key=lambda k: -fe[k][0]):
        f_kib, nf = fe[name]
        w_kib, _ = wr[name]
        rows.append(f"| `{name}` | {nf} | {f_kib:.1f} | {w_kib:.1f} | {f_kib * 1024 * f_scale / 1e6:.2f} | "
                    f"{w_kib * 1024 * w_scale / 1e6:.2f} |")
    return "\n".join(rows)


def traffic_summary(fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel, each
    scaled by what the same counter reads for the 1 GiB calibration kernel."""
    true_bytes = COPY_CAL_ELEMS * 4
    f_attn, nf = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", "attn_bf16")
    w_attn, nw = _pmc_per_dispatch(write_dir, "WRITE_SIZE", "attn_bf16")
    f_cal, _ = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", "neg")
    w_cal, _ = _pmc_per_dispatch(write_dir, "WRITE_SIZE", "neg")
    f_scale = true_bytes / (f_cal * 1024.0)
    w_scale = true_bytes / (w_cal * 1024.0)
    fetch = f_attn * 1024.0 * f_scale
    write = w_attn * 1024.0 * w_scale
    from learned_token_pruning_03_amd.workloads import SHAPES
    sh = SHAPES["qwen1p7b_32k"]
    algo = stage_bytes(sh)["attn"]
    rec = {
        "kernel": "attn_bf16_pp_kernel<128, false>",
        "workload": "qwen1p7b_32k",
        "kernel_source_sha256_16": _file_sha(ATTN_KERNEL_SOURCE),
        "hbm_bytes_per_launch": round(fetch + write),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "algorithmic_bytes_per_launch": algo,
        "fetch_calibration": {"counter_kib_per_launch": f_cal, "true_bytes": true_bytes, "scale": f_scale},
        "write_calibration": {"counter_kib_per_launch": w_cal, "true_bytes": true_bytes, "scale": w_scale},
        "dispatches": {"fetch": nf, "write": nw},
    }
    print(traffic_table(fetch_dir, write_dir, f_scale, w_scale))
    return rec


def main(argv=None):
    args = parse_args(argv)
    if args.traffic_summary:
        rec = traffic_summary(*args.traffic_summary)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec, indent=1))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        return 2
    import torch

    import learned_token_pruning_03_amd as tg
    import learned_token_pruning_03_amd.workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    tg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    path = Path(tg, W, args.workload, dev, select=args.select)
    sh = path.sh
    print(f"[bench] workload {args.workload}: N={sh.n} K={sh.k} layers={sh.layers}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # One event pair around every attention launch of the timed region: the
    # roofline's launch duration is measured live, not in a separate loop.
    attn_ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(sh.layers)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        path.step(attn_ev[s])
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    attn_launch_us = [a.elapsed_time(b) * 1e3 for per_step in attn_ev for (a, b) in per_step]
    attn_avg_us = sum(attn_launch_us) / len(attn_launch_us)
    ms_per_step = ms_total / args.steps
    tokens_per_s = sh.n * args.steps / (ms_total / 1e3)
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    graph = graph_steps(torch, path, args.steps, args.warmup)
    print(f"[bench] HIP graph replay: {graph['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    med, mean = time_stages(path, args.stage_reps)
    print(f"[bench] stage medians in path (us): {json.dumps({k: round(v, 2) for k, v in med.items()})}",
          file=sys.stderr, flush=True)
    cold = cold_stages(path, max(3, args.stage_reps // 3))
    b2b = back_to_back(path)
    print(f"[bench] cold per launch (us): {json.dumps({k: round(v, 2) for k, v in cold.items()})}; "
          f"back to back: {json.dumps({k: round(v, 2) for k, v in b2b.items()})}", file=sys.stderr, flush=True)
    fl_attn = attn_flops(sh)
    fl_gate = gate_flops(sh)
    by = stage_bytes(sh)
    attn_tflops = fl_attn / (attn_avg_us * 1e-6) / 1e12
    traffic = load_traffic(args.workload)
    roofline = {
        "kernel": "attn_bf16_pp_kernel<128, false>",
        "bound": "mfma",
        "achieved": round(attn_tflops, 1),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "flops_per_launch": fl_attn,
        "avg_launch_us": round(attn_avg_us, 2),
        "launches_timed": len(attn_launch_us),
        "duration_basis": ("avg_launch_us: mean of the HIP event pairs around every attention launch of the timed "
                           "region (each pair also holds a few us of dispatch latency); avg_launch_us_back_to_back: "
                           "24 launches in a row between one pair, which is what the kernel trace measures"),
        "avg_launch_us_back_to_back": round(b2b["attn"], 2),
        "frac_back_to_back": round(fl_attn / (b2b["attn"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }
    stages = {}
    for n in list(med) + [x for x, _ in reference_fns(path) if x not in med]:
        e = {}
        if n in med:
            e["median_us"] = round(med[n], 2)
            e["mean_us"] = round(mean[n], 2)
            e["GB/s"] = round(by[n] / (med[n] * 1e-6) / 1e9, 1)
        else:
            e["in_path"] = False  # timed for reference only: the step runs the fused call
        e["cold_us"] = round(cold[n], 2)
        if n in b2b:
            e["us_back_to_back"] = round(b2b[n], 2)
            e["GB/s_back_to_back"] = round(by[n] / (b2b[n] * 1e-6) / 1e9, 1)
            e["back_to_back_cache"] = "warm" if n in ("attn", "select") else "cold"
        if n in ("gate", "gate_select", "prune") and n in b2b:
            e["TFLOP/s_back_to_back"] = round(fl_gate / (b2b[n] * 1e-6) / 1e12, 1)
        if n == "attn":
            e["TFLOP/s"] = round(fl_attn / (med[n] * 1e-6) / 1e12, 1)
        stages[n] = e

    def pct(name):
        return round(100 * by[name] / (b2b[name] * 1e-6) / 1e9 / PEAK_HBM_GBS, 2)

    pruning = None
    if path.fused:
        # The gate's own time (the plain gate kernel, same grid and main loop)
        # is taken out of the fused call: what is left is the ranking in the
        # gate's last workgroup plus the compaction-and-gather kernel.
        sel_gather = b2b["prune"] - b2b["gate"]
        pruning = {
            "prune_us": round(b2b["prune"], 2), "gate_us": round(b2b["gate"], 2),
            "gate_select_us": round(b2b["gate_select"], 2),
            "select_plus_gather_us": round(sel_gather, 2),
            "select_plus_gather_GB/s": round((by["select"] + by["gather"]) / (sel_gather * 1e-6) / 1e9, 1),
            "select_plus_gather_pct_hbm_peak": round(
                100 * (by["select"] + by["gather"]) / (sel_gather * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
            "standalone_gather_us": round(b2b["gather"], 2),
            "basis": "back-to-back launches on cold footprints; select_plus_gather = tg_gate_select_gather minus "
                     "the plain gate (the ranking in the gate's last workgroup plus the compaction + gather kernel)",
        }
    full = upper = stack = None
    if not args.no_full_context:
        print("[bench] timing one upper layer on the K kept tokens and on all N tokens ...", file=sys.stderr,
              flush=True)
        up_k = upper_layer(tg, W, sh, dev, sh.k, gated=True)
        up_n = upper_layer(tg, W, sh, dev, sh.n, gated=False)
        layer_gated = med["rope_kv"] + med["attn"]
        full = {"n": sh.n, "rope_kv_us": up_n["stage_us"]["rope_kv"], "attn_us": up_n["stage_us"]["attn"],
                "attn_TFLOP/s": up_n["attn_TFLOP/s"]}
        full["layer_us"] = round(full["rope_kv_us"] + full["attn_us"], 2)
        full["layer_speedup_vs_pruned"] = round(full["layer_us"] / layer_gated, 2)
        # One selection layer's overhead (gate, select, gather) is paid once per
        # prompt; every upper layer then runs on K tokens instead of N.
        full["pruning_overhead_us"] = round(sum(med[x] for x in med if x not in ("rope_kv", "attn")), 2)
        upper = {"ffn": FFN, "pruned": up_k, "full": up_n,
                 "layer_speedup_vs_pruned": round(up_n["total_us"] / up_k["total_us"], 2)}
    if not args.no_stack:
        print("[bench] timing the 28-layer stack, gated at layer 9 (N = 65536, K = 4096) ...", file=sys.stderr,
              flush=True)
        stack = stack_ratio(tg, W, dev)

    dec = None
    if not args.no_decode:
        print("[bench] timing decode attention over compact caches ...", file=sys.stderr, flush=True)
        dec = decode_step(tg, W, sh, dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(W, args.workload)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "n": sh.n, "k": sh.k, "q_len": sh.q_len, "d": sh.d,
                   "gate_hidden": sh.hidden, "hq": sh.hq, "hkv": sh.hkv, "dh": sh.dh,
                   "upper_layers": sh.layers, "global_batch": 1, "seq_len": sh.n},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prune_entry": "tg_gate_select_gather" if path.fused else "tg_gate_score + tg_select_topk_ws + tg_gather",
        "stages": stages,
        "pruning": pruning,
        "hip_graph": graph,
        "full_context": full,
        "upper_layer": upper,
        "stack": stack,
        "decode": dec,
        "attn_pct_mfma_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "gate_pct_hbm_peak": pct("gate"),
        "gather_pct_hbm_peak": pct("gather"),
        "rope_kv_pct_hbm_peak": pct("rope_kv"),
        "hbm_pct_basis": "algorithmic bytes over back-to-back launches on footprints last touched more than 256 MB "
                         "of traffic earlier (cold last-level cache)",
    }
    if args.copy_calibration:
        copy_calibration(torch, dev)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

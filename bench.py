#!/usr/bin/env python3
"""Decode-step throughput of the TokenSelect hot path on one MI355X.

Headline workload: one request at N = 1,048,576 cached tokens, Llama-3-8B layer
shapes (32 query / 8 KV heads, d = 128), bf16 paged pool (page 16, shuffled),
TopK 2048 united with 512 local tokens, 32 independent layers (seeds 2000 + l).
A step is one full decode step of one layer through tokenselect_decode_step:
cache check, paged scoring, per-head softmax, soft vote, radix TopK, sparse
attention. Every timed step reselects (theta = 2 forces a cache miss), and the
steps cycle through the 32 layers, so each step streams a different 2 GiB K pool.

Prints one JSON line: decode steps/s (value), the scoring kernel's achieved HBM
bandwidth against the 8 TB/s peak (roofline; roofline.ceiling adds a plain streaming
probe over the same K pools, read-only and with the scoring pass's 16:1 read/write
mix, as the achievable reference), the same metric at N = 131072
(secondary), the 16-request ragged batch (ragged_batch), the 256-step
Selection Cache sequence on Qwen2-7B shapes (selection_cache: steps/s, hit rate,
hit vector), chunk-wise prefill at 128K and 1M cached tokens with 512-token chunks
(prefill: chunks/s, selection GB/s, chunk-attention TFLOP/s against the bf16
matrix-core peak), the 1M decode step with the dynamic top-p budget (top_p: p = 0.9,
capped at k), the selection-function ablations at 128K (ablations: time from logits
to TopK and recall for the soft vote, naive TopK, head hard vote and block selection
at block sizes 2-128), and the fp64 oracle timed on host cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 matrix-core peak of MI355X


def log(msg):
    print(msg, file=sys.stderr, flush=True)


SCORE_SOURCES = ("score.hip", "cache.h", "common.h", "kernels.h", "timeline.h")


def score_source_digest() -> str:
    """sha256 over the score kernel's source files, in SCORE_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for name in SCORE_SOURCES:
        with open(os.path.join(ROOT, "token_level_sparse_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per scoring launch from the committed counter summary, or None.

    The summary records the sha256 of the score kernel's sources it was measured on;
    if they have changed since, the figure no longer describes the kernel.
    """
    path = os.path.join(ROOT, "profiles", "score_kernel_traffic_llama3-8b-1m.md")
    try:
        fields = {}
        for line in open(path):
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "score_source_sha256"):
                k, v = line.split(":", 1)
                fields[k] = v.strip()
        if fields.get("score_source_sha256") != score_source_digest():
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def score_bytes_per_token(geo) -> float:
    """Algorithmic bytes the scoring kernel moves per cached token.

    K rows of every KV head (H_kv * d * element size), the fp32 logits of every
    query head (H * 4) and the block-table entry shared by a page (4 / P).
    """
    esize = 4 if geo.dtype == "f32" else 2
    return geo.num_kv_heads * geo.head_dim * esize + geo.num_q_heads * 4 + 4.0 / geo.page_size


def kv_cache(geo, n_layers, dev):
    """The K and V page pools of all layers as two tensors [layer][pages][H_kv][P][d],
    allocated once up front the way a serving engine sizes its KV cache.

    The V pools are allocated first. A decode step streams all of K but reads only the
    selected rows of V (about 10 MB at 1M tokens), and on the MI355X boxes measured
    here the first ~90 GiB a fresh process allocates deliver ~10% less streaming
    bandwidth than the rest of the 288 GiB; allocating V first leaves more of the
    streamed K pools outside that region. Every layer is still generated and timed."""
    import torch
    pages = -(-geo.seq_len // geo.page_size) * geo.batch
    shp = (n_layers, pages, geo.num_kv_heads, geo.page_size, geo.head_dim)
    v = torch.empty(shp, dtype=geo.torch_dtype, device=dev)
    k = torch.empty(shp, dtype=geo.torch_dtype, device=dev)
    return k, v


class Layer:
    """Device buffers of one layer's request: paged pool, query, cache state."""

    def __init__(self, geo, layer, dev, keep_host=False, pools=None):
        import torch
        import token_level_sparse_amd as ts
        from synth import workloads as wl
        b = wl.make_batch(geo, device=dev, layer=layer, pools=pools)
        self.q, self.k_pool, self.v_pool = b.q, b.k_pool, b.v_pool
        self.block_table, self.seq_lens = b.block_table, b.seq_lens
        self.total = b.total_tokens
        self.host = None
        if keep_host:
            r = b.requests[0]
            self.host = tuple(x.float().cpu().numpy() for x in (r.q, r.k, r.v))
        del b
        H, d = geo.num_q_heads, geo.head_dim
        self.cache = ts.CacheState.allocate(1, H, d, geo.top_k, geo.torch_dtype, dev)
        self.hit = torch.zeros(1, dtype=torch.int32, device=dev)
        self.out = torch.empty(1, H, d, dtype=geo.torch_dtype, device=dev)


class StepCall:
    """One tokenselect_decode_step call with its ctypes arguments built once, so a timed
    loop of short steps spends its host time in the library call alone (the binding's
    per-call marshalling is tens of microseconds, as long as a Selection Cache hit step
    on the GPU)."""

    def __init__(self, shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache, hit, out, ws):
        import ctypes
        import torch
        import token_level_sparse_amd as ts
        self.fn = ts.load_library().tokenselect_decode_step
        self.cs = cache.c_struct()
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        self.args = (ctypes.byref(shape), ctypes.byref(sel), P(q), P(k_pool), P(v_pool), P(block_table),
                     P(seq_lens), ctypes.byref(self.cs), P(hit), P(out), P(ws), ws.numel(),
                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        self._keep = (shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache, hit, out, ws)

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            raise RuntimeError(f"tokenselect_decode_step failed ({rc})")


def stream_ceiling(pools, steps, dev):
    """Time the streaming-bandwidth probe (libts_stream_probe.so) over the same K
    pools the scoring launches read: a plain read of each pool, and the same read
    with 1 byte written per 16 read (the scoring pass's K : logits mix at these
    head counts). Returns GB/s of bytes moved, or None without the probe library."""
    import ctypes
    import torch
    from token_level_sparse_amd import build as tb
    if not os.path.exists(tb.PROBE_LIB):
        log("[ceiling] libts_stream_probe.so not built; no ceiling figures")
        return None
    lib = ctypes.CDLL(tb.PROBE_LIB)
    f = lib.ts_stream_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    nbytes = pools[0].numel() * pools[0].element_size()
    dst = torch.empty(nbytes // 16, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for write in (0, 1):
        def launch(s):
            P = pools[s % len(pools)]
            rc = f(ctypes.c_void_p(P.data_ptr()), nbytes, ctypes.c_void_p(dst.data_ptr()), write, 2048,
                   ctypes.c_void_p(sink.data_ptr()), st)
            if rc != 0:
                raise RuntimeError(f"ts_stream_probe failed ({rc})")
        for s in range(4):
            launch(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(steps):
            launch(s)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        moved = nbytes + (nbytes // 16 if write else 0)
        res["read_plus_1_16_write" if write else "read_only"] = dict(ms=ms, gbps=moved / (ms * 1e-3) / 1e9)
    del dst
    log(f"[ceiling] probe over the same pools: read {res['read_only']['ms']:.4f} ms "
        f"({res['read_only']['gbps']:.0f} GB/s), read + 1/16 write {res['read_plus_1_16_write']['ms']:.4f} ms "
        f"({res['read_plus_1_16_write']['gbps']:.0f} GB/s)")
    return res


def phase_probe(dev):
    """Time the chunk-attention phase probe (ts_chunk_phase_probe in
    libts_stream_probe.so): the instruction mix of one phase of the bf16 chunk
    attention's block loop repeated on LDS-resident data, 256 workgroups of 8 waves (two
    per SIMD), no staging and no barriers. Prints a markdown table: wave time per loop
    iteration and SIMD cycles per phase (at 2.4 GHz; each SIMD runs two waves, each
    doing two phases per iteration)."""
    import ctypes
    import numpy as np
    import torch
    from token_level_sparse_amd import build as tb
    lib = ctypes.CDLL(tb.PROBE_LIB)
    f = lib.ts_chunk_phase_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    grid, iters = 256, 64
    g = torch.Generator().manual_seed(7)
    src = (torch.rand(2560 * 8, generator=g) * 0.05).to(torch.bfloat16).to(dev)
    out = torch.empty(grid * 512, dtype=torch.float32, device=dev)
    times = torch.zeros(grid * 16, dtype=torch.int64, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    names = {0: "EXP: 16 MFMA (next scores) + 32 exp2 of this block, K reads",
             1: "PV: 16 MFMA + 32 transposed V reads + 16 cvt",
             2: "EXP then PV (waves 0-3) / PV then EXP (waves 4-7)",
             3: "EXP without exp2 (fma argument only)",
             4: "EXP without MFMA (one add per product)"}
    print("| mode | phase mix | wave time per iteration p50 / p90 (ns) | SIMD cycles per phase at 2.4 GHz |")
    print("|---|---|---|---|")
    for mode in range(5):
        for rep in range(2):
            rc = f(mode, iters, grid, ctypes.c_void_p(src.data_ptr()), src.numel() * 2, ctypes.c_void_p(out.data_ptr()),
                   ctypes.c_void_p(times.data_ptr()), st)
            if rc != 0:
                raise RuntimeError(f"ts_chunk_phase_probe failed ({rc})")
            torch.cuda.synchronize()
        t = times.cpu().numpy().reshape(-1, 2)
        per_it = (t[:, 1] - t[:, 0]) * 10.0 / iters
        p50, p90 = np.percentile(per_it, [50, 90])
        # per iteration a SIMD runs 2 waves x 2 phases
        print(f"| {mode} | {names[mode]} | {p50:.0f} / {p90:.0f} | {p50 * 2.4 / 4:.0f} |")
    print("(a v_mfma_f32_32x32x16_bf16 occupies the matrix core 32 cycles, so 16 of them take 512 cycles)")


def time_workload(geo, n_layers, steps, warmup, dev, keep_host=False, ceiling=False, then=None):
    """Decode steps over n_layers rotating layers, then the score launches alone
    (and the streaming probe with ceiling=True); `then(layers)`, if given, runs on
    the same layers before they are freed and its result is returned as res["then"]."""
    import torch
    import token_level_sparse_amd as ts
    t0 = time.time()
    KC, VC = kv_cache(geo, n_layers, dev)
    layers = [Layer(geo, l, dev, keep_host and l == 0, (KC[l], VC[l])) for l in range(n_layers)]
    torch.cuda.synchronize()
    log(f"[{geo.name}] generated {n_layers} layers in {time.time() - t0:.1f}s")
    L0 = layers[0]
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, 1, L0.block_table.shape[1], L0.total,
                          geo.torch_dtype)
    # theta = 2 > any cosine: every step reselects (a full miss step)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 2.0)
    ws = ts.alloc_workspace(shape, sel, dev)

    calls = [StepCall(shape, sel, L.q, L.k_pool, L.v_pool, L.block_table, L.seq_lens, L.cache,
                      L.hit, L.out, ws) for L in layers]

    def step(s):
        calls[s % n_layers]()

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        step(s)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / steps
    # the spread: each step of a second pass between its own events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s, (a, b) in enumerate(evs):
        a.record()
        step(s)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    pct = {q: per[min(len(per) - 1, int(q / 100 * len(per)))] for q in (10, 50, 90)}
    log(f"[{geo.name}] decode step {ms_step:.4f} ms (wall {wall / steps * 1e3:.4f} ms; per step "
        f"p10 {pct[10]:.4f} p50 {pct[50]:.4f} p90 {pct[90]:.4f} ms)")

    # the scoring kernel alone (tokenselect_score with head_stats NULL: one kernel), timed
    # per launch on the same stream; then the full tokenselect_score launch (that kernel
    # plus the small kernel folding the per-unit softmax pairs) for reference
    H = geo.num_q_heads
    logits = torch.empty(H * L0.total, dtype=torch.float32, device=dev)
    stats = torch.empty(H * 2, dtype=torch.float32, device=dev)

    def time_score(st):
        for s in range(min(warmup, 4)):
            L = layers[s % n_layers]
            ts.score(shape, sel, L.q, L.k_pool, L.block_table, L.seq_lens, logits, st, ws)
        torch.cuda.synchronize()
        evs = []
        for s in range(steps):
            L = layers[s % n_layers]
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ts.score(shape, sel, L.q, L.k_pool, L.block_table, L.seq_lens, logits, st, ws)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    score_ms = time_score(None)
    launch_ms = time_score(stats)
    algo = score_bytes_per_token(geo) * L0.total
    kbytes = geo.num_kv_heads * geo.head_dim * (2 if geo.dtype == "bf16" else 4) * L0.total
    res = dict(ms_per_step=ms_step, wall_ms_per_step=wall / steps * 1e3,
               step_ms_p10=pct[10], step_ms_p50=pct[50], step_ms_p90=pct[90], score_ms=score_ms,
               score_with_stats_ms=launch_ms,
               score_gbps=algo / (score_ms * 1e-3) / 1e9, k_gbps=kbytes / (score_ms * 1e-3) / 1e9,
               score_bytes=algo, tokens=L0.total)
    log(f"[{geo.name}] score kernel {score_ms:.4f} ms -> {res['score_gbps']:.0f} GB/s "
        f"(K stream {res['k_gbps']:.0f} GB/s); with the statistics kernel {launch_ms:.4f} ms")
    if ceiling:
        res["ceiling"] = stream_ceiling([L.k_pool for L in layers], steps, dev)
    if then is not None:
        res["then"] = then(layers)
    host = L0.host
    del calls, layers, ws, logits, KC, VC
    torch.cuda.empty_cache()
    return res, host


def time_topp(geo, n_layers, steps, warmup, dev, top_p=0.9, layers=None):
    """Decode steps with the dynamic top-p budget (ts_select.top_p) instead of the
    fixed TopK, every step reselecting; reports steps/s and the mean budget. Given
    `layers` (the headline's, same workload), it runs on their first n_layers pools,
    so both figures come from the same memory."""
    import torch
    import token_level_sparse_amd as ts
    KC = VC = None
    if layers is None:
        KC, VC = kv_cache(geo, n_layers, dev)
        layers = [Layer(geo, l, dev, False, (KC[l], VC[l])) for l in range(n_layers)]
    else:
        layers = layers[:n_layers]
    L0 = layers[0]
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, 1, L0.block_table.shape[1], L0.total,
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 2.0, top_p)
    ws = ts.alloc_workspace(shape, sel, dev)

    calls = [StepCall(shape, sel, L.q, L.k_pool, L.v_pool, L.block_table, L.seq_lens, L.cache,
                      L.hit, L.out, ws) for L in layers]

    def step(s):
        calls[s % n_layers]()

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        step(s)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    budgets = [int(L.cache.cached_count[0]) for L in layers]
    log(f"[{geo.name}] top-p {top_p}: decode step {ms:.4f} ms, mean budget {sum(budgets) / len(budgets):.1f}")
    res = {"workload": geo.name, "top_p": top_p, "top_k_cap": geo.top_k, "layers": n_layers,
           "decode_steps_per_s": 1e3 / ms, "ms_per_step": ms,
           "mean_budget": sum(budgets) / len(budgets), "budgets": budgets}
    del calls, layers, ws, KC, VC
    torch.cuda.empty_cache()
    return res


def time_ablations(geo, dev, reps=10):
    """Selection-function ablations on one layer: time from logits to TopK for the
    head soft vote, the naive TopK, the head hard vote and block selection; recall of
    the planted critical tokens and of the soft-vote TopK (recall vs granularity)."""
    import numpy as np
    import torch
    import token_level_sparse_amd as ts
    from synth import workloads as wl
    batch = wl.make_batch(geo, device=dev)
    H, total = geo.num_q_heads, batch.total_tokens
    shape = ts.make_shape(H, geo.num_kv_heads, 1, batch.block_table.shape[1], total, geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale)
    ws = ts.alloc_workspace(shape, sel, dev)
    logits = torch.empty(H * total, dtype=torch.float32, device=dev)
    stats = torch.empty(H * 2, dtype=torch.float32, device=dev)
    ts.score(shape, sel, batch.q, batch.k_pool, batch.block_table, batch.seq_lens, logits, stats, ws)
    planted = np.unique(batch.requests[0].planted_pos.cpu().numpy())
    si = torch.empty(1, geo.top_k, dtype=torch.int32, device=dev)
    sc = torch.empty(1, dtype=torch.int32, device=dev)
    runs = [("soft_vote", ts.SELECT_SOFT_VOTE, 1), ("naive_topk", ts.SELECT_NAIVE_TOPK, 1),
            ("hard_vote", ts.SELECT_HARD_VOTE, 1)] + [(f"block_{B}", ts.SELECT_BLOCK, B) for B in (2, 4, 8, 16, 32, 64, 128)]
    res, soft = {}, None
    for name, fn, B in runs:
        aws = ts.alloc_ablation_workspace(shape, sel, fn, B, dev)
        call = lambda: ts.select_ablation(shape, sel, fn, B, logits, stats, batch.seq_lens, None, si, sc, aws)
        call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(); call(); b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        T = si[0, : int(sc[0])].cpu().numpy()
        if soft is None:
            soft = T
        res[name] = {"ms": ms, "selected": int(len(T)),
                     "planted_recall": float(np.isin(planted, T).mean()),
                     "recall_of_soft_vote_topk": float(np.isin(soft, T).mean())}
        del aws
    log(f"[{geo.name}] ablations: " + ", ".join(f"{k} {v['ms']:.3f} ms planted {v['planted_recall']:.3f} "
                                                 f"soft-recall {v['recall_of_soft_vote_topk']:.3f}" for k, v in res.items()))
    del batch, ws, logits
    torch.cuda.empty_cache()
    return {"workload": geo.name, "N": total, "top_k": geo.top_k, "selectors": res}


def time_score_launches(shape, sel, b, H, B, reps, dev, ws):
    """Mean time of tokenselect_score launches (score + stats kernels) over a batch,
    launched back to back between two events on the current stream."""
    import torch
    import token_level_sparse_amd as ts
    logits = torch.empty(H * b.total_tokens, dtype=torch.float32, device=dev)
    stats = torch.empty(B * H * 2, dtype=torch.float32, device=dev)
    ts.score(shape, sel, b.q, b.k_pool, b.block_table, b.seq_lens, logits, stats, ws)
    torch.cuda.synchronize()
    # back to back between two events: a host stall while the queue still holds work
    # does not enter the figure
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        ts.score(shape, sel, b.q, b.k_pool, b.block_table, b.seq_lens, logits, stats, ws)
    e.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / reps
    del logits, stats
    return ms


def time_ragged(geo, steps, warmup, dev):
    """Ragged batch: 16 requests in one shared shuffled pool, one launch per kernel per step."""
    import torch
    import token_level_sparse_amd as ts
    from synth import workloads as wl
    b = wl.make_batch(geo, device=dev)
    B, H, d = geo.batch, geo.num_q_heads, geo.head_dim
    shape = ts.make_shape(H, geo.num_kv_heads, B, b.block_table.shape[1], b.total_tokens, geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 2.0)
    ws = ts.alloc_workspace(shape, sel, dev)
    cache = ts.CacheState.allocate(B, H, d, geo.top_k, geo.torch_dtype, dev)
    hit = torch.zeros(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, H, d, dtype=geo.torch_dtype, device=dev)

    step = StepCall(shape, sel, b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens, cache, hit, out, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kbytes = geo.num_kv_heads * geo.head_dim * 2 * b.total_tokens
    score_ms = time_score_launches(shape, sel, b, H, B, steps, dev, ws)
    algo = score_bytes_per_token(geo) * b.total_tokens
    log(f"[{geo.name}] batch of {B}, sum N = {b.total_tokens}: decode step {ms:.4f} ms; score launch "
        f"{score_ms:.4f} ms -> {algo / (score_ms * 1e-3) / 1e9:.0f} GB/s")
    res = {"workload": geo.name, "batch": B, "total_tokens": b.total_tokens,
           "decode_steps_per_s": 1e3 / ms, "ms_per_step": ms,
           "k_stream_gbps_whole_step": kbytes / (ms * 1e-3) / 1e9,
           "score_ms": score_ms, "score_bytes": algo, "score_gbps": algo / (score_ms * 1e-3) / 1e9,
           "score_frac_of_peak": algo / (score_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "score_what": "one tokenselect_score launch over the whole batch (about 3.7 GB of K, "
                         "beyond the 256 MB MALL)"}
    del step, b, ws
    torch.cuda.empty_cache()
    return res


def time_cache_sequence(geo, dev):
    """Consecutive decode steps with the Selection Cache: N grows by one token per
    step, queries follow the AR(1) recursion, theta = 0.9. The whole sequence is
    timed once after one untimed pass (the cache is reset in between)."""
    import torch
    import token_level_sparse_amd as ts
    from synth import workloads as wl
    steps = geo.steps
    gen = torch.Generator(device=dev).manual_seed(geo.seed)
    req = wl.make_request(gen, geo, geo.seq_len, dev, extra_tokens=steps - 1)
    batch = wl.page_requests([req], geo, gen, dev)
    qs, _ = wl.ar1_queries(geo, req.q_master, steps, seed=geo.seed + 1, device=dev)
    qs = [qs[t:t + 1].contiguous() for t in range(steps)]
    lens = torch.arange(geo.seq_len, geo.seq_len + steps, dtype=torch.int32, device=dev)
    lens = [lens[t:t + 1] for t in range(steps)]
    H, d = geo.num_q_heads, geo.head_dim
    shape = ts.make_shape(H, geo.num_kv_heads, 1, batch.block_table.shape[1], geo.seq_len + steps - 1,
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, geo.cos_threshold)
    ws = ts.alloc_workspace(shape, sel, dev)
    cache = ts.CacheState.allocate(1, H, d, geo.top_k, geo.torch_dtype, dev)
    hits = torch.zeros(steps, dtype=torch.int32, device=dev)
    out = torch.empty(1, H, d, dtype=geo.torch_dtype, device=dev)

    calls = [StepCall(shape, sel, qs[t], batch.k_pool, batch.v_pool, batch.block_table, lens[t],
                      cache, hits[t:t + 1], out, ws) for t in range(steps)]

    def run():
        for c in calls:
            c()

    run()
    torch.cuda.synchronize()
    cache.valid.zero_()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    hv = hits.cpu().tolist()
    # untimed third pass: how much of each reselected TopK the previous one already held
    cache.valid.zero_()
    snaps = []
    for t in range(steps):
        ts.decode_step(shape, sel, qs[t], batch.k_pool, batch.v_pool, batch.block_table, lens[t],
                       cache, hits[t:t + 1], out, ws)
        snaps.append((cache.cached_idx.clone(), cache.cached_count.clone()))
    torch.cuda.synchronize()
    hv3 = hits.cpu().tolist()
    miss_sets = [set(snaps[t][0][0, :int(snaps[t][1][0])].tolist()) for t in range(steps) if hv3[t] == 0]
    overlaps = [len(a & b) / max(1, len(b)) for a, b in zip(miss_sets, miss_sets[1:])]
    overlap = sum(overlaps) / len(overlaps) if overlaps else None
    # untimed fourth pass, each step between its own events: hit and miss steps apart
    cache.valid.zero_()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for t, (a, e) in enumerate(evs):
        a.record()
        calls[t]()
        e.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(e) for a, e in evs]
    hit_ms = [x for x, h in zip(per, hv) if h]
    miss_ms = [x for x, h in zip(per, hv) if not h]
    # the scoring pass of a miss step at the first step's length: K is 128 MiB, which the
    # 256 MB MALL holds across steps, so its bandwidth is an effective (cache-assisted) one
    from types import SimpleNamespace
    b1 = SimpleNamespace(q=qs[0], k_pool=batch.k_pool, block_table=batch.block_table, seq_lens=lens[0],
                         total_tokens=geo.seq_len + steps - 1)
    score_ms = time_score_launches(shape, sel, b1, H, 1, 32, dev, ws)
    algo = score_bytes_per_token(geo) * geo.seq_len
    log(f"[{geo.name}] {steps} steps: {ms:.4f} ms/step, hit rate {sum(hv) / steps:.3f}, "
        f"mean overlap of consecutive reselections {overlap if overlap is None else round(overlap, 4)}; "
        f"hit steps {sum(hit_ms) / max(1, len(hit_ms)):.4f} ms, miss steps {sum(miss_ms) / max(1, len(miss_ms)):.4f} ms; "
        f"score launch {score_ms:.4f} ms")
    res = {"workload": geo.name, "steps": steps, "decode_steps_per_s": 1e3 / ms, "ms_per_step": ms,
           "hit_rate": sum(hv) / steps, "hits": "".join(str(h) for h in hv),
           "miss_topk_overlap": overlap, "same_hits_on_rerun": hv3 == hv,
           "hit_step_ms": sum(hit_ms) / max(1, len(hit_ms)), "miss_step_ms": sum(miss_ms) / max(1, len(miss_ms)),
           "score_ms": score_ms, "score_bytes": algo,
           "score_gbps_effective": algo / (score_ms * 1e-3) / 1e9,
           "score_frac_of_peak_effective": algo / (score_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "score_what": "effective: tokenselect_score over the sequence's first step (N = 131072, "
                         "128 MiB of K, held by the 256 MB MALL between launches)"}
    del calls, batch, ws
    torch.cuda.empty_cache()
    return res


def time_dense(geo, decode_ms, read_gbps, dev, reps=10):
    """Dense attention at the workload's N for reference. Timed: the sparse attention
    kernel with every position selected (k = N), which reads all of K and V of one
    layer; it is built for gathers, not for a dense stream, so the fair reference is
    the bound: K + V bytes at the measured plain-read bandwidth (read_gbps)."""
    import torch
    import token_level_sparse_amd as ts
    KC, VC = kv_cache(geo, 1, dev)
    L = Layer(geo, 0, dev, False, (KC[0], VC[0]))
    N, H = L.total, geo.num_q_heads
    shape = ts.make_shape(H, geo.num_kv_heads, 1, L.block_table.shape[1], N, geo.torch_dtype)
    sel = ts.make_select(N, geo.n_local, 1.0, geo.attn_scale, 2.0)
    ws = ts.alloc_workspace(shape, sel, dev)
    idx = torch.arange(N, dtype=torch.int32, device=dev).reshape(1, N)
    cnt = torch.full((1,), N, dtype=torch.int32, device=dev)
    out = torch.empty(1, H, geo.head_dim, dtype=geo.torch_dtype, device=dev)

    def run():
        ts.sparse_attn(shape, sel, L.q, L.k_pool, L.v_pool, L.block_table, L.seq_lens, idx, cnt, out, ws)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    kv_bytes = 2 * geo.num_kv_heads * geo.head_dim * (2 if geo.dtype == "bf16" else 4) * N
    bound_ms = kv_bytes / (read_gbps * 1e9) * 1e3 if read_gbps else None
    log(f"[{geo.name}] dense attention over all {N} positions: sparse kernel with k = N {ms:.4f} ms "
        f"({kv_bytes / (ms * 1e-3) / 1e9:.0f} GB/s of K+V); K+V at the plain-read bandwidth "
        f"{bound_ms if bound_ms is None else round(bound_ms, 4)} ms; decode step {decode_ms:.4f} ms")
    res = {"workload": geo.name, "N": N, "kv_bytes": kv_bytes,
           "sparse_kernel_k_eq_n_ms": ms, "sparse_kernel_k_eq_n_gbps": kv_bytes / (ms * 1e-3) / 1e9,
           "dense_bound_ms": bound_ms,
           "decode_step_vs_dense_bound": (bound_ms / decode_ms) if bound_ms else None,
           "what": "dense attention reference for one decode step at this N: the bound is all of "
                   "K and V read at the plain streaming bandwidth measured on the same box "
                   "(roofline.ceiling.read_only_gbps); the ratio compares it with one whole "
                   "TokenSelect decode step, selection included"}
    del L, ws, KC, VC
    torch.cuda.empty_cache()
    return res


def time_prefill(geo, n_layers, steps, warmup, dev):
    """Chunk-wise prefill: one chunk of c queries per step over rotating layers
    (tokenselect_prefill_chunk: mean query, selection over the past, chunk attention).
    The chunk attention and the selection are also timed per launch on the same
    stream; the attention's algorithmic FLOPs are 4 d H sum_j |S_j| (two products of
    d multiply-adds per attended key, query and head)."""
    import torch
    import token_level_sparse_amd as ts
    from synth import workloads as wl
    t0 = time.time()
    KC, VC = kv_cache(geo, n_layers, dev)
    cbs = [wl.make_chunk_batch(geo, dev, layer=l, pools=(KC[l], VC[l])) for l in range(n_layers)]
    torch.cuda.synchronize()
    log(f"[{geo.name}] generated {n_layers} layers in {time.time() - t0:.1f}s")
    H, d, c = geo.num_q_heads, geo.head_dim, geo.chunk
    N = geo.seq_len
    P = N - c
    shape = ts.make_shape(H, geo.num_kv_heads, 1, cbs[0].paged.block_table.shape[1], N, geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 2.0)
    ws = ts.alloc_prefill_workspace(shape, sel, c, dev)
    sel_idx = [torch.empty(1, geo.top_k, dtype=torch.int32, device=dev) for _ in range(n_layers)]
    sel_count = [torch.empty(1, dtype=torch.int32, device=dev) for _ in range(n_layers)]
    out = torch.empty(1, c, H, d, dtype=geo.torch_dtype, device=dev)

    def chunk(s):
        cb, l = cbs[s % n_layers], s % n_layers
        ts.prefill_chunk(shape, sel, c, cb.q_chunk, cb.chunk_lens, cb.paged.k_pool, cb.paged.v_pool,
                         cb.paged.block_table, cb.seq_lens, sel_idx[l], sel_count[l], out, ws)

    def timed(fn, n):
        evs = []
        for s in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(s)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n

    for s in range(max(warmup, n_layers)):
        chunk(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        chunk(s)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps

    def attn(s):
        cb, l = cbs[s % n_layers], s % n_layers
        ts.chunk_attn(shape, sel, c, cb.q_chunk, cb.chunk_lens, cb.paged.k_pool, cb.paged.v_pool,
                      cb.paged.block_table, cb.seq_lens, sel_idx[l], sel_count[l], out, ws)

    def select(s):
        cb, l = cbs[s % n_layers], s % n_layers
        ts.prefill_select(shape, sel, c, cb.q_chunk, cb.chunk_lens, cb.paged.k_pool, cb.paged.block_table,
                          cb.seq_lens, None, None, None, sel_idx[l], sel_count[l], ws)

    attn_ms = timed(attn, steps)
    select_ms = timed(select, steps)
    # attended keys of every chunk query: base + j + 1, base = |T below the window| + (P - w0)
    w0 = max(0, P - geo.n_local)
    flops = 0.0
    for l in range(n_layers):
        T = sel_idx[l][0, : int(sel_count[l][0])].cpu()
        base = int((T < w0).sum()) + (P - w0)
        flops += 4.0 * d * H * (c * base + c * (c + 1) / 2)
    flops /= n_layers
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    sel_bytes = score_bytes_per_token(geo) * P
    log(f"[{geo.name}] chunk of {c}: {ms:.4f} ms ({c * 1e3 / ms:.0f} prefill tokens/s); "
        f"selection {select_ms:.4f} ms ({sel_bytes / (select_ms * 1e-3) / 1e9:.0f} GB/s), "
        f"chunk attention {attn_ms:.4f} ms ({attn_tflops:.1f} TFLOP/s)")
    res = {"workload": geo.name, "N": N, "chunk": c, "top_k": geo.top_k, "n_local": geo.n_local,
           "layers": n_layers, "ms_per_chunk": ms, "chunks_per_s": 1e3 / ms,
           "prefill_tokens_per_s": c * 1e3 / ms, "select_ms": select_ms,
           "select_gbps": sel_bytes / (select_ms * 1e-3) / 1e9, "attn_ms": attn_ms,
           "attn_flops": flops, "attn_tflops": attn_tflops,
           "attn_mfma_frac": attn_tflops / PEAK_BF16_TFLOPS}
    del cbs, ws, KC, VC
    torch.cuda.empty_cache()
    return res


def counter_run(geo, dev, launches=4, layers=4):
    """Short program for rocprofv3 --pmc passes: a few scoring launches on the 1M
    workload, then a plain device copy of 1 GiB (the calibration kernel whose true
    traffic is known: 1 GiB read, 1 GiB written)."""
    import torch
    import token_level_sparse_amd as ts
    KC, VC = kv_cache(geo, layers, dev)
    Ls = [Layer(geo, l, dev, pools=(KC[l], VC[l])) for l in range(layers)]
    L0 = Ls[0]
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, 1, L0.block_table.shape[1], L0.total,
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 2.0)
    ws = ts.alloc_workspace(shape, sel, dev)
    logits = torch.empty(geo.num_q_heads * L0.total, dtype=torch.float32, device=dev)
    stats = torch.empty(geo.num_q_heads * 2, dtype=torch.float32, device=dev)
    for s in range(launches):
        L = Ls[s % layers]
        ts.score(shape, sel, L.q, L.k_pool, L.block_table, L.seq_lens, logits, stats, ws)
    torch.cuda.synchronize()
    del Ls, ws, logits, KC, VC
    torch.cuda.empty_cache()
    x = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    for _ in range(launches):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"[counters] {launches} score launches and {launches} 1 GiB copies done")


def _host(t):
    return t.float().cpu().numpy()


def kernel_counter_run(dev, steps=4):
    """Short program for rocprofv3 --pmc passes over the decode-step kernels and the
    chunk attention: decode steps on the 128K workload (every step reselects), then
    prefill chunks of 512 queries at 128K; no timing."""
    import torch
    import token_level_sparse_amd as ts
    from synth import workloads as wl
    geo = wl.workload("llama3-8b-128k")
    KC, VC = kv_cache(geo, 2, dev)
    layers = [Layer(geo, l, dev, pools=(KC[l], VC[l])) for l in range(2)]
    L0 = layers[0]
    shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, 1, L0.block_table.shape[1], L0.total,
                          geo.torch_dtype)
    sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, 2.0)
    ws = ts.alloc_workspace(shape, sel, dev)
    for s in range(steps + 1):
        L = layers[s % 2]
        ts.decode_step(shape, sel, L.q, L.k_pool, L.v_pool, L.block_table, L.seq_lens, L.cache, L.hit,
                       L.out, ws)
    torch.cuda.synchronize()
    del layers, ws, KC, VC
    torch.cuda.empty_cache()
    g = wl.workload("prefill-llama3-128k")
    KC, VC = kv_cache(g, 1, dev)
    cb = wl.make_chunk_batch(g, dev, layer=0, pools=(KC[0], VC[0]))
    shape = ts.make_shape(g.num_q_heads, g.num_kv_heads, 1, cb.paged.block_table.shape[1], g.seq_len,
                          g.torch_dtype)
    sel = ts.make_select(g.top_k, g.n_local, 1.0, g.attn_scale, 2.0)
    ws = ts.alloc_prefill_workspace(shape, sel, g.chunk, dev)
    si = torch.empty(1, g.top_k, dtype=torch.int32, device=dev)
    sc = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty(1, g.chunk, g.num_q_heads, g.head_dim, dtype=g.torch_dtype, device=dev)
    for _ in range(steps + 1):
        ts.prefill_chunk(shape, sel, g.chunk, cb.q_chunk, cb.chunk_lens, cb.paged.k_pool, cb.paged.v_pool,
                         cb.paged.block_table, cb.seq_lens, si, sc, out, ws)
    torch.cuda.synchronize()
    log(f"[kernel counters] {steps + 1} decode steps at 128K and {steps + 1} prefill chunks done")


TIMELINE_KERNELS = {("score", 0): "score_kernel", ("score", 1): "stats_kernel", ("select", 2): "vote_kernel",
                    ("select", 3): "refine digit 1", ("select", 4): "refine digit 2", ("select", 6): "write",
                    ("attn", 8): "attn_kernel", ("attn", 9): "combine_kernel", ("prefill", 7): "chunk_attn_bf16"}


def timeline_run(dev, reps=5):
    """Per-wave timeline (libtokenselect_timeline.so, the kernels built with the wall-clock
    records of csrc/timeline.h): the kernels of one decode step, one after another,
    with the gaps between them, at 128K (a miss step and a Selection Cache hit step),
    on the 28/4-head 128K geometry of the cache sequence (miss and hit) and at 1M;
    the 128K scoring launch without the cache (tokenselect_score; one dispatch round
    of workgroups) split into dispatch ramp, request tables, stream and tail, and the
    wave time the decode step's score kernel adds; and the 128K prefill chunk attention.
    Medians over `reps` launches; prints a markdown report."""
    import ctypes
    import numpy as np
    import torch
    import token_level_sparse_amd as ts
    from token_level_sparse_amd import build as tb
    from synth import workloads as wl
    if not os.path.exists(tb.TIMELINE_LIB):
        log("[timeline] libtokenselect_timeline.so not built")
        return
    lib = ts.load_library(tb.TIMELINE_LIB)
    tus = ("score", "select", "attn", "prefill")
    for t in tus:
        getattr(lib, f"ts_timeline_read_{t}").argtypes = [ctypes.c_void_p]
    KT, KW, KWD = 10, 16384, 10
    us = lambda x: x * 0.01                                     # s_memrealtime ticks (100 MHz) -> us
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def capture(fn):
        for t in tus:
            assert getattr(lib, f"ts_timeline_clear_{t}")() == 0
        torch.cuda.synchronize()
        fn()
        torch.cuda.synchronize()
        recs = {}
        for t in tus:
            buf = np.zeros(KT * KW * KWD, dtype=np.uint64)
            assert getattr(lib, f"ts_timeline_read_{t}")(ctypes.c_void_p(buf.ctypes.data)) == 0
            buf = buf.reshape(KT, KW, KWD)
            for k in range(KT):
                v = buf[k][buf[k][:, 9] == 1]
                if len(v) and (t, k) in TIMELINE_KERNELS:
                    recs[TIMELINE_KERNELS[(t, k)]] = v.astype(np.int64)
        return recs

    def kernel_rows(runs):
        """Median over runs of each kernel's first entry, entry spread, span, wave
        duration p50 / p90, last exit, relative to the first kernel's first entry."""
        rows = {}
        for recs in runs:
            t0 = min(v[:, 0].min() for v in recs.values())
            for name, v in recs.items():
                ent, ex = v[:, 0] - t0, v[:, 1] - t0
                dur = v[:, 1] - v[:, 0]
                rows.setdefault(name, []).append((ent.min(), ent.max() - ent.min(), ex.max() - ent.min(),
                                                  np.median(dur), np.percentile(dur, 90), ex.max(), len(v),
                                                  np.median(ex)))
        out = []
        for name, vals in sorted(rows.items(), key=lambda kv: np.median([x[0] for x in kv[1]])):
            a = np.array(vals, dtype=np.float64)
            out.append((name, *np.median(a, axis=0)))
        return out

    def print_step(title, runs):
        rows = kernel_rows(runs)
        print(f"\n### {title}\n")
        print("| kernel | waves | first entry µs | entry spread µs | span µs | wave p50 µs | wave p90 µs | gap before µs |")
        print("|---|---|---|---|---|---|---|---|")
        prev = None
        for name, first, spread, span, d50, d90, last, nw, ex50 in rows:
            gap = "" if prev is None else f"{us(first - prev):.2f}"
            print(f"| {name} | {int(nw)} | {us(first):.2f} | {us(spread):.2f} | {us(span):.2f} | {us(d50):.2f} | "
                  f"{us(d90):.2f} | {gap} |")
            prev = last
        print(f"\nstep (first entry to last exit): {us(max(r[6] for r in rows)):.2f} µs; kernel time "
              f"{us(sum(r[3] for r in rows)):.2f} µs, gaps {us(max(r[6] for r in rows) - sum(r[3] for r in rows)):.2f} µs")

    def score_split(title, runs_nc, runs_c):
        """tokenselect_score without the cache (runs_nc) and the decode step's score
        kernel with it (runs_c, a miss step)."""
        def stats(runs):
            vals = []
            for recs in runs:
                v = recs["score_kernel"]
                ent = v[:, 0] - v[:, 0].min()
                ex = v[:, 1] - v[:, 0].min()
                tables = v[:, 2] - v[:, 0]
                vals.append((ent.max(), np.median(ent), np.median(tables), np.median(v[:, 1] - v[:, 2]),
                             np.median(ex), ex.max()))
            return np.median(np.array(vals, dtype=np.float64), axis=0)
        ramp, ent50, tables, rest, ex50, span = stats(runs_nc)
        _, _, tables_c, rest_c, _, span_c = stats(runs_c)
        print(f"\n### scoring launch split, {title}\n")
        print("| part | µs |\n|---|---|")
        print(f"| dispatch ramp: last wave entry after the first (median entry {us(ent50):.2f}) | {us(ramp):.2f} |")
        print(f"| request tables (entry to tables ready, wave median) | {us(tables):.2f} |")
        print(f"| stream: tables ready to exit, wave median (no cache) | {us(rest):.2f} |")
        print(f"| tail: last exit after the median exit | {us(span - ex50):.2f} |")
        print(f"| kernel span, first entry to last exit (no cache) | {us(span):.2f} |")
        print(f"| decode miss step minus tokenselect_score, wave median (theta = 2: no cosine is computed) | "
              f"{us(rest_c - rest):.2f} |")
        print(f"| kernel span in the decode miss step | {us(span_c):.2f} |")

    print("# Decode-step and scoring-launch timeline (per-wave wall clock, timeline build)")
    for wname, nl in (("llama3-8b-128k", 8), ("qwen2-7b-cache256", 2), ("llama3-8b-1m", 4)):
        geo = wl.workload(wname)
        KC, VC = kv_cache(geo, nl, dev)
        layers = [Layer(geo, l, dev, False, (KC[l], VC[l])) for l in range(nl)]
        L0 = layers[0]
        shape = ts.make_shape(geo.num_q_heads, geo.num_kv_heads, 1, L0.block_table.shape[1], L0.total,
                              geo.torch_dtype)
        H = geo.num_q_heads
        logits = torch.empty(H * L0.total, dtype=torch.float32, device=dev)
        stats_t = torch.empty(H * 2, dtype=torch.float32, device=dev)
        runs = {}
        for tag, theta in (("miss", 2.0), ("hit", -2.0)):
            sel = ts.make_select(geo.top_k, geo.n_local, 1.0, geo.attn_scale, theta)
            need = lib.tokenselect_workspace_size(ctypes.byref(shape), ctypes.byref(sel))
            ws = torch.empty(need, dtype=torch.uint8, device=dev)

            def step(L):
                cs = L.cache.c_struct()
                assert lib.tokenselect_decode_step(ctypes.byref(shape), ctypes.byref(sel), P(L.q), P(L.k_pool),
                                                   P(L.v_pool), P(L.block_table), P(L.seq_lens), ctypes.byref(cs),
                                                   P(L.hit), P(L.out), P(ws), ws.numel(), st) == 0

            def score(L):
                assert lib.tokenselect_score(ctypes.byref(shape), ctypes.byref(sel), P(L.q), P(L.k_pool),
                                             P(L.block_table), P(L.seq_lens), P(logits), P(stats_t), P(ws),
                                             ws.numel(), st) == 0
            for i in range(2 * nl):
                step(layers[i % nl])
            torch.cuda.synchronize()
            runs[tag] = [capture(lambda: step(layers[i % nl])) for i in range(reps)]
            if tag == "miss" and wname == "llama3-8b-128k":
                runs["score"] = [capture(lambda: score(layers[i % nl])) for i in range(reps)]
            del ws
        print_step(f"{wname}: decode miss step (every step reselects)", runs["miss"])
        print_step(f"{wname}: decode Selection Cache hit step", runs["hit"])
        if wname == "llama3-8b-128k":   # one dispatch round (512 workgroups); 1M has two
            score_split(wname, runs["score"], runs["miss"])
        del layers, KC, VC, logits
        torch.cuda.empty_cache()
    g = wl.workload("prefill-llama3-128k")
    KC, VC = kv_cache(g, 2, dev)
    cbs = [wl.make_chunk_batch(g, dev, layer=l, pools=(KC[l], VC[l])) for l in range(2)]
    shape = ts.make_shape(g.num_q_heads, g.num_kv_heads, 1, cbs[0].paged.block_table.shape[1], g.seq_len,
                          g.torch_dtype)
    sel = ts.make_select(g.top_k, g.n_local, 1.0, g.attn_scale, 2.0)
    need = lib.tokenselect_prefill_workspace_size(ctypes.byref(shape), ctypes.byref(sel), g.chunk)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    si = [torch.empty(1, g.top_k, dtype=torch.int32, device=dev) for _ in range(2)]
    sc = [torch.empty(1, dtype=torch.int32, device=dev) for _ in range(2)]
    out = torch.empty(1, g.chunk, g.num_q_heads, g.head_dim, dtype=g.torch_dtype, device=dev)

    def chunk(l, attn_only):
        cb = cbs[l]
        fn = lib.tokenselect_chunk_attn if attn_only else lib.tokenselect_prefill_chunk
        assert fn(ctypes.byref(shape), ctypes.byref(sel), g.chunk, P(cb.q_chunk), P(cb.chunk_lens),
                  P(cb.paged.k_pool), P(cb.paged.v_pool), P(cb.paged.block_table), P(cb.seq_lens), P(si[l]),
                  P(sc[l]), P(out), P(ws), ws.numel(), st) == 0
    for l in (0, 1, 0, 1):
        chunk(l, False)
    torch.cuda.synchronize()
    pruns = [capture(lambda: chunk(i % 2, True))["chunk_attn_bf16"] for i in range(reps)]
    vals = []
    for v in pruns:
        ent = v[:, 0] - v[:, 0].min()
        vals.append((ent.max(), np.median(v[:, 2] - v[:, 0]), np.median(v[:, 3] - v[:, 2]),
                     np.median(v[:, 1] - v[:, 3]), np.median(v[:, 1] - v[:, 0]), (v[:, 1] - v[:, 0].min()).max()))
    ramp, setup, pro, loop, dur, span = np.median(np.array(vals, dtype=np.float64), axis=0)
    blk = []
    for v in pruns:
        v = v[(v[:, 8] & 0xff) >= 6]
        blk.append((np.median(v[:, 5] - v[:, 4]), np.median(v[:, 6] - v[:, 5]), np.median(v[:, 7] - v[:, 6]),
                    np.median(v[:, 7] - v[:, 4])))
    b_qk, b_pv, b_bar, b_all = np.median(np.array(blk, dtype=np.float64), axis=0)
    print("\n### prefill-llama3-128k: chunk attention (chunk of 512, k = 3072, L = 512)\n")
    print("| part | µs |\n|---|---|")
    print(f"| dispatch ramp: last wave entry after the first | {us(ramp):.2f} |")
    print(f"| setup: the split's key list into LDS (wave median) | {us(setup):.2f} |")
    print(f"| prologue: first blocks staged, first scores (wave median) | {us(pro):.2f} |")
    print(f"| block loop and partial stores (wave median) | {us(loop):.2f} |")
    print(f"| wave duration (median) | {us(dur):.2f} |")
    print(f"| kernel span, first entry to last exit | {us(span):.2f} |")
    print("\nOne 64-key iteration of the block loop (the ninth; wave medians; marks taken where the wave "
          "reaches the point):\n")
    print("| part | µs |\n|---|---|")
    print(f"| staging of K issued, rescale, scores of the next block with this block's exp2 | {us(b_qk):.3f} |")
    print(f"| staging of V issued, P V with the next block's maximum | {us(b_pv):.3f} |")
    print(f"| wait for the staging started one iteration earlier, barrier | {us(b_bar):.3f} |")
    print(f"| whole iteration | {us(b_all):.3f} |")
    del cbs, KC, VC, ws
    torch.cuda.empty_cache()


def cpu_baseline(geo, host, dev):
    """The fp64 oracle, as it stands, timed on the host cores beside the GPU figures.

    Every workload is run through the oracle's own entry points (select, window,
    attention; decode_sequence with the Selection Cache for the 256-step sequence):
    the tiny fp32 workload, the 128K request, the 16-request ragged batch (one step of
    the whole batch) and the 256-step Selection Cache sequence in full, and one decode
    step of layer 0 of the 1M workload (the headline's unit). The matmuls run on a
    BLAS pool set to every core of the process's CPU affinity; numpy's elementwise
    steps (exp, sums, sorts) run on one thread. Each workload is also timed with the
    BLAS pool limited to one thread (the sequence on its first 16 steps). Inputs are
    generated on the GPU by the same seeded generators and copied to the host; no
    input is shared with the GPU timings."""
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import tokenselect_oracle as ora
    from synth import workloads as wl
    cores = len(os.sched_getaffinity(0))

    def step_fn(g, q, K, V):
        return lambda: ora.decode_step(q, K, V, g.top_k, g.n_local, 1.0, g.attn_scale)

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def both(fn, one_thread_fn=None):
        with threadpool_limits(limits=cores, user_api="blas"):
            blas = max([i.get("num_threads") or 1 for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
            t_all = timed(fn)
        with threadpool_limits(limits=1, user_api="blas"):
            t_one = timed(one_thread_fn or fn)
        return t_all, t_one, blas

    out = {}
    # one untimed small step first, so no figure below carries numpy's first-call costs
    g0 = wl.workload("tiny-f32-8k", seq_len=2048, top_k=64, n_local=16)
    b0 = wl.make_batch(g0, device=dev)
    r0 = b0.requests[0]
    step_fn(g0, _host(r0.q), _host(r0.k), _host(r0.v))()
    del b0, r0
    # c2: one decode step of layer 0 of the 1M workload (the headline unit)
    q, K, V = host
    t_all, t_one, blas = both(step_fn(geo, q, K, V))
    out[geo.name] = {"decode_steps_per_s": 1.0 / t_all, "decode_steps_per_s_1thread": 1.0 / t_one,
                     "sample": f"one decode step of layer 0 (N = {K.shape[1]})", "seconds": t_all + t_one}
    del host, q, K, V
    # c0, c1: one full decode step of the tiny fp32 and the 128K workloads
    for name in ("tiny-f32-8k", "llama3-8b-128k"):
        g = wl.workload(name)
        b = wl.make_batch(g, device=dev)
        r = b.requests[0]
        args = (_host(r.q), _host(r.k), _host(r.v))
        del b, r
        t_all, t_one, _ = both(step_fn(g, *args))
        out[name] = {"decode_steps_per_s": 1.0 / t_all, "decode_steps_per_s_1thread": 1.0 / t_one,
                     "sample": f"one decode step (N = {args[1].shape[1]})", "seconds": t_all + t_one}
    # c3: one decode step of the whole 16-request batch
    g = wl.workload("llama3-8b-ragged16")
    b = wl.make_batch(g, device=dev)
    reqs = [(_host(r.q), _host(r.k), _host(r.v)) for r in b.requests]
    total = b.total_tokens
    del b
    run = lambda rs: [ora.decode_step(q, K, V, g.top_k, g.n_local, 1.0, g.attn_scale) for q, K, V in rs]
    sub = reqs[:4]
    sub_tokens = sum(K.shape[1] for _, K, _ in sub)
    t_all, t_one, _ = both(lambda: run(reqs), lambda: run(sub))
    out[g.name] = {"decode_steps_per_s": 1.0 / t_all,
                   "decode_steps_per_s_1thread": sub_tokens / total / t_one,
                   "sample": f"one decode step of all {len(reqs)} requests (sum N = {total}); 1 thread: "
                             f"the first 4 requests ({sub_tokens} tokens), scaled to the whole batch",
                   "seconds": t_all + t_one}
    del reqs
    # c4: the 256-step Selection Cache sequence (oracle decode_sequence: fp64 cosine, the
    # selection on misses, the attention every step)
    g = wl.workload("qwen2-7b-cache256")
    gen = torch.Generator(device=dev).manual_seed(g.seed)
    req = wl.make_request(gen, g, g.seq_len, dev, extra_tokens=g.steps - 1)
    qs, _ = wl.ar1_queries(g, req.q_master, g.steps, seed=g.seed + 1, device=dev)
    qs, K, V = _host(qs), _host(req.k), _host(req.v)
    del req
    lens = np.arange(g.seq_len, g.seq_len + g.steps)
    seq = lambda n: ora.decode_sequence(qs[:n], K, V, lens[:n], g.top_k, g.n_local, g.cos_threshold,
                                        1.0, g.attn_scale)
    t_all, t_one, _ = both(lambda: seq(g.steps), lambda: seq(16))
    out[g.name] = {"decode_steps_per_s": g.steps / t_all, "decode_steps_per_s_1thread": 16 / t_one,
                   "sample": f"all {g.steps} steps (1 thread: the first 16 steps)", "seconds": t_all + t_one}
    del qs, K, V
    spent = sum(v["seconds"] for v in out.values())
    log("[cpu oracle] " + ", ".join(f"{k} {v['decode_steps_per_s']:.3g} steps/s "
                                    f"({v['decode_steps_per_s_1thread']:.3g} on 1 thread)" for k, v in out.items())
        + f"; {spent:.1f} s on {cores} cores")
    head = out[geo.name]
    return {"value": head["decode_steps_per_s"], "unit": "decode steps/s", "cores": cores,
            "threads": blas, "kind": "oracle",
            "sample": f"{head['sample']} of {geo.name} with every core of the CPU affinity "
                      f"({cores}) in the BLAS pool; per-config figures (all cores and 1 thread) in "
                      f"configs; {spent:.0f} s of host work in total",
            "value_1thread": head["decode_steps_per_s_1thread"], "configs": out}


def guarded(name, fn):
    """Run a secondary section. A Python-level failure is logged with its traceback
    and reported as {"error": ...} in that section's field instead of ending the run,
    so the headline line is always printed."""
    try:
        return fn()
    except Exception as e:  # noqa: BLE001 - any failure of a secondary section
        import traceback
        log(f"[{name}] failed: {e!r}")
        traceback.print_exc(file=sys.stderr)
        try:
            import torch
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        except Exception:  # noqa: BLE001
            pass
        return {"error": repr(e)}


def ceiling_line(res):
    """The scoring launch against the probe's measured ceilings on the same pools."""
    c = res.get("ceiling")
    if not c:
        return None
    mixed = c["read_plus_1_16_write"]
    return {"kernel": "ts_stream_probe (same K pools, 2048 workgroups)",
            "read_only_gbps": c["read_only"]["gbps"], "read_only_ms": c["read_only"]["ms"],
            "mixed_gbps": mixed["gbps"], "mixed_ms": mixed["ms"],
            "score_frac_of_mixed": mixed["ms"] / res["score_ms"]}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="short program for rocprofv3 --pmc passes (scoring launches + a 1 GiB copy)")
    ap.add_argument("--kernel-counters", action="store_true",
                    help="short program for rocprofv3 --pmc passes over the decode-step kernels at "
                         "128K and the prefill chunk attention")
    ap.add_argument("--phase-probe", action="store_true",
                    help="time the chunk-attention phase probe (libts_stream_probe.so); prints a markdown table")
    ap.add_argument("--timeline", action="store_true",
                    help="per-wave timeline of the decode-step kernels, the scoring launch and the chunk "
                         "attention (libtokenselect_timeline.so); prints a markdown report")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import workloads as wl
    import token_level_sparse_amd as ts
    ts.load_library()
    dev = "cuda:0"
    torch.cuda.set_device(0)

    geo = wl.workload("llama3-8b-1m")
    if args.counters:
        counter_run(geo, dev)
        return
    if args.kernel_counters:
        kernel_counter_run(dev)
        return
    if args.phase_probe:
        phase_probe(dev)
        return
    if args.timeline:
        timeline_run(dev)
        return
    topp_run = None if args.no_secondary else (
        lambda layers: guarded("top_p", lambda: time_topp(geo, 8, max(16, args.steps // 2), 4, dev,
                                                            layers=layers)))
    # every generated layer is timed at least once: with fewer timed steps than layers,
    # only as many layers as steps are generated (and reported)
    n_layers = max(1, min(args.layers, args.steps))
    main_res, host = time_workload(geo, n_layers, args.steps, args.warmup, dev,
                                   keep_host=not args.no_cpu_baseline, ceiling=True, then=topp_run)
    secondary = tiny = None
    if not args.no_secondary:
        def run_128k():
            g1 = wl.workload("llama3-8b-128k")
            # 8 rotating layers: 8 x 256 MiB of K, so no step finds its pool in the 256 MB MALL
            r1, _ = time_workload(g1, 8, max(args.steps, 32), args.warmup, dev, ceiling=True)
            return {"workload": g1.name, "N": g1.seq_len, "decode_steps_per_s": 1e3 / r1["ms_per_step"],
                    "ms_per_step": r1["ms_per_step"],
                    "step_ms_percentiles": {q: r1[f"step_ms_p{q}"] for q in (10, 50, 90)},
                    "score_ms": r1["score_ms"], "score_bytes": r1["score_bytes"],
                    "score_gbps": r1["score_gbps"], "score_frac_of_peak": r1["score_gbps"] / PEAK_HBM_GBPS,
                    "score_with_stats_ms": r1["score_with_stats_ms"],
                    "score_what": "the scoring kernel alone (tokenselect_score with head_stats NULL), as in "
                                  "the decode step, whose vote kernel folds the statistics at this size",
                    "k_gbps": r1["k_gbps"], "rotating_layers": 8, "ceiling": ceiling_line(r1)}
        secondary = guarded("llama3-8b-128k", run_128k)

        def run_tiny():
            g0 = wl.workload("tiny-f32-8k")
            r0, _ = time_workload(g0, 1, max(args.steps, 32), args.warmup, dev)
            return {"workload": g0.name, "N": g0.seq_len, "dtype": "f32",
                    "decode_steps_per_s": 1e3 / r0["ms_per_step"], "ms_per_step": r0["ms_per_step"],
                    "step_ms_percentiles": {q: r0[f"step_ms_p{q}"] for q in (10, 50, 90)},
                    "score_ms": r0["score_ms"], "score_bytes": r0["score_bytes"],
                    "score_gbps_effective": r0["score_gbps"],
                    "score_frac_of_peak_effective": r0["score_gbps"] / PEAK_HBM_GBPS,
                    "what": "correctness-sized workload (8 MiB of fp32 K, cache-resident): "
                            "latency-bound, its bandwidth is an effective one"}
        tiny = guarded("tiny-f32-8k", run_tiny)
    ragged = cache_seq = prefill = topp = ablations = dense = None
    if not args.no_secondary:
        ceil = main_res.get("ceiling") or {}
        dense = guarded("dense", lambda: time_dense(geo, main_res["ms_per_step"],
                                                    (ceil.get("read_only") or {}).get("gbps"), dev))
        ragged = guarded("ragged", lambda: time_ragged(wl.workload("llama3-8b-ragged16"),
                                                       max(8, args.steps // 4), 2, dev))
        cache_seq = guarded("selection_cache", lambda: time_cache_sequence(wl.workload("qwen2-7b-cache256"), dev))
        topp = main_res.get("then")
        ablations = guarded("ablations", lambda: time_ablations(wl.workload("llama3-8b-128k"), dev))
        prefill = [guarded("prefill-128k", lambda: time_prefill(wl.workload("prefill-llama3-128k"), 8,
                                                                 max(16, args.steps // 2), 4, dev)),
                   guarded("prefill-1m", lambda: time_prefill(wl.workload("prefill-llama3-1m"), 4,
                                                               max(8, args.steps // 8), 2, dev))]
    cpu = guarded("cpu_baseline", lambda: cpu_baseline(geo, host, dev)) if host is not None else None

    ms = main_res["ms_per_step"]
    line = {
        "metric": "decode steps/s and K-scoring HBM GB/s (% peak) at N=128K and 1M, 1 GPU",
        "value": 1e3 / ms,
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_ms_percentiles": {q: main_res[f"step_ms_p{q}"] for q in (10, 50, 90)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": geo.name, "N": geo.seq_len, "batch": 1,
                   "heads": f"{geo.num_q_heads}/{geo.num_kv_heads}/{geo.head_dim}",
                   "top_k": geo.top_k, "n_local": geo.n_local, "page_size": geo.page_size,
                   "layers": n_layers, "cache": "every step reselects"},
        "roofline": {"bound": "hbm", "achieved": main_res["score_gbps"], "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": main_res["score_gbps"] / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(),
                     "kernel": "score_kernel (tokenselect_score with head_stats NULL: the scoring kernel alone)",
                     "bytes_per_launch": main_res["score_bytes"], "launch_ms": main_res["score_ms"],
                     "launch_with_stats_ms": main_res["score_with_stats_ms"],
                     "ceiling": ceiling_line(main_res)},
        "k_stream_gbps": main_res["k_gbps"],
        "scored_tokens_per_s": main_res["tokens"] * 1e3 / ms,
        "secondary": secondary,
        "tiny": tiny,
        "ragged_batch": ragged,
        "selection_cache": cache_seq,
        "prefill": prefill,
        "top_p": topp,
        "ablations": ablations,
        "dense_reference": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

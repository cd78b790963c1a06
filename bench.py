#!/usr/bin/env python3
"""Benchmark of the ISPA hot path on one MI355X.

One step = the whole warmup-to-absorption pass of the 14B-class workload:
for each of 4 warmup chunks (history 0 -> 36 latent frames) and each of the
40 layers, the decomposable attention (O_full token-major for the model;
X = O_local and D feature-major, kept resident for all warmup chunks); then
the Gram statistics of all 40 layers over all their warmup tokens in one
call; then, batched over the 40 layers, the ridge solve for dW, the layer
errors, the selection of K = 20 layers and the in-place bf16 update of their
output projections. All inputs are resident in HBM before timing
starts; W_o is restored from a pristine copy at the start of every step.

Prints one JSON line. `value` is the decomposable-attention throughput in
algorithmic TFLOP/s (4 * n_q * n_kv * hidden per launch, QK^T and PV only)
measured with HIP events around the attention launches of the timed steps.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import re
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
METRIC = "decomp-attention TFLOP/s (% bf16 MFMA peak) + \u0394W absorb ms/layer, 14B-class"

# HBM traffic of the attention and Gram kernels, from two rocprofv3 --pmc
# runs (FETCH_SIZE, WRITE_SIZE) of this script, written by --pmc-summary. The
# figures are used only while the kernel sources still hash to the recorded
# value; otherwise `traffic` is null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_gram_wan14b_warmup_hbm_traffic.md")
KERNEL_SOURCES = {
    "attn_decomp_kernel<128, false>": ["kv_cache_absorption_attn_amd/csrc/attn_decomp.hip",
                                       "kv_cache_absorption_attn_amd/csrc/device_common.h"],
    "gram_t_kernel": ["kv_cache_absorption_attn_amd/csrc/gemm256.hip",
                      "kv_cache_absorption_attn_amd/csrc/device_common.h",
                      "kv_cache_absorption_attn_amd/csrc/lds_dma_asm.h"],
}
COPY_BYTES = 1 << 30


def attn_flops(n_q, n_kv, hidden):
    return 4.0 * n_q * n_kv * hidden


def gram_flops(n_tok, hidden):
    return 4.0 * n_tok * hidden * hidden


def absorb_flops(hidden):
    h = float(hidden)
    return 2 * h ** 3 + h ** 3 / 3 + 2 * h ** 3 + h ** 3


class Inputs:
    """Device-resident synthetic inputs of one warmup workload, drawn with a
    seeded torch generator on the GPU (values do not affect dense timing)."""

    def __init__(self, w: wl.Workload, seed: int = 0):
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        nh, d, h = w.n_heads, w.head_dim, w.hidden
        bf = torch.bfloat16
        temps = wl.layer_temperatures(w)

        def rnd(*shape, std=1.0):
            t = torch.randn(*shape, generator=g, device=dev, dtype=torch.float32)
            return (t * std).to(bf)

        self.w = w
        self.q = [[rnd(w.n_q, nh, d, std=w.qkv_std * float(temps[l])) for _ in range(w.n_steps)]
                  for l in range(w.n_layers)]
        self.k_sink = [rnd(w.n_sink, nh, d, std=w.qkv_std) for _ in range(w.n_layers)]
        self.v_sink = [rnd(w.n_sink, nh, d, std=w.qkv_std) for _ in range(w.n_layers)]
        self.k_cur = [[rnd(w.n_cur, nh, d, std=w.qkv_std) for _ in range(w.n_steps)]
                      for _ in range(w.n_layers)]
        self.v_cur = [[rnd(w.n_cur, nh, d, std=w.qkv_std) for _ in range(w.n_steps)]
                      for _ in range(w.n_layers)]
        hm = w.n_hist_max
        self.k_hist = [rnd(hm, nh, d, std=w.qkv_std) if hm else None for _ in range(w.n_layers)]
        self.v_hist = [rnd(hm, nh, d, std=w.qkv_std) if hm else None for _ in range(w.n_layers)]
        self.wo0 = rnd(w.n_layers, h, h, std=w.wo_std)
        self.wo = self.wo0.clone()
        # outputs / state
        self.o_full = torch.empty(w.n_q, h, dtype=bf, device=dev)
        self.x = torch.empty(w.n_q, h, dtype=bf, device=dev)
        # every warmup step's X and D stay resident until the transition,
        # feature-major (token-contiguous per feature), the warmup steps of a
        # layer side by side: [L, h, T_warm * N] bf16, 15.3 GB for both at 14B
        self.xt = torch.empty(w.n_layers, h, w.n_steps * w.n_q, dtype=bf, device=dev)
        self.dt = torch.empty_like(self.xt)
        self.y = torch.empty(w.n_q, h, dtype=bf, device=dev)
        f32 = torch.float32
        self.G = torch.empty(w.n_layers, h, h, dtype=f32, device=dev)
        self.C = torch.empty_like(self.G)
        self.E = torch.empty_like(self.G)
        self.dW = torch.empty_like(self.G)
        self.info = torch.empty(w.n_layers, dtype=torch.int32, device=dev)
        self.eps_abs = torch.empty(w.n_layers, dtype=torch.float64, device=dev)
        self.eps_rel = torch.empty(w.n_layers, dtype=torch.float64, device=dev)
        self.selected = torch.empty(w.n_layers, dtype=torch.int32, device=dev)

    def hist_view(self, layer, step):
        n = self.w.hist_per_step[step]
        if n == 0:
            return None, None
        return self.k_hist[layer][:n], self.v_hist[layer][:n]


def run_step(ispa, inp: Inputs, ws, timing: dict | None):
    """One pass of the whole hot path. When `timing` is given, HIP events are
    recorded around each stage on the launch stream."""
    w = inp.w
    ev = []

    def mark(tag):
        if timing is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev.append((tag, e))

    inp.wo.copy_(inp.wo0)
    n = w.n_q
    for s in range(w.n_steps):
        for l in range(w.n_layers):
            kh, vh = inp.hist_view(l, s)
            mark("attn0")
            ispa.ispa_attn_decomp_t(inp.q[l][s], inp.k_sink[l], inp.v_sink[l],
                                    inp.k_cur[l][s], inp.v_cur[l][s], kh, vh, w.sm_scale,
                                    inp.xt[l], inp.dt[l], col=s * n, o_full=inp.o_full)
            mark("attn1")
    # the warmup statistics of every layer in one call over all warmup tokens
    # (the per-call cost is paid once, and the 40 layers' tiles fill the chip
    # with no partial last round)
    mark("gram0")
    ispa.ispa_gram_accumulate_t(inp.xt, inp.dt, w.n_steps * n, inp.G, inp.C, inp.E,
                                zero_first=True)
    mark("gram1")
    mark("absorb0")
    ispa.ispa_ridge_solve(inp.G, inp.C, inp.wo, w.lam, inp.dW, inp.info, ws)
    mark("ridge1")
    ispa.ispa_layer_score(inp.G, inp.C, inp.E, inp.wo, inp.dW, w.lam, inp.info, w.k_select, ws,
                          inp.eps_abs, inp.eps_rel, inp.selected)
    mark("score1")
    ispa.ispa_apply_dW(inp.selected, inp.dW, inp.wo)
    mark("absorb1")
    # The first chunk after absorption, at the last warmup history: selected
    # layers (L-layers) attend their local KV only and project through the
    # updated W_o; the others (F-layers) run full attention, O_F only, and
    # project through their own W_o. Which layers are L is a host decision
    # (their history KV is freed), hence the one read of `selected` here.
    sel = inp.selected.cpu().tolist()
    s = w.n_steps - 1
    mark("post0")
    for l in range(w.n_layers):
        if sel[l]:
            ispa.ispa_attn_decomp(inp.q[l][s], inp.k_sink[l], inp.v_sink[l], inp.k_cur[l][s],
                                  inp.v_cur[l][s], None, None, w.sm_scale, o_local=inp.x)
        else:
            kh, vh = inp.hist_view(l, s)
            ispa.ispa_attn_decomp(inp.q[l][s], inp.k_sink[l], inp.v_sink[l], inp.k_cur[l][s],
                                  inp.v_cur[l][s], kh, vh, w.sm_scale, o_full=inp.x)
        ispa.ispa_project(inp.x, inp.wo[l], inp.y)
    mark("post1")
    if timing is not None:
        timing.setdefault("events", []).append(ev)


def summarize_events(timing):
    tot = {"attn": 0.0, "gram": 0.0, "ridge": 0.0, "score": 0.0, "apply": 0.0, "post": 0.0}
    n_attn = 0
    for ev in timing["events"]:
        prev = None
        for tag, e in ev:
            if prev is not None:
                dt = prev[1].elapsed_time(e)
                key = {("attn0", "attn1"): "attn", ("gram0", "gram1"): "gram",
                       ("absorb0", "ridge1"): "ridge", ("ridge1", "score1"): "score",
                       ("score1", "absorb1"): "apply", ("post0", "post1"): "post"
                       }.get((prev[0], tag))
                if key:
                    tot[key] += dt
                    n_attn += key == "attn"
            prev = (tag, e)
    return tot, n_attn


def stream_measure(ispa, w: wl.Workload, frames=(36, 60, 90, 120), reps: int = 2,
                   seed: int = 1):
    """Long-horizon streaming after absorption (14B-class) through the KV
    cache (ispa_kv_*): chunks of 3 latent frames stream in and every
    full-history layer's history grows, chunk by chunk, to `frames` latent
    frames. Two runs, one after the other: ISPA (k_select L-layers, every
    other layer, whose history is evicted at the transition; the rest
    F-layers) and every layer full. At each listed history length the
    attention + output projection of all layers for one chunk is timed with
    HIP events (`reps` passes); writing the chunk K/V into the cache (a copy
    here, the K/V projection's own output in a model) is not timed, and the
    host time of advancing the cache (mapping the next slot's pages) is
    reported beside it. KV bytes are the cache's mapped bytes."""
    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    nh, d, h = w.n_heads, w.head_dim, w.hidden
    tok_per_frame = w.n_cur // 3
    chunk_frames = w.n_cur // tok_per_frame
    targets = {fr // chunk_frames: fr for fr in frames}
    n_chunks = max(targets) + 1

    def rnd(*shape):
        return (torch.randn(*shape, generator=g, device=dev) * w.qkv_std).to(bf)

    L = w.n_layers
    q = [rnd(w.n_q, nh, d) for _ in range(L)]
    k_sink, v_sink = rnd(w.n_sink, nh, d), rnd(w.n_sink, nh, d)
    k_chunk, v_chunk = rnd(w.n_cur, nh, d), rnd(w.n_cur, nh, d)
    wo = rnd(L, h, h)
    x = torch.empty(w.n_q, h, dtype=bf, device=dev)
    y = torch.empty_like(x)
    is_l = [l % 2 == 0 for l in range(L)]
    assert sum(is_l) == w.k_select

    def one_chunk(cache):
        for l in range(L):
            cache.layer_forward(l, q[l], w.sm_scale, wo[l], x, y)

    res = {"frames": list(frames), "l_layers": sum(is_l), "f_layers": L - sum(is_l),
           "ispa_ms": [], "all_full_ms": [], "speedup": [], "ispa_kv_gb": [],
           "all_full_kv_gb": [], "ispa_advance_host_ms": None, "all_full_advance_host_ms": None}
    for split in (True, False):
        tag = "ispa" if split else "all_full"
        cache = ispa.KVCache(L, nh, d, w.n_sink, w.n_cur, (n_chunks - 1) * w.n_cur)
        try:
            for l in range(L):
                cache.write(l, k_sink, v_sink, sink=True)
                if split and is_l[l]:
                    cache.evict_history(l)
            adv_s = 0.0
            for c in range(n_chunks):
                for l in range(L):
                    cache.write(l, k_chunk, v_chunk)
                if c in targets:
                    one_chunk(cache)
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(reps):
                        one_chunk(cache)
                    e1.record()
                    torch.cuda.synchronize()
                    ms = e0.elapsed_time(e1) / reps
                    res[f"{tag}_ms"].append(round(ms, 2))
                    res[f"{tag}_kv_gb"].append(round(cache.resident_bytes() / 1e9, 2))
                    print(f"[bench] stream {tag} {targets[c]} frames: {ms:.1f} ms per chunk, "
                          f"{cache.resident_bytes() / 1e9:.1f} GB KV", file=sys.stderr, flush=True)
                if c + 1 < n_chunks:
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    cache.advance()
                    adv_s += time.perf_counter() - t0
            res[f"{tag}_advance_host_ms"] = round(adv_s / max(1, n_chunks - 1) * 1e3, 3)
        finally:
            cache.close()
    res["speedup"] = [round(f / i, 3) for i, f in zip(res["ispa_ms"], res["all_full_ms"])]
    return res


def session_measure(ispa, w: wl.Workload, n_stream: int = 3, seed: int = 2, flags: int = 0):
    """The 14B-class life cycle through the native streaming session
    (ispa_session_*): a fresh stream of t_warm warmup chunks (every layer
    dual-stream, Gram accumulation, projection), the transition (solve,
    score, selection, update, eviction, drift factors), then n_stream
    streaming chunks with the drift check of the L-layers on. Per chunk the
    layer calls are timed with HIP events; end_chunk (which reads the
    selection or the drift scores back, so it waits for the stream) with
    the host clock. K/V writes are outside the timed regions. `flags` selects
    the quantized variant (W8A8 projections, E4M3 attention while
    streaming)."""
    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    nh, d, h, L = w.n_heads, w.head_dim, w.hidden, w.n_layers

    def rnd(*shape, std=w.qkv_std):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(bf)

    wo = rnd(L, h, h, std=w.wo_std)
    q = [rnd(w.n_cur, nh, d) for _ in range(L)]
    k_sink, v_sink = rnd(w.n_sink, nh, d), rnd(w.n_sink, nh, d)
    k_chunk, v_chunk = rnd(w.n_cur, nh, d), rnd(w.n_cur, nh, d)
    y = torch.empty(w.n_cur, h, dtype=bf, device=dev)
    t_warm = w.n_steps
    n_chunks = t_warm + n_stream
    sess = ispa.Session(wo, n_heads=nh, head_dim=d, n_sink=w.n_sink, n_cur=w.n_cur,
                        hist_capacity=n_chunks * w.n_cur, k_select=w.k_select, t_warm=t_warm,
                        sm_scale=w.sm_scale, lam=w.lam, drift_threshold=1e30, drift_stride=16,
                        flags=flags)
    res = {"flags": flags, "t_warm": t_warm, "warmup_chunk_ms": [], "stream_chunk_ms": [], "events": [],
           "end_chunk_host_ms": [], "workspace_gb": round(sess.workspace.numel() / 1e9, 2)}
    try:
        for l in range(L):
            sess.cache.write(l, k_sink, v_sink, sink=True)
        for c in range(n_chunks):
            for l in range(L):
                sess.cache.write(l, k_chunk, v_chunk)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(L):
                sess.layer(l, q[l], y)
            e1.record()
            t0 = time.perf_counter()
            ev = sess.end_chunk()
            torch.cuda.synchronize()
            t_end = (time.perf_counter() - t0) * 1e3
            ms = e0.elapsed_time(e1)
            res["warmup_chunk_ms" if c < t_warm else "stream_chunk_ms"].append(round(ms, 2))
            res["events"].append(ev)
            res["end_chunk_host_ms"].append(round(t_end, 2))
            print(f"[bench] session chunk {c}: layers {ms:.1f} ms, end_chunk {t_end:.1f} ms, "
                  f"event {ev}", file=sys.stderr, flush=True)
        st, loc, eps, drift = sess.state()
        res["l_layers"] = sum(loc)
        res["drift_scores_l_layers"] = [round(x, 3) for x, on in zip(drift, loc) if on][:4]
        res["kv_gb"] = round(sess.cache.resident_bytes() / 1e9, 2)
    finally:
        sess.close()
    return res


def quantized_measure(ispa, w: wl.Workload, reps: int = 10, seed: int = 3):
    """The E4M3 variants at the headline launch shape (the last warmup step:
    O_local, O_full and D of one layer) and at one chunk's output projection,
    each beside its bf16 counterpart, HIP events on the launch stream. The
    E4M3 attention time includes the quantization of Q and K (the key mean is
    timed on its own); the W8A8 projection time includes the per-token
    quantization of X."""
    dev, bf = "cuda", torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    nh, d, h = w.n_heads, w.head_dim, w.hidden
    n_hist = w.hist_per_step[-1]

    def rnd(*shape, std=1.0):
        return (torch.randn(*shape, device=dev, generator=gen) * std).to(bf)

    q = rnd(w.n_q, nh, d, std=w.qkv_std)
    kv = [rnd(n, nh, d, std=w.qkv_std) for n in (w.n_sink, w.n_sink, w.n_cur, w.n_cur,
                                                 n_hist, n_hist)]
    outs = [torch.empty(w.n_q, h, dtype=bf, device=dev) for _ in range(3)]
    ws = torch.empty(ispa.ispa_attn_fp8_workspace_bytes(w.n_q, w.n_sink, w.n_cur, n_hist, nh, d),
                     dtype=torch.uint8, device=dev)
    mu = torch.empty(nh, d, dtype=bf, device=dev)
    mws = torch.empty(ispa.ispa_key_mean_workspace_bytes(nh, d), dtype=torch.uint8, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    o3 = dict(o_local=outs[0], o_full=outs[1], d_out=outs[2])
    t_bf16 = timed(lambda: ispa.ispa_attn_decomp(q, *kv, w.sm_scale, **o3))
    t_mean = timed(lambda: ispa.ispa_key_mean(kv[0], kv[2], kv[4], mu, mws))
    t_fp8 = timed(lambda: ispa.ispa_attn_decomp_fp8(q, *kv, w.sm_scale, ws, k_mean=mu, **o3))
    fl = attn_flops(w.n_q, w.n_sink + w.n_cur + n_hist, h)
    del kv, ws
    x = rnd(w.n_q, h, std=0.3)
    wo = rnd(h, h, std=h ** -0.5)
    y = torch.empty(w.n_q, h, dtype=bf, device=dev)
    wq = torch.empty(h, h, dtype=torch.uint8, device=dev)
    wsc = torch.empty(h, dtype=torch.float32, device=dev)
    ispa.ispa_quantize_fp8(wo, wq, wsc)
    pws = torch.empty(ispa.ispa_project_w8a8_workspace_bytes(w.n_q, h), dtype=torch.uint8,
                      device=dev)
    t_pb = timed(lambda: ispa.ispa_project(x, wo, y))
    t_p8 = timed(lambda: ispa.ispa_project_w8a8(x, wq, wsc, y, pws))
    pfl = 2.0 * w.n_q * h * h
    return {
        "attn_launch": f"n_q {w.n_q}, {w.n_sink} + {w.n_cur} local + {n_hist} history keys, "
                       "O_local, O_full, D",
        "attn_bf16_ms": round(t_bf16, 3),
        "attn_fp8_ms": round(t_fp8, 3),
        "attn_fp8_speedup": round(t_bf16 / t_fp8, 3),
        "attn_fp8_tflops_bf16_equiv": round(fl / (t_fp8 * 1e-3) / 1e12, 1),
        "key_mean_ms": round(t_mean, 3),
        "proj_shape": [w.n_q, h, h],
        "proj_bf16_us": round(t_pb * 1e3, 1),
        "proj_w8a8_us": round(t_p8 * 1e3, 1),
        "proj_w8a8_speedup": round(t_pb / t_p8, 3),
        "proj_w8a8_tflops": round(pfl / (t_p8 * 1e-3) / 1e12, 1),
    }


def multi_instance_measure(ispa, w: wl.Workload, n_inst: int = 8, n_q: int = 512,
                           reps: int = 5, seed: int = 4):
    """Concurrent streams with their own KV and their own W + dW: n_inst
    short chunks (n_q queries each, the workload's heads, sink and longest
    warmup history) as separate calls and as one grouped call, for the
    attention (O_full) and the output projection. HIP events on the launch
    stream."""
    dev, bf = "cuda", torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    nh, d, h = w.n_heads, w.head_dim, w.hidden
    n_hist = w.hist_per_step[-1]

    def rnd(*shape, std=1.0):
        return (torch.randn(*shape, device=dev, generator=gen) * std).to(bf)

    calls = [dict(q=rnd(n_q, nh, d), k_sink=rnd(w.n_sink, nh, d), v_sink=rnd(w.n_sink, nh, d),
                  k_cur=rnd(n_q, nh, d), v_cur=rnd(n_q, nh, d), k_hist=rnd(n_hist, nh, d),
                  v_hist=rnd(n_hist, nh, d), o_full=torch.empty(n_q, h, dtype=bf, device=dev))
             for _ in range(n_inst)]
    xs = [rnd(n_q, h, std=0.3) for _ in range(n_inst)]
    ws = [rnd(h, h, std=h ** -0.5) for _ in range(n_inst)]
    ys = [torch.empty(n_q, h, dtype=bf, device=dev) for _ in range(n_inst)]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def attn_sep():
        for c in calls:
            ispa.ispa_attn_decomp(c["q"], c["k_sink"], c["v_sink"], c["k_cur"], c["v_cur"],
                                  c["k_hist"], c["v_hist"], w.sm_scale, o_full=c["o_full"])

    def proj_sep():
        for x, wo, y in zip(xs, ws, ys):
            ispa.ispa_project(x, wo, y)

    t_as = timed(attn_sep)
    t_ag = timed(lambda: ispa.ispa_attn_decomp_grouped(calls, w.sm_scale))
    t_ps = timed(proj_sep)
    t_pg = timed(lambda: ispa.ispa_project_grouped(xs, ws, ys))
    fl = attn_flops(n_q, w.n_sink + n_q + n_hist, h) * n_inst
    return {
        "instances": n_inst,
        "chunk": f"{n_q} queries x {nh} heads, {w.n_sink} + {n_q} local + {n_hist} history keys",
        "attn_separate_ms": round(t_as, 3),
        "attn_grouped_ms": round(t_ag, 3),
        "attn_grouped_speedup": round(t_as / t_ag, 3),
        "attn_grouped_tflops": round(fl / (t_ag * 1e-3) / 1e12, 1),
        "proj_separate_us": round(t_ps * 1e3, 1),
        "proj_grouped_us": round(t_pg * 1e3, 1),
        "proj_grouped_speedup": round(t_ps / t_pg, 3),
    }


def gram_deferred_measure(ispa, w: wl.Workload, reps: int = 5, seed: int = 5):
    """One layer's warmup statistics three ways: one token-major Gram call
    per warmup step (N tokens each), a single token-major call over all
    T_warm steps' X and D kept resident (T_warm * N tokens), which pays the
    per-call cost (pipeline fill, tile write-out, fp32 read-modify-write of
    G, C, E) once, and the single feature-major call the warmup pass makes
    (ispa_gram_accumulate_t, here for one layer). Same sums; HIP events on
    the launch stream."""
    dev, bf = "cuda", torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    h, n, T = w.hidden, w.n_q, w.n_steps
    x = (torch.randn(T * n, h, device=dev, generator=gen) * 0.3).to(bf)
    d = (torch.randn(T * n, h, device=dev, generator=gen) * 0.05).to(bf)
    G, C, E = (torch.empty(h, h, dtype=torch.float32, device=dev) for _ in range(3))

    def per_step():
        for s in range(T):
            ispa.ispa_gram_accumulate(x[s * n:(s + 1) * n], d[s * n:(s + 1) * n], G, C, E,
                                      zero_first=s == 0)

    def once():
        ispa.ispa_gram_accumulate(x, d, G, C, E, zero_first=True)

    xt, dt = x.t().contiguous(), d.t().contiguous()

    def once_t():
        ispa.ispa_gram_accumulate_t(xt, dt, T * n, G, C, E, zero_first=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_step, t_once, t_once_t = timed(per_step), timed(once), timed(once_t)
    fl = gram_flops(T * n, h)
    return {"tokens": T * n, "per_step_calls_ms": round(t_step, 3),
            "one_call_ms": round(t_once, 3), "per_step_tflops": round(fl / t_step / 1e9, 1),
            "one_call_tflops": round(fl / t_once / 1e9, 1),
            "feature_major_one_call_ms": round(t_once_t, 3),
            "feature_major_one_call_tflops": round(fl / t_once_t / 1e9, 1),
            "resident_activation_gb_per_layer": round(2 * T * n * h * 2 / 1e9, 3)}


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed, so that
    a change to comments or layout alone keeps the hash of the code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel: str) -> str:
    """sha256 (first 16 hex digits) of the code of the sources a kernel is
    built from, comments and whitespace aside."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (fetch + write, calibrated) from the
    committed pmc summary, or None when it is missing or was taken on other
    kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = source_hash(kernel)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            m = line.strip().strip("|").split("|")
            if len(m) >= 6 and m[0].strip() == kernel and m[1].strip() == want:
                return float(m[5])
    return None


def copy_calibration():
    """A plain 1 GiB device-to-device copy: the reference reading of the HBM
    byte counters (it reads and writes exactly COPY_BYTES)."""
    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1.0)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()


def pmc_summary(fetch_csv: str, write_csv: str, w: wl.Workload):
    """Markdown table of calibrated HBM bytes per launch for the attention and
    Gram kernels from the counter_collection CSVs of two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE) of one step of `bench.py --copy-calibration`.
    Attention figures average the decomposable launches of the warmup pass
    (the post-absorption chunk that follows them in each step is left out),
    as the `achieved` throughput does."""
    n_warm, n_post = w.n_steps * w.n_layers, w.n_layers

    def read(path, counter):
        with open(path) as f:
            rows = sorted((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                          for r in csv.DictReader(f) if r["Counter_Name"] == counter)
        # the calibration copy is the last large copy of the run (smaller
        # device-to-host reads of the results follow it)
        copy = [v for _, n, v in rows if "copyBuffer" in n and v > 1024][-1]
        attn = [v for _, n, v in rows if "attn_decomp_kernel<128, false>" in n]
        attn = [v for i, v in enumerate(attn) if i % (n_warm + n_post) < n_warm]
        # each step: one feature-major Gram launch over every layer and all
        # warmup tokens (the G-only W_o^T W_o of the layer score is another
        # kernel)
        gram = [v for _, n, v in rows if "gram_t_kernel" in n]
        return copy, {"attn_decomp_kernel<128, false>": attn, "gram_t_kernel": gram}

    fc, fe = read(fetch_csv, "FETCH_SIZE")
    wc, wr = read(write_csv, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024.0
    f_fac, w_fac = copy_kib / fc, copy_kib / wc
    run = "python3 $REPO/bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-stream --copy-calibration"
    lines = [
        f"# HBM traffic per launch: attention and Gram kernels, {w.name}", "",
        "Commands (run from the repository root on one MI355X):", "", "```",
        "cd /tmp && export TMPDIR=/tmp    # REPO: the repository root; OUT: a results directory",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o fetch -- {run}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o write -- {run}",
        "python3 $REPO/bench.py --pmc-summary $OUT/pmc_fetch/fetch_counter_collection.csv "
        "$OUT/pmc_write/write_counter_collection.csv",
        "```", "",
        f"Calibration: the plain 1 GiB copy (the last large copy of the run) reads FETCH_SIZE = {fc:.0f} KiB "
        f"and WRITE_SIZE = {wc:.0f} KiB, so fetch counts are scaled by {f_fac:.4f} and write counts "
        f"by {w_fac:.4f}.", "",
        "| kernel | code sha256[:16] (comments aside) | launches | fetch GB/launch | write GB/launch | "
        "bytes/launch (fetch+write) |",
        "|---|---|---:|---:|---:|---:|",
    ]
    for k in KERNEL_SOURCES:
        if not fe.get(k) or not wr.get(k):
            continue
        fb = sum(fe[k]) / len(fe[k]) * 1024 * f_fac
        wb = sum(wr[k]) / len(wr[k]) * 1024 * w_fac
        lines.append(f"| {k} | {source_hash(k)} | {len(fe[k])} | {fb / 1e9:.4f} | {wb / 1e9:.4f} | "
                     f"{fb + wb:.6g} |")
    return "\n".join(lines) + "\n"


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16"


def pmc_mfma_summary(csv_path: str, w: wl.Workload):
    """Markdown table of matrix-core counters per launch of the attention and
    Gram kernels from one rocprofv3 --pmc run of MFMA_COUNTERS over one step
    of this script. GRBM_GUI_ACTIVE reads as the sum of the 8 XCDs' active
    cycles, so the shader clock of a launch is GUI / 8 / duration, and the
    matrix-pipe busy fraction is SQ_VALU_MFMA_BUSY_CYCLES (summed over all
    SIMDs) / (GUI / 8 x SIMDs). The MFMA FLOP the hardware counted
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) is set against the algorithmic FLOP
    (the excess is the padded rows of partial tiles)."""
    vals: dict = {}
    names: dict = {}
    dur: dict = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            i = int(r["Dispatch_Id"])
            k = (i, r["Counter_Name"])
            vals[k] = vals.get(k, 0.0) + float(r["Counter_Value"])
            names[i] = r["Kernel_Name"]
            dur[i] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    simds, xcds = 256 * 4, 8
    n_warm, n_post = w.n_steps * w.n_layers, w.n_layers
    n_kv = [w.n_sink + w.n_cur + hs for hs in w.hist_per_step]
    attn_ids = sorted(i for i, n in names.items() if "attn_decomp_kernel<128, false>" in n)
    attn_ids = [i for j, i in enumerate(attn_ids) if j % (n_warm + n_post) < n_warm]
    gram_ids = sorted(i for i, n in names.items() if "gram_t_kernel" in n)
    rows = [("attn_decomp_kernel<128, false>", attn_ids,
             sum(attn_flops(w.n_q, nk, w.hidden) for nk in n_kv) / len(n_kv)),
            ("gram_t_kernel", gram_ids, gram_flops(w.n_steps * w.n_q, w.hidden) * w.n_layers)]
    run = "python3 $REPO/bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-stream"
    lines = [f"# Matrix-core counters per launch: attention and Gram kernels, {w.name}", "",
             "Commands (run from the repository root on one MI355X):", "", "```",
             "cd /tmp && export TMPDIR=/tmp    # REPO: the repository root; OUT: a results directory",
             f"rocprofv3 --pmc {MFMA_COUNTERS} --output-format csv -d $OUT/pmc_mfma "
             f"-o mfma -- {run}",
             "python3 $REPO/bench.py --pmc-mfma-summary "
             "$OUT/pmc_mfma/mfma_counter_collection.csv", "```", "",
             "| kernel | launches | matrix pipe busy | shader clock (GHz) | counted MFMA FLOP / "
             "algorithmic |", "|---|---:|---:|---:|---:|"]
    for name, ids, fl in rows:
        if not ids:
            continue
        busy = sum(vals.get((i, "SQ_VALU_MFMA_BUSY_CYCLES"), 0.0) for i in ids)
        gui = sum(vals.get((i, "GRBM_GUI_ACTIVE"), 0.0) for i in ids) / xcds
        ns = sum(dur[i] for i in ids)
        mops = sum(vals.get((i, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), 0.0) for i in ids)
        lines.append(f"| {name} | {len(ids)} | {100 * busy / (gui * simds):.1f} % | "
                     f"{gui / ns:.2f} | {mops * 512 / (fl * len(ids)):.3f} |")
    return "\n".join(lines) + "\n"


def _short_kernel_name(n: str) -> str:
    n = n.replace("void ", "").replace("ispa::(anonymous namespace)::", "")
    if n.startswith("at::native") or "at::native" in n[:40]:
        return "torch " + n.split("<")[0].split("::")[-1] + " (input generation / restore)"
    return n.split("(")[0][:70]


def trace_table(trace_csv: str, command: str):
    """Markdown table of every kernel in a rocprofv3 --kernel-trace CSV:
    launches, average and total time (the whole run, all measurement legs)."""
    agg: dict = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            k = _short_kernel_name(r["Kernel_Name"])
            c, t = agg.get(k, (0, 0))
            agg[k] = (c + 1, t + int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(t for _, t in agg.values())
    lines = ["Command (run from the repository root on one MI355X):", "", "```",
             "cd /tmp && export TMPDIR=/tmp    # REPO: the repository root; OUT: a results directory", command,
             "python3 $REPO/bench.py --trace-table $OUT/ktq/ktq_kernel_trace.csv",
             "```", "", "| Kernel | Calls | Avg (us) | Total (ms) | % |",
             "|---|---:|---:|---:|---:|"]
    for k, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        if t / total < 1e-4:
            continue
        lines.append(f"| {k} | {c} | {t / c / 1e3:.1f} | {t / 1e6:.2f} | {100 * t / total:.2f} |")
    return "\n".join(lines) + "\n"


def trace_summary(trace_csv: str, w: wl.Workload, passes: int):
    """Markdown summary of a rocprofv3 --kernel-trace CSV of `passes` steps of
    this script: per-kernel totals, and the attention launches split into the
    decomposable launches of the warmup pass and the post-absorption chunk."""
    with open(trace_csv) as f:
        rows = sorted((int(r["Dispatch_Id"]), r["Kernel_Name"],
                       int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                      for r in csv.DictReader(f))
    agg: dict = {}
    for _, n, dt in rows:
        k = _short_kernel_name(n)
        c, t = agg.get(k, (0, 0))
        agg[k] = (c + 1, t + dt)
    total = sum(t for _, t in agg.values())
    n_warm, n_post = w.n_steps * w.n_layers, w.n_layers
    attn = [dt for _, n, dt in rows if "attn_decomp_kernel<128, false>" in n]
    warm = [dt for i, dt in enumerate(attn) if i % (n_warm + n_post) < n_warm]
    post = [dt for i, dt in enumerate(attn) if i % (n_warm + n_post) >= n_warm]
    gram = [dt for _, n, dt in rows if "gram_t_kernel" in n]
    n_kv = [w.n_sink + w.n_cur + hs for hs in w.hist_per_step]
    fl = sum(attn_flops(w.n_q, nk, w.hidden) for nk in n_kv) / len(n_kv)
    lines = [
        f"# Kernel trace: {w.name}, {passes} steps (1 warmup + 1 timed)", "",
        "Command (run from the repository root on one MI355X):", "", "```",
        "cd /tmp && export TMPDIR=/tmp    # REPO: the repository root; OUT: a results directory",
        "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o kt -- "
        "python3 $REPO/bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-stream",
        f"python3 $REPO/bench.py --trace-summary $OUT/kt/kt_kernel_trace.csv",
        "```", "",
        "| Kernel | Calls | Avg (us) | Total (ms) | % |", "|---|---:|---:|---:|---:|",
    ]
    for k, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        if t / total < 1e-4:
            continue
        lines.append(f"| {k} | {c} | {t / c / 1e3:.1f} | {t / 1e6:.2f} | {100 * t / total:.2f} |")
    if warm:
        avg = sum(warm) / len(warm)
        lines += ["", f"Decomposable attention launches of the warmup pass: {len(warm)}, average "
                  f"{avg / 1e3:.1f} us for {fl / 1e12:.4f} TFLOP each = "
                  f"{fl / (avg * 1e-9) / 1e12:.1f} TFLOP/s ({100 * fl / (avg * 1e-9) / 1e12 / PEAK_BF16_TFLOPS:.1f} % of the "
                  f"dense bf16 peak)."]
    if post:
        lines.append(f"Post-absorption chunk attention launches (L-layers local only, F-layers "
                     f"full only): {len(post)}, average {sum(post) / len(post) / 1e3:.1f} us.")
    if gram:
        avg = sum(gram) / len(gram)
        gf = gram_flops(w.n_steps * w.n_q, w.hidden) * w.n_layers
        lines.append(f"Gram launches (all {w.n_layers} layers, all warmup tokens): {len(gram)}, "
                     f"average {avg / 1e3:.1f} us for {gf / 1e9:.1f} GFLOP = "
                     f"{gf / (avg * 1e-9) / 1e12:.1f} TFLOP/s.")
    proj = [dt for _, n, dt in rows
            if "nt_gemm256_kernel<false, false>" in n or "g256_kernel<0," in n]
    if proj:
        avg = sum(proj) / len(proj)
        pf = 2.0 * w.n_q * w.hidden * w.hidden
        lines.append(f"Output projections (post-absorption chunk): {len(proj)}, average "
                     f"{avg / 1e3:.1f} us for {pf / 1e9:.1f} GFLOP = "
                     f"{pf / (avg * 1e-9) / 1e12:.1f} TFLOP/s.")
    cw = [dt for _, n, dt in rows if "g256_kernel<1," in n]
    if cw:
        avg = sum(cw) / len(cw)
        cf = 2.0 * 2.0 * w.n_layers * w.hidden ** 3  # two bf16 planes of the fp32 operand
        lines.append(f"Y W_o and C W_o products (absorb, all layers, two bf16 planes of the fp32 "
                     f"operand): {len(cw)}, average {avg / 1e3:.1f} us = "
                     f"{cf / (avg * 1e-9) / 1e12:.1f} TFLOP/s.")
    return "\n".join(lines) + "\n"


def cpu_baseline(w: wl.Workload, n_rows: int):
    """The fp64 oracle on the host: decomposable attention for `n_rows` query
    rows x all heads at the last warmup step (full KV), plus one layer's
    closed-form absorb (ridge solve + error) at full hidden size."""
    import numpy as np
    from oracle import ispa_oracle as orc
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([p.get("num_threads", 1) for p in info] or [1])
        blas = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in info
                         if p.get("user_api") == "blas") or blas
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):  # pragma: no cover
        pass
    step = w.n_steps - 1
    st = wl.step_inputs(w, 0, step, n_q=n_rows)
    n_kv = w.n_sink + w.n_cur + w.hist_per_step[step]
    t0 = time.perf_counter()
    orc.decomposable_attention(st.q, st.k_sink, st.v_sink, st.k_cur, st.v_cur, st.k_hist,
                               st.v_hist, w.sm_scale)
    t_attn = time.perf_counter() - t0
    attn_tflops = attn_flops(n_rows, n_kv, w.hidden) / t_attn / 1e12
    del st
    # one layer's absorb on synthetic statistics of the right size (G SPD by
    # diagonal dominance, E symmetric); only the solve and the error are timed
    h = w.hidden
    rng = np.random.default_rng(0)
    r = rng.standard_normal((h, h)) / math.sqrt(h)
    g = np.eye(h) + 0.01 * (r + r.T)
    c = rng.standard_normal((h, h)) * 0.01
    r = rng.standard_normal((h, h)) / math.sqrt(h)
    e = 0.5 * np.eye(h) + 0.01 * (r + r.T)
    wo = rng.standard_normal((h, h)) * w.wo_std
    t0 = time.perf_counter()
    dw = orc.ridge_delta_w(g, c, wo, w.lam)
    orc.layer_error_from_stats(g, c, e, wo, dw, w.lam)
    t_abs = time.perf_counter() - t0
    # one layer-step's statistics over a token sample (plain matrix products)
    n_g = 1024
    xg = rng.standard_normal((n_g, h))
    dg = rng.standard_normal((n_g, h))
    t0 = time.perf_counter()
    orc.gram_statistics([xg], [dg])
    t_gram = time.perf_counter() - t0
    return {"value": round(attn_tflops, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model, "blas": blas,
            "gram_tflops": round(gram_flops(n_g, h) / t_gram / 1e12, 4),
            "gram_sample": f"{n_g} tokens x hidden {h}: {t_gram:.2f} s",
            "sample": (f"decomposable attention of {n_rows} query rows x {w.n_heads} heads at "
                       f"the last warmup step ({n_kv} keys; the oracle computes local, history "
                       f"and full attention separately, so it does ~2x the algorithmic FLOP "
                       f"counted here) took {t_attn:.2f} s; one layer's absorb (dense fp64 "
                       f"solve + error, hidden {h}) took {t_abs:.2f} s"),
            "absorb_ms_per_layer": round(t_abs * 1e3, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="wan14b_warmup", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=128)
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the measurements after the warmup step: the quantized variants, "
                         "the grouped launches, the long-horizon streaming comparison (ISPA vs "
                         "all-full) and the session")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB copy (reference for the HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--pmc-mfma-summary", metavar="MFMA_CSV",
                    help="print the matrix-core counter summary of a rocprofv3 --pmc run and exit")
    ap.add_argument("--trace-table", metavar="TRACE_CSV",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace CSV and exit")
    ap.add_argument("--trace-summary", metavar="TRACE_CSV",
                    help="print the summary of a rocprofv3 --kernel-trace CSV and exit")
    a = ap.parse_args()

    if a.trace_table:
        sys.stdout.write(trace_table(
            a.trace_table, "rocprofv3 --kernel-trace --stats --output-format csv -d "
            "$OUT/ktq -o ktq -- python3 $REPO/bench.py --steps 1 --warmup 0 "
            "--no-cpu-baseline"))
        return
    if a.trace_summary:
        sys.stdout.write(trace_summary(a.trace_summary, wl.WORKLOADS[a.workload], 2))
        return
    if a.pmc_mfma_summary:
        sys.stdout.write(pmc_mfma_summary(a.pmc_mfma_summary, wl.WORKLOADS[a.workload]))
        return
    if a.pmc_summary:
        sys.stdout.write(pmc_summary(a.pmc_summary[0], a.pmc_summary[1],
                                     wl.WORKLOADS[a.workload]))
        return

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import kv_cache_absorption_attn_amd as ispa

    w = wl.WORKLOADS[a.workload]
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = Inputs(w)
    ws = torch.empty(ispa.ispa_ridge_workspace_bytes(w.n_layers, w.hidden), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()

    for i in range(a.warmup):
        run_step(ispa, inp, ws, None)
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i} done", file=sys.stderr, flush=True)

    timing: dict = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        run_step(ispa, inp, ws, timing)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {a.steps} timed steps in {wall:.3f} s", file=sys.stderr, flush=True)

    if a.copy_calibration:
        copy_calibration()

    tot, n_attn = summarize_events(timing)
    K = a.steps
    n_kv = [w.n_sink + w.n_cur + hs for hs in w.hist_per_step]
    attn_fl = sum(attn_flops(w.n_q, nk, w.hidden) for nk in n_kv) * w.n_layers
    gram_fl = gram_flops(w.n_q, w.hidden) * w.n_steps * w.n_layers
    abs_fl = absorb_flops(w.hidden) * w.n_layers
    attn_ms = tot["attn"] / K
    attn_tflops = attn_fl / (attn_ms * 1e-3) / 1e12
    gram_tflops = gram_fl / (tot["gram"] / K * 1e-3) / 1e12
    absorb_ms = (tot["ridge"] + tot["score"] + tot["apply"]) / K
    absorb_tflops = abs_fl / ((tot["ridge"] + tot["score"]) / K * 1e-3) / 1e12
    n_launch = w.n_steps * w.n_layers
    sel = inp.selected.cpu().tolist()
    eps = inp.eps_rel.cpu().tolist()
    info = inp.info.cpu().tolist()
    order = sorted(range(w.n_layers), key=lambda i: (eps[i], i))
    gap = (eps[order[w.k_select]] - eps[order[w.k_select - 1]]
           if w.k_select < w.n_layers else None)

    attn_traffic = recorded_traffic("attn_decomp_kernel<128, false>")
    kv_bytes = sum(nk * w.n_heads * w.head_dim * 2 * 2 for nk in n_kv) * w.n_layers
    out = {
        "metric": METRIC,
        "value": round(attn_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(wall / K * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V with per-layer query temperature, "
                "W_o ~ N(0, 1/hidden))",
        "config": {"workload": w.name, "layers": w.n_layers, "heads": w.n_heads,
                   "head_dim": w.head_dim, "n_q": w.n_q, "n_sink": w.n_sink,
                   "n_cur": w.n_cur, "hist_per_step": list(w.hist_per_step),
                   "k_select": w.k_select, "lambda": w.lam},
        "attn_pct_bf16_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "attn_ms_per_step": round(attn_ms, 3),
        "dW_absorb_ms_per_layer": round(absorb_ms / w.n_layers, 3),
        "absorb_ms_per_step": round(absorb_ms, 3),
        "absorb_tflops": round(absorb_tflops, 2),
        "gram_tflops": round(gram_tflops, 2),
        "gram_pct_bf16_peak": round(100 * gram_tflops / PEAK_BF16_TFLOPS, 2),
        "gram_ms_per_step": round(tot["gram"] / K, 3),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": attn_traffic,
                     "kernel": "attn_decomp_kernel<128, false>",
                     "launches_per_step": n_launch,
                     "flop_per_launch_avg": attn_fl / n_launch},
        "attn_kv_stream_gbs": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1),
        "attn_traffic_gbs": (round(attn_traffic / (attn_ms / n_launch * 1e-3) / 1e9, 1)
                             if attn_traffic else None),
        "gram_traffic_bytes_per_launch": recorded_traffic("gram_t_kernel"),
        "post_absorb_chunk_ms": round(tot["post"] / K, 3),
        "selected_layers": [i for i, s in enumerate(sel) if s],
        "eps_rel_range": [min(eps), max(eps)],
        "eps_gap_at_k": gap,
        "solve_info_nonzero": sum(1 for v in info if v != 0),
    }
    if not a.no_stream:
        del inp, ws, timing
        torch.cuda.empty_cache()
        print("[bench] E4M3 attention and W8A8 projection", file=sys.stderr, flush=True)
        out["quantized"] = quantized_measure(ispa, w)
        torch.cuda.empty_cache()
        print("[bench] grouped launches of concurrent instances", file=sys.stderr, flush=True)
        out["multi_instance"] = multi_instance_measure(ispa, w)
        torch.cuda.empty_cache()
        out["gram_deferred"] = gram_deferred_measure(ispa, w)
        torch.cuda.empty_cache()
        out["stream"] = stream_measure(ispa, w)
        torch.cuda.empty_cache()
        out["session"] = session_measure(ispa, w)
        torch.cuda.empty_cache()
        out["session_quantized"] = session_measure(
            ispa, w, flags=ispa.SESSION_W8A8 | ispa.SESSION_FP8_ATTN)
        s0, s1 = out["session"]["stream_chunk_ms"], out["session_quantized"]["stream_chunk_ms"]
        out["session_quantized"]["stream_speedup_vs_bf16"] = round(sum(s0) / sum(s1), 3)
    if not a.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

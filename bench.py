#!/usr/bin/env python3
"""Benchmark of the ISPA hot path on one MI355X.

One step = the whole warmup-to-absorption pass of the 14B-class workload:
for each of 4 warmup chunks (history 0 -> 36 latent frames) and each of the
40 layers, the decomposable attention (O_full, X = O_local, D) and the Gram
accumulation; then, batched over the 40 layers, the ridge solve for dW, the
layer errors, the selection of K = 20 layers and the in-place bf16 update of
their output projections. All inputs are resident in HBM before timing
starts; W_o is restored from a pristine copy at the start of every step.

Prints one JSON line. `value` is the decomposable-attention throughput in
algorithmic TFLOP/s (4 * n_q * n_kv * hidden per launch, QK^T and PV only)
measured with HIP events around the attention launches of the timed steps.
"""
from __future__ import annotations

import argparse
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
        self.dd = torch.empty(w.n_q, h, dtype=bf, device=dev)
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
    for s in range(w.n_steps):
        for l in range(w.n_layers):
            kh, vh = inp.hist_view(l, s)
            mark("attn0")
            ispa.ispa_attn_decomp(inp.q[l][s], inp.k_sink[l], inp.v_sink[l], inp.k_cur[l][s],
                                  inp.v_cur[l][s], kh, vh, w.sm_scale, o_local=inp.x,
                                  o_full=inp.o_full, d_out=inp.dd)
            mark("attn1")
            ispa.ispa_gram_accumulate(inp.x, inp.dd, inp.G[l], inp.C[l], inp.E[l],
                                      zero_first=(s == 0))
            mark("gram1")
    mark("absorb0")
    ispa.ispa_ridge_solve(inp.G, inp.C, inp.wo, w.lam, inp.dW, inp.info, ws)
    mark("ridge1")
    ispa.ispa_layer_score(inp.G, inp.C, inp.E, inp.wo, inp.dW, w.lam, inp.info, w.k_select, ws,
                          inp.eps_abs, inp.eps_rel, inp.selected)
    mark("score1")
    ispa.ispa_apply_dW(inp.selected, inp.dW, inp.wo)
    mark("absorb1")
    if timing is not None:
        timing.setdefault("events", []).append(ev)


def summarize_events(timing):
    tot = {"attn": 0.0, "gram": 0.0, "ridge": 0.0, "score": 0.0, "apply": 0.0}
    n_attn = 0
    for ev in timing["events"]:
        prev = None
        for tag, e in ev:
            if prev is not None:
                dt = prev[1].elapsed_time(e)
                key = {("attn0", "attn1"): "attn", ("attn1", "gram1"): "gram",
                       ("absorb0", "ridge1"): "ridge", ("ridge1", "score1"): "score",
                       ("score1", "absorb1"): "apply"}.get((prev[0], tag))
                if key:
                    tot[key] += dt
                    n_attn += key == "attn"
            prev = (tag, e)
    return tot, n_attn


def cpu_baseline(w: wl.Workload, n_rows: int):
    """The fp64 oracle on the host: decomposable attention for `n_rows` query
    rows x all heads at the last warmup step (full KV), plus one layer's
    closed-form absorb (ridge solve + error) at full hidden size."""
    import numpy as np
    from oracle import ispa_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
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
    return {"value": round(attn_tflops, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
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
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
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

    out = {
        "metric": "decomp-attention TFLOP/s (% bf16 MFMA peak) + dW absorb ms/layer, 14B-class",
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
        "absorb_fp32_tflops": round(absorb_tflops, 2),
        "gram_tflops": round(gram_tflops, 2),
        "gram_pct_bf16_peak": round(100 * gram_tflops / PEAK_BF16_TFLOPS, 2),
        "gram_ms_per_step": round(tot["gram"] / K, 3),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_decomp_kernel<128>",
                     "launches_per_step": n_launch,
                     "flop_per_launch_avg": attn_fl / n_launch},
        "selected_layers": [i for i, s in enumerate(sel) if s],
        "eps_rel_range": [min(eps), max(eps)],
        "eps_gap_at_k": gap,
        "solve_info_nonzero": sum(1 for v in info if v != 0),
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

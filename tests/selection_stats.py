"""Oracle statistics of a whole multi-layer warmup, for the layer-selection
parity tests (ISPA paper §3.3: every layer gets an error from its warmup
statistics and the K lowest become L-layers; Table 1 caption: K = x N).

For each layer the oracle runs its attention over `rows` sampled query rows
of every warmup step (attention rows are independent, so each sampled row is
exact) at the full KV lengths of the workload, keeps the bf16 activations a
model stores (oracle.stored_activations) and sums G, C, E over the steps.
The statistics are rounded to fp32, the form the GPU solve takes; the
oracle's fp64 ridge solution and error are computed from those same fp32
values.

Per layer the cost is dominated by drawing the seeded inputs, so layers run
in a pool of worker processes started with the spawn method (the workers
import only `workloads` and `oracle`, never the GPU package) and each worker
limits its BLAS to one thread.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
from typing import Dict, List

import numpy as np


_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def layer_statistics(wname: str, layer: int, rows_per_step: int, with_oracle: bool) -> Dict:
    """The oracle's fp32 statistics of one layer (and, when with_oracle, its
    fp64 dW and errors on them). Inputs are those of workloads.step_inputs;
    the sink and the full-length history are drawn once per layer (the same
    seeds give the same bits as drawing them per step)."""
    import workloads as wl
    from oracle import ispa_oracle as orc

    w = wl.WORKLOADS[wname]
    nh, d = w.n_heads, w.head_dim
    std = w.qkv_std
    temp = wl.layer_temperatures(w)[layer]
    ks = wl.draw_bf16((w.n_sink, nh, d), std, wl.rng_for(w, layer, 0, wl.T_K_SINK))
    vs = wl.draw_bf16((w.n_sink, nh, d), std, wl.rng_for(w, layer, 0, wl.T_V_SINK))
    kh_all = wl.draw_bf16((w.n_hist_max, nh, d), std, wl.rng_for(w, layer, 0, wl.T_K_HIST))
    vh_all = wl.draw_bf16((w.n_hist_max, nh, d), std, wl.rng_for(w, layer, 0, wl.T_V_HIST))
    rows = np.linspace(0, w.n_q - 1, rows_per_step).astype(np.int64)
    xs, ds = [], []
    for s in range(w.n_steps):
        q = wl.draw_bf16((w.n_q, nh, d), std * temp, wl.rng_for(w, layer, s, wl.T_Q))[rows]
        kc = wl.draw_bf16((w.n_cur, nh, d), std, wl.rng_for(w, layer, s, wl.T_K_CUR))
        vc = wl.draw_bf16((w.n_cur, nh, d), std, wl.rng_for(w, layer, s, wl.T_V_CUR))
        n = w.hist_per_step[s]
        r = orc.decomposable_attention(q, ks, vs, kc, vc, kh_all[:n], vh_all[:n], w.sm_scale)
        x, dd = orc.stored_activations(r["o_local"], r["o_full"])
        xs.append(x)
        ds.append(dd)
        del r, kc, vc
    del kh_all, vh_all
    g, c, e = (a.astype(np.float32) for a in orc.gram_statistics(xs, ds))
    wo = wl.output_projection(w, layer)
    out = {"layer": layer, "g": g, "c": c, "e": e, "wo": wo.astype(np.float32)}
    if with_oracle:
        g64, c64, e64 = (a.astype(np.float64) for a in (g, c, e))
        dw = orc.ridge_delta_w(g64, c64, wo, w.lam)
        ea, er = orc.layer_error_from_stats(g64, c64, e64, wo, dw, w.lam)
        out.update(dw=dw.astype(np.float32), eps_abs=ea, eps_rel=er)
    return out


def _worker(args):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return layer_statistics(*args)


def warmup_statistics(wname: str, rows_per_step: int, with_oracle: bool = True,
                      workers: int = 0, progress=None) -> List[Dict]:
    """layer_statistics for every layer of the workload, in a spawn pool;
    progress(message) is called as each layer finishes."""
    import workloads as wl

    w = wl.WORKLOADS[wname]
    if workers <= 0:
        workers = min(16, os.cpu_count() or 1)
    ctx = mp.get_context("spawn")
    jobs = [(wname, l, rows_per_step, with_oracle) for l in range(w.n_layers)]
    # one BLAS thread per worker, fixed before the workers import numpy
    saved = {v: os.environ.get(v) for v in _THREAD_VARS}
    os.environ.update({v: "1" for v in _THREAD_VARS})
    try:
        res = []
        with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
            for fut in cf.as_completed([ex.submit(_worker, j) for j in jobs]):
                res.append(fut.result())
                if progress is not None:
                    progress(f"  layer {res[-1]['layer']} done ({len(res)}/{len(jobs)})")
    finally:
        for v, val in saved.items():
            if val is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = val
    return sorted(res, key=lambda r: r["layer"])

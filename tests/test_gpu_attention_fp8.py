"""GPU parity of the E4M3 decomposable attention (ispa_attn_decomp_fp8) and
of the key mean (ispa_key_mean) against the oracle's quantized attention
(oracle.decomposable_attention_fp8, the same codes and scales from the same
inputs and the same smoothing vector).

Tolerances: the attention bounds of the bf16 path (outputs max-abs 1e-2 of
max(1, max|O|), relative Frobenius 1e-2; LSE 1e-3) plus the accumulation
inside the E4M3 matrix cores. One instruction keeps up to ~1.3e-4 of the
sum of |products| it adds (measured); with a 4x margin a score may be off by
delta = 5e-4 * scale * sum_c |dq(q_c) dq(k_c)|. An LSE moves by at most the
largest delta of its query; an output by at most 2 delta max|V|.
"""
import dataclasses

import numpy as np
import pytest
import torch

import kv_cache_absorption_attn_amd as ispa
import workloads as wl
from oracle import ispa_oracle as orc
from tests.gpu_helpers import O_RELFRO, compare_attention, dev_bf16, host, log

pytestmark = pytest.mark.gpu

ALL = ("o_local", "lse_local", "o_hist", "lse_hist", "o_full", "lse_full", "d")


def custom(n_q, n_sink, n_cur, n_hist, heads, seed=0):
    return dataclasses.replace(wl.TINY, name=f"fp8custom{seed}", config_id=200 + seed,
                               n_heads=heads, head_dim=128, n_q=n_q, n_sink=n_sink,
                               n_cur=n_cur, hist_per_step=(n_hist,), qkv_std=1.0)


def run_fp8(st, scale, mu, outputs=ALL):
    q = dev_bf16(st.q)
    n_q, nh, d = q.shape
    kv = [dev_bf16(a) if a.shape[0] else None for a in
          (st.k_sink, st.v_sink, st.k_cur, st.v_cur, st.k_hist, st.v_hist)]
    ws = torch.empty(ispa.ispa_attn_fp8_workspace_bytes(n_q, st.k_sink.shape[0],
                                                        st.k_cur.shape[0], st.k_hist.shape[0],
                                                        nh, d),
                     dtype=torch.uint8, device="cuda")
    out, kw = {}, {}
    for name in outputs:
        if name.startswith("lse"):
            t = torch.full((nh, n_q), float("nan"), dtype=torch.float32, device="cuda")
        else:
            t = torch.full((n_q, nh * d), float("nan"), dtype=torch.bfloat16, device="cuda")
        out[name] = t
        kw["d_out" if name == "d" else name] = t
    ispa.ispa_attn_decomp_fp8(q, *kv, scale, ws, k_mean=None if mu is None else dev_bf16(mu),
                              **kw)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def accumulation_delta(q, keys, scale, mu, heads=None):
    """delta[h, i] = 5e-4 * scale * max_j sum_c |dq(q_ic) dq(k_jc)| over all keys."""
    qc, qs = orc.quantize_queries(q)
    qd = np.abs(orc.e4m3_decode(qc) * qs.T[:, :, None])
    kd = np.abs(np.concatenate([orc.dequantized_keys(k, mu) for k in keys if k.shape[0]]))
    nh = q.shape[1]
    out = np.zeros((nh, q.shape[0]))
    for h in range(nh):
        out[h] = (qd[:, h, :] @ kd[:, h, :].T).max(axis=1)
    return 5e-4 * scale * out


def check(gpu, ref, delta, vmax):
    lse_keys = [k for k in gpu if k.startswith("lse")]
    o_keys = [k for k in gpu if not k.startswith("lse")]
    for k in lse_keys:
        g, r = gpu[k], ref[k]
        fin = np.isfinite(r)
        assert np.array_equal(np.isfinite(g), fin), f"{k}: non-finite pattern differs"
        err = np.abs(g[fin] - r[fin])
        tol = (1e-3 + delta)[fin]
        log(f"  {k}: max err {err.max() if err.size else 0:.2e}, "
            f"max err/bound {np.max(err / tol) if err.size else 0:.3f}")
        assert np.all(err <= tol), k
    extra = 2.0 * float(delta.max()) * vmax
    rep = compare_attention({k: gpu[k] for k in o_keys}, ref, keys=o_keys,
                            o_tol=1e-2 + extra, lse_tol=1e-3, rel=O_RELFRO)
    log(f"  outputs (max abs, rel fro): {rep}; accumulation term {extra:.2e}")


def oracle_fp8(st, scale, mu, rows=None, heads=None):
    sel = lambda a: a if heads is None else a[:, heads]
    q = sel(st.q if rows is None else st.q[rows])
    m = None if mu is None else (mu if heads is None else mu[heads])
    segs = [sel(a) for a in (st.k_sink, st.v_sink, st.k_cur, st.v_cur, st.k_hist, st.v_hist)]
    ref = orc.decomposable_attention_fp8(q, *segs, scale, m)
    delta = accumulation_delta(q, segs[0::2], scale, m)
    return ref, delta


@pytest.mark.parametrize("n_q,n_sink,n_cur,n_hist,heads,smooth", [
    (300, 64, 200, 333, 2, True),     # ragged query, key and tile tails; several tiles
    (257, 100, 37, 0, 3, True),       # empty history
    (64, 1, 1, 65, 1, False),         # single-key segments, no smoothing
    (513, 0, 130, 700, 2, True),      # no sink
])
def test_fp8_all_outputs(n_q, n_sink, n_cur, n_hist, heads, smooth):
    w = custom(n_q, n_sink, n_cur, n_hist, heads, seed=n_q)
    st = wl.step_inputs(w, 0, 0)
    scale = 1.0 / np.sqrt(128)
    mu = orc.bf16_round(orc.key_mean(st.k_sink, st.k_cur, st.k_hist)) if smooth else None
    log(f"fp8 attn n_q={n_q} sink={n_sink} cur={n_cur} hist={n_hist} heads={heads} "
        f"smooth={smooth}")
    gpu = run_fp8(st, scale, mu)
    ref, delta = oracle_fp8(st, scale, mu)
    vmax = max(float(np.max(np.abs(a))) for a in (st.v_sink, st.v_cur, st.v_hist) if a.size)
    check(gpu, ref, delta, vmax)


def test_fp8_full_only_and_biased_keys():
    """The one-pass path (only O_full / LSE_full) on keys with a common bias
    10x their spread, smoothed by the GPU's own key mean (checked against
    the oracle's mean first, then passed to both sides)."""
    w = custom(400, 64, 256, 500, 2, seed=7)
    st = wl.step_inputs(w, 0, 0)
    bias = 10.0 * wl.random_bf16((1, 2, 128), 1.0, 77)
    st = dataclasses.replace(st, k_sink=orc.bf16_round(st.k_sink + bias),
                             k_cur=orc.bf16_round(st.k_cur + bias),
                             k_hist=orc.bf16_round(st.k_hist + bias))
    mu_d = torch.empty((2, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ispa.ispa_key_mean_workspace_bytes(2, 128), dtype=torch.uint8,
                     device="cuda")
    ispa.ispa_key_mean(dev_bf16(st.k_sink), dev_bf16(st.k_cur), dev_bf16(st.k_hist), mu_d, ws)
    torch.cuda.synchronize()
    mu = host(mu_d)
    exact = orc.key_mean(st.k_sink, st.k_cur, st.k_hist)
    assert np.all(np.abs(mu - exact) <= 2.0 ** -7 * np.abs(exact) + 1e-6)
    scale = 1.0 / np.sqrt(128)
    gpu = run_fp8(st, scale, mu, outputs=("o_full", "lse_full"))
    ref, delta = oracle_fp8(st, scale, mu)
    check(gpu, {k: ref[k] for k in ("o_full", "lse_full")}, delta,
          max(float(np.max(np.abs(a))) for a in (st.v_sink, st.v_cur, st.v_hist)))
    # and the quantized result stays close to the exact attention
    plain = orc.decomposable_attention(st.q, st.k_sink, st.v_sink, st.k_cur, st.v_cur,
                                       st.k_hist, st.v_hist, scale)
    rel = np.linalg.norm(gpu["o_full"] - plain["o_full"]) / np.linalg.norm(plain["o_full"])
    lse = np.max(np.abs(gpu["lse_full"] - plain["lse_full"]))
    log(f"  vs exact attention: O rel fro {rel:.4f}, LSE max abs {lse:.4f}")
    assert rel <= 0.05 and lse <= 0.1


@pytest.mark.parametrize("segs", [(10, 20, 30), (0, 300, 0), (1, 0, 5000)])
def test_key_mean(segs):
    keys = [wl.random_bf16((n, 3, 128), 1.0, 90 + i) + 3.0 * (i + 1) for i, n in enumerate(segs)]
    keys = [orc.bf16_round(k) for k in keys]
    mu_d = torch.empty((3, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ispa.ispa_key_mean_workspace_bytes(3, 128), dtype=torch.uint8,
                     device="cuda")
    ispa.ispa_key_mean(*[dev_bf16(k) if k.shape[0] else None for k in keys], mu_d, ws)
    torch.cuda.synchronize()
    exact = orc.key_mean(*keys)
    err = np.abs(host(mu_d) - exact)
    assert np.all(err <= 2.0 ** -7 * np.abs(exact) + 1e-6)


def test_fp8_wan14_sampled_rows_and_heads():
    """14B-class last warmup step (40 heads, 4680 queries, 1560 + 4680 local
    and 56160 history keys), smoothed by the oracle's key mean; the oracle
    runs on 32 sampled query rows of 3 heads (rows and heads are
    independent, quantization blocks never span heads)."""
    w = wl.WAN14_WARMUP
    st = wl.step_inputs(w, 0, 3)
    log(f"fp8 attn full-size {w.name}: n_q={st.q.shape[0]} hist={st.k_hist.shape[0]}")
    mu = orc.bf16_round(orc.key_mean(st.k_sink, st.k_cur, st.k_hist))
    gpu = run_fp8(st, w.sm_scale, mu)
    rows = np.sort(np.random.default_rng(5).choice(st.q.shape[0], 32, replace=False))
    heads = [0, 17, 39]
    ref, delta = oracle_fp8(st, w.sm_scale, mu, rows=rows, heads=heads)
    d = st.q.shape[2]
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    sub = {k: (v[heads][:, rows] if k.startswith("lse") else v[rows][:, cols])
           for k, v in gpu.items()}
    vmax = max(float(np.max(np.abs(a[:, heads]))) for a in (st.v_sink, st.v_cur, st.v_hist))
    check(sub, ref, delta, vmax)


def test_fp8_wan13_layer_sampled_rows():
    """1.3B-class layer (12 heads, 4680 queries, 1560 + 4680 local and 28080
    history keys), smoothed by the oracle's key mean; 48 sampled query rows
    of every head against the oracle."""
    w = wl.WAN13_LAYER
    st = wl.step_inputs(w, 0, 0)
    log(f"fp8 attn {w.name}: n_q={st.q.shape[0]} hist={st.k_hist.shape[0]}")
    mu = orc.bf16_round(orc.key_mean(st.k_sink, st.k_cur, st.k_hist))
    gpu = run_fp8(st, w.sm_scale, mu)
    rows = np.sort(np.random.default_rng(6).choice(st.q.shape[0], 48, replace=False))
    ref, delta = oracle_fp8(st, w.sm_scale, mu, rows=rows)
    sub = {k: (v[:, rows] if k.startswith("lse") else v[rows]) for k, v in gpu.items()}
    vmax = max(float(np.max(np.abs(a))) for a in (st.v_sink, st.v_cur, st.v_hist))
    check(sub, ref, delta, vmax)

"""GPU parity of the grouped launches (multi-instance batching: several
concurrent streams, each with its own KV cache and its own W + dW, ISPA
paper §3.3's instance-specific state).

Every instance of a grouped launch must equal the oracle at the bounds of
its single-call counterpart (attention: max-abs 1e-2, relative Frobenius
1e-2, LSE 1e-3; projection: half a bf16 ulp plus 1e-3 of the row scale),
and be bit-identical to that counterpart run alone.
"""
import dataclasses

import numpy as np
import pytest
import torch

import kv_cache_absorption_attn_amd as ispa
import workloads as wl
from oracle import ispa_oracle as orc
from tests.gpu_helpers import compare_attention, dev_bf16, host, log

pytestmark = pytest.mark.gpu

ALL = ("o_local", "lse_local", "o_hist", "lse_hist", "o_full", "lse_full", "d_out")


def inputs(n_q, n_sink, n_cur, n_hist, heads, d, seed):
    w = dataclasses.replace(wl.TINY, name=f"group{seed}", config_id=300 + seed, n_heads=heads,
                            head_dim=d, n_q=n_q, n_sink=n_sink, n_cur=n_cur,
                            hist_per_step=(n_hist,), qkv_std=1.0)
    return wl.step_inputs(w, 0, 0)


def device_call(st, outputs):
    n_q, nh, d = st.q.shape
    c = {"q": dev_bf16(st.q)}
    for name in ("k_sink", "v_sink", "k_cur", "v_cur", "k_hist", "v_hist"):
        a = getattr(st, name)
        c[name] = dev_bf16(a) if a.shape[0] else None
    for name in outputs:
        shape = (nh, n_q) if name.startswith("lse") else (n_q, nh * d)
        dt = torch.float32 if name.startswith("lse") else torch.bfloat16
        c[name] = torch.full(shape, float("nan"), dtype=dt, device="cuda")
    return c


def single(c, scale):
    kw = {k: v for k, v in c.items() if k in ALL}
    fresh = {k: torch.full_like(v, float("nan")) for k, v in kw.items()}
    ispa.ispa_attn_decomp(c["q"], c["k_sink"], c["v_sink"], c["k_cur"], c["v_cur"], c["k_hist"],
                          c["v_hist"], scale, **fresh)
    return fresh


@pytest.mark.parametrize("d", [128, 64])
def test_grouped_attention(d):
    """Four instances: all outputs with history, the one-pass full-only path
    on a longer history, local-only output without history, and an instance
    with no queries (skipped)."""
    scale = 1.0 / np.sqrt(d)
    specs = [((300, 64, 200, 333, 2, d, 1), ALL),
             ((257, 32, 100, 900, 2, d, 2), ("o_full", "lse_full")),
             ((64, 1, 70, 0, 2, d, 3), ("o_local", "lse_local")),
             ((0, 16, 16, 16, 2, d, 4), ("o_full",))]
    sts = [inputs(*a) for a, _ in specs]
    calls = [device_call(st, outs) for st, (_, outs) in zip(sts, specs)]
    log(f"grouped attention d={d}: {[a for a, _ in specs]}")
    ispa.ispa_attn_decomp_grouped(calls, scale)
    torch.cuda.synchronize()
    for st, c, (args, outs) in zip(sts, calls, specs):
        if st.q.shape[0] == 0:
            continue
        alone = single(c, scale)
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(c[k], alone[k]) or (torch.isnan(c[k]).equal(torch.isnan(alone[k]))
                                                    and torch.equal(c[k].nan_to_num(),
                                                                    alone[k].nan_to_num())), k
        ref = orc.decomposable_attention(st.q, st.k_sink, st.v_sink, st.k_cur, st.v_cur,
                                         st.k_hist, st.v_hist, scale)
        gpu = {("d" if k == "d_out" else k): host(c[k]) for k in outs}
        rep = compare_attention(gpu, ref)
        log(f"  instance {args}: {rep}")


def test_grouped_projection_per_instance_weights():
    """Five instances with their own weights (W + dW of each stream): ragged
    and empty token counts, several tiles."""
    h_in, h_out = 256, 392
    ns = [300, 0, 1, 517, 256]
    xs = [wl.random_bf16((n, h_in), 1.0, 400 + i) for i, n in enumerate(ns)]
    ws = [wl.random_bf16((h_out, h_in), 1.0 / np.sqrt(h_in), 410 + i) for i in range(len(ns))]
    xd, wd = [dev_bf16(x) for x in xs], [dev_bf16(w) for w in ws]
    ys = [torch.full((n, h_out), float("nan"), dtype=torch.bfloat16, device="cuda") for n in ns]
    log(f"grouped projection {ns} x {h_in} -> {h_out}")
    ispa.ispa_project_grouped(xd, wd, ys)
    torch.cuda.synchronize()
    for x, w, xg, wg, y in zip(xs, ws, xd, wd, ys):
        alone = torch.full_like(y, float("nan"))
        if x.shape[0]:
            ispa.ispa_project(xg, wg, alone)
        torch.cuda.synchronize()
        assert torch.equal(y, alone)
        ref = orc.project(x, w)
        got = host(y)
        tol = 2.0 ** -9 * np.abs(ref) + 1e-3 * (np.abs(x) @ np.abs(w).T)
        assert np.all(np.abs(got - ref) <= tol)


def test_grouped_attention_eight_instances_wan13_heads():
    """The largest group: eight 1.3B-shaped instances (12 heads of 128) with
    different history lengths, O_full only, against single launches."""
    scale = 1.0 / np.sqrt(128)
    sts = [inputs(512, 128, 256, 64 * i + 7, 12, 128, 20 + i) for i in range(8)]
    calls = [device_call(st, ("o_full", "lse_full")) for st in sts]
    ispa.ispa_attn_decomp_grouped(calls, scale)
    torch.cuda.synchronize()
    for st, c in zip(sts, calls):
        alone = single(c, scale)
        torch.cuda.synchronize()
        assert torch.equal(c["o_full"], alone["o_full"])
        assert torch.equal(c["lse_full"], alone["lse_full"])
    rows = np.arange(0, 512, 37)
    for st, c in zip(sts[::3], calls[::3]):
        ref = orc.decomposable_attention(st.q[rows], st.k_sink, st.v_sink, st.k_cur, st.v_cur,
                                         st.k_hist, st.v_hist, scale)
        gpu = {"o_full": host(c["o_full"])[rows], "lse_full": host(c["lse_full"])[:, rows]}
        compare_attention(gpu, ref)


def test_grouped_mixed_large_and_small():
    """A call whose grid covers half the chip (16 query tiles x 8 heads = 128
    workgroups) runs as a launch of its own inside the grouped call; two
    small calls share the grouped launch. All equal their single calls."""
    scale = 1.0 / np.sqrt(128)
    sts = [inputs(4096, 64, 128, 200, 8, 128, 40), inputs(100, 64, 64, 300, 8, 128, 41),
           inputs(300, 32, 96, 0, 8, 128, 42)]
    calls = [device_call(st, ("o_local", "o_full", "d_out", "lse_full")) for st in sts]
    ispa.ispa_attn_decomp_grouped(calls, scale)
    torch.cuda.synchronize()
    for st, c in zip(sts, calls):
        alone = single(c, scale)
        torch.cuda.synchronize()
        for k in ("o_local", "o_full", "d_out", "lse_full"):
            assert torch.equal(c[k], alone[k]), k
    rows = np.arange(0, 4096, 97)
    st, c = sts[0], calls[0]
    ref = orc.decomposable_attention(st.q[rows], st.k_sink, st.v_sink, st.k_cur, st.v_cur,
                                     st.k_hist, st.v_hist, scale)
    gpu = {"o_local": host(c["o_local"])[rows], "o_full": host(c["o_full"])[rows],
           "d": host(c["d_out"])[rows], "lse_full": host(c["lse_full"])[:, rows]}
    compare_attention(gpu, ref)


def test_grouped_sessions_match_single_sessions():
    """Two concurrent sessions (own weights, own streams of K/V/Q) stepped
    layer by layer through ispa_session_layer_grouped, beside twin sessions
    stepped alone with ispa_session_layer: every output bit-identical, the
    same events, through warmup, absorption and streaming (drift scores on,
    threshold out of reach)."""
    L, nh, d, ns, nc, t_warm, n_chunks = 3, 2, 64, 64, 256, 2, 5
    h = nh * d
    scale = 1.0 / np.sqrt(d)
    rnd = lambda shape, seed, std=1.0: wl.random_bf16(shape, std, 7000 + seed)
    kw = dict(n_heads=nh, head_dim=d, n_sink=ns, n_cur=nc, hist_capacity=8 * nc, k_select=1,
              t_warm=t_warm, sm_scale=scale, lam=1e-2, drift_threshold=1e30, drift_stride=2)
    wos = [dev_bf16(rnd((L, h, h), 100 * i, 1.0 / np.sqrt(h))) for i in range(2)]
    grouped = [ispa.Session(wos[i], **kw) for i in range(2)]
    alone = [ispa.Session(wos[i], **kw) for i in range(2)]
    try:
        for i in range(2):
            for l in range(L):
                k, v = dev_bf16(rnd((ns, nh, d), 10 * i + l)), dev_bf16(rnd((ns, nh, d), 50 + l))
                grouped[i].cache.write(l, k, v, sink=True)
                alone[i].cache.write(l, k, v, sink=True)
        ys_g = [torch.empty((nc, h), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        ys_a = [torch.empty((nc, h), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        for c in range(n_chunks):
            for i in range(2):
                for l in range(L):
                    k = dev_bf16(rnd((nc, nh, d), 1000 * c + 10 * i + l))
                    v = dev_bf16(rnd((nc, nh, d), 1000 * c + 10 * i + l + 500))
                    grouped[i].cache.write(l, k, v)
                    alone[i].cache.write(l, k, v)
            for l in range(L):
                qs = [dev_bf16(rnd((nc, nh, d), 90000 + 100 * c + 10 * i + l, 0.5 + l))
                      for i in range(2)]
                ispa.ispa_session_layer_grouped(grouped, l, qs, ys_g)
                for i in range(2):
                    alone[i].layer(l, qs[i], ys_a[i])
                torch.cuda.synchronize()
                for i in range(2):
                    assert torch.equal(ys_g[i], ys_a[i]), f"chunk {c} layer {l} session {i}"
            ev_g = [sess.end_chunk() for sess in grouped]
            ev_a = [sess.end_chunk() for sess in alone]
            log(f"chunk {c}: events grouped {ev_g} alone {ev_a}")
            assert ev_g == ev_a
        for sg, sa in zip(grouped, alone):
            st_g, loc_g, _, dr_g = sg.state()
            st_a, loc_a, _, dr_a = sa.state()
            assert loc_g == loc_a and st_g.phase == st_a.phase == 1
            assert dr_g == dr_a
    finally:
        for sess in grouped + alone:
            sess.close()

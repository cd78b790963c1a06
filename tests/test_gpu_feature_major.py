"""GPU parity of the feature-major warmup path: ispa_attn_decomp_t (X and D
written token-contiguous per feature) and ispa_gram_accumulate_t (the
statistics from those operands), against the oracle and, bit for bit,
against the token-major entry points on the same inputs.

Tolerances as in the attention and absorb tests: attention outputs max-abs
<= 1e-2 and relative Frobenius <= 1e-2; statistics relative Frobenius
<= 1e-5 (fp32 accumulation of exact bf16 products); G and E exactly
symmetric.
"""
import dataclasses

import numpy as np
import pytest
import torch

import kv_cache_absorption_attn_amd as ispa
import workloads as wl
from oracle import ispa_oracle as orc
from tests.gpu_helpers import compare_attention, dev_bf16, host, log, run_attention

pytestmark = pytest.mark.gpu

GRAM_REL = 1e-5


def relfro(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))


def custom(n_q, n_sink, n_cur, n_hist, heads, d, seed=0):
    return dataclasses.replace(wl.TINY, name=f"fm{seed}", config_id=200 + seed, n_heads=heads,
                               head_dim=d, n_q=n_q, n_sink=n_sink, n_cur=n_cur,
                               hist_per_step=(n_hist,), qkv_std=1.0)


def attention_t(st, scale, ld, col):
    """ispa_attn_decomp_t into columns [col, col + n_q) of [h, ld] buffers
    pre-filled with a sentinel; returns the X^T, D^T and O_F buffers."""
    q = dev_bf16(st.q)
    n_q, nh, d = q.shape
    kv = [dev_bf16(a) if a.shape[0] else None for a in
          (st.k_sink, st.v_sink, st.k_cur, st.v_cur, st.k_hist, st.v_hist)]
    h = nh * d
    xt = torch.full((h, ld), 7.0, dtype=torch.bfloat16, device="cuda")
    dt = torch.full((h, ld), 7.0, dtype=torch.bfloat16, device="cuda")
    o_full = torch.full((n_q, h), float("nan"), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_attn_decomp_t(q, *kv, scale, xt, dt, col=col, o_full=o_full)
    torch.cuda.synchronize()
    return xt, dt, o_full


@pytest.mark.parametrize("n_q,n_sink,n_cur,n_hist,heads,d,ld,col",
                         [(200, 37, 101, 301, 3, 128, 216, 8),
                          (130, 64, 70, 0, 2, 128, 136, 0),
                          (300, 40, 90, 200, 2, 64, 640, 320),
                          (64, 32, 96, 256, 2, 64, 64, 0)])
def test_attention_feature_major_outputs(n_q, n_sink, n_cur, n_hist, heads, d, ld, col):
    """X^T and D^T equal the token-major O_local and D transposed, bit for
    bit; O_full likewise; columns outside [col, col + n_q) are untouched; and
    all of them against the oracle. Ragged query tiles, an empty history
    (D = 0 exactly), head_dim 64 and 128, column offsets."""
    w = custom(n_q, n_sink, n_cur, n_hist, heads, d, seed=n_q + d)
    log(f"attn feature-major n_q={n_q} hist={n_hist} d={d} ld={ld} col={col}")
    st = wl.step_inputs(w, 0, 0, q_gain=2.0)
    scale = 1.0 / np.sqrt(d)
    ref_gpu, _ = run_attention(st, scale, outputs=("o_local", "o_full", "d"))
    xt, dt, o_full = attention_t(st, scale, ld, col)
    xh, dh = host(xt), host(dt)
    np.testing.assert_array_equal(xh[:, col:col + n_q].T, ref_gpu["o_local"])
    np.testing.assert_array_equal(dh[:, col:col + n_q].T, ref_gpu["d"])
    for a in (xh, dh):
        assert np.all(a[:, :col] == 7.0) and np.all(a[:, col + n_q:] == 7.0)
    np.testing.assert_array_equal(host(o_full), ref_gpu["o_full"])
    if n_hist == 0:
        assert np.all(dh[:, col:col + n_q] == 0)
    ref = orc.decomposable_attention(st.q, st.k_sink, st.v_sink, st.k_cur, st.v_cur, st.k_hist,
                                     st.v_hist, scale)
    got = {"o_local": xh[:, col:col + n_q].T, "d": dh[:, col:col + n_q].T}
    compare_attention(got, ref)


def _fm(a, ld):
    """[n, h] host array -> [h, ld] feature-major bf16 tensor (zero padded)."""
    t = np.zeros((a.shape[1], ld), dtype=np.float32)
    t[:, :a.shape[0]] = a.T
    return dev_bf16(t)


@pytest.mark.parametrize("n_tok,h,batch,ld,with_e", [(4680, 256, 2, 4680, True),
                                                     (333, 320, 3, 344, True),
                                                     (200, 5120, 1, 200, True),
                                                     (1, 64, 1, 8, True),
                                                     (4675, 200, 2, 4680, False),
                                                     (18720, 1536, 2, 18720, True)])
def test_gram_feature_major(n_tok, h, batch, ld, with_e):
    """Statistics of seeded activations from feature-major operands against
    the oracle, two accumulating calls (the second over the first half of the
    tokens), ragged token counts (a partial last 32-token stage), hidden
    sizes off the 256 tile edge, the 14B hidden size, and a 1.3B layer's
    four warmup steps at once."""
    log(f"gram feature-major n={n_tok} h={h} b={batch} ld={ld}")
    x = wl.random_bf16((batch, n_tok, h), 0.5, 81 + h)
    d = wl.random_bf16((batch, n_tok, h), 0.2, 82 + h)
    xt = torch.stack([_fm(x[b], ld) for b in range(batch)])
    dt = torch.stack([_fm(d[b], ld) for b in range(batch)])
    G = torch.full((batch, h, h), float("nan"), dtype=torch.float32, device="cuda")
    C, E = torch.full_like(G, float("nan")), torch.full_like(G, float("nan")) if with_e else None
    ispa.ispa_gram_accumulate_t(xt, dt, n_tok, G, C, E, zero_first=True)
    half = n_tok // 2
    ispa.ispa_gram_accumulate_t(xt, dt, half, G, C, E)
    torch.cuda.synchronize()
    for b in range(batch):
        g, c, e = orc.gram_statistics([x[b], x[b][:half]], [d[b], d[b][:half]])
        Gh = host(G[b])
        assert relfro(Gh, g) <= GRAM_REL
        assert relfro(host(C[b]), c) <= GRAM_REL
        np.testing.assert_array_equal(Gh, Gh.T)
        if with_e:
            Eh = host(E[b])
            assert relfro(Eh, e) <= GRAM_REL
            np.testing.assert_array_equal(Eh, Eh.T)


def test_gram_feature_major_zero_tokens():
    h = 128
    xt = torch.zeros((h, 8), dtype=torch.bfloat16, device="cuda")
    G = torch.full((h, h), float("nan"), dtype=torch.float32, device="cuda")
    C, E = torch.full_like(G, float("nan")), torch.full_like(G, float("nan"))
    ispa.ispa_gram_accumulate_t(xt, xt, 0, G, C, E, zero_first=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(G).item() == 0 and torch.count_nonzero(C).item() == 0
    assert torch.count_nonzero(E).item() == 0


def test_warmup_chain_feature_major_equals_token_major():
    """The tiny warmup through the feature-major path (attention into
    side-by-side step columns, one Gram call) gives the statistics of the
    token-major path (per-step Gram calls) to fp32 summation order, and the
    oracle's to the Gram bound on its stored activations."""
    w = wl.TINY
    h, n = w.hidden, w.n_q
    ld = n * w.n_steps
    xt = torch.empty((h, ld), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty_like(xt)
    o_full = torch.empty((n, h), dtype=torch.bfloat16, device="cuda")
    G0 = torch.empty((h, h), dtype=torch.float32, device="cuda")
    C0, E0 = torch.empty_like(G0), torch.empty_like(G0)
    xs, ds = [], []
    for s in range(w.n_steps):
        st = wl.step_inputs(w, 0, s)
        kv = [dev_bf16(a) if a.shape[0] else None for a in
              (st.k_sink, st.v_sink, st.k_cur, st.v_cur, st.k_hist, st.v_hist)]
        ispa.ispa_attn_decomp_t(dev_bf16(st.q), *kv, w.sm_scale, xt, dt, col=s * n,
                                o_full=o_full)
        _, dev = run_attention(st, w.sm_scale, outputs=("o_local", "d"))
        ispa.ispa_gram_accumulate(dev["o_local"], dev["d"], G0, C0, E0, zero_first=(s == 0))
        xs.append(host(dev["o_local"]))
        ds.append(host(dev["d"]))
    G1 = torch.empty_like(G0)
    C1, E1 = torch.empty_like(G0), torch.empty_like(G0)
    ispa.ispa_gram_accumulate_t(xt, dt, ld, G1, C1, E1, zero_first=True)
    torch.cuda.synchronize()
    g, c, e = orc.gram_statistics(xs, ds)
    for t0, t1, r in ((G0, G1, g), (C0, C1, c), (E0, E1, e)):
        assert relfro(host(t1), host(t0)) <= GRAM_REL
        assert relfro(host(t1), r) <= GRAM_REL

"""GPU parity of ispa_attn_decomp against the fp64 oracle.

Tolerances (bf16 inputs): outputs max-abs <= 1e-2 and relative Frobenius
<= 1e-2, LSE max-abs <= 1e-3. Sizes span several 128-query and 64-key tiles
with ragged tails; the full 1.3B- and 14B-class shapes are checked on sampled
query rows (rows are independent, so those rows are exact).
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import ispa_oracle as orc
from tests.gpu_helpers import compare_attention, log, run_attention

pytestmark = pytest.mark.gpu

ALL = ("o_local", "lse_local", "o_hist", "lse_hist", "o_full", "lse_full", "d")


def oracle_for(st, scale, rows=None):
    q = st.q if rows is None else st.q[rows]
    return orc.decomposable_attention(q, st.k_sink, st.v_sink, st.k_cur, st.v_cur, st.k_hist,
                                      st.v_hist, scale)


def custom(n_q, n_sink, n_cur, n_hist, heads, d, seed=0):
    return dataclasses.replace(wl.TINY, name=f"custom{seed}", config_id=100 + seed,
                               n_heads=heads, head_dim=d, n_q=n_q, n_sink=n_sink, n_cur=n_cur,
                               hist_per_step=(n_hist,), qkv_std=1.0)


@pytest.mark.parametrize("step", [0, 2])
def test_tiny_all_outputs(step):
    w = wl.TINY
    log(f"attn tiny step {step}")
    st = wl.step_inputs(w, 0, step)
    gpu, _ = run_attention(st, w.sm_scale)
    compare_attention(gpu, oracle_for(st, w.sm_scale))


def test_tiny_single_head():
    w = wl.TINY_1HEAD
    log("attn tiny 1 head")
    st = wl.step_inputs(w, 0, 0)
    gpu, _ = run_attention(st, w.sm_scale)
    compare_attention(gpu, oracle_for(st, w.sm_scale))


@pytest.mark.parametrize("d,gain", [(128, 1.0), (128, 4.0), (64, 4.0)])
def test_ragged_tiles(d, gain):
    """200 queries (two q tiles, ragged), segment lengths that end mid-tile."""
    w = custom(200, 37, 101, 301, 3, d, seed=d)
    log(f"attn ragged d={d} gain={gain}")
    st = wl.step_inputs(w, 0, 0, q_gain=gain)
    scale = 1.0 / np.sqrt(d)
    gpu, _ = run_attention(st, scale)
    compare_attention(gpu, oracle_for(st, scale))


def test_empty_history_exact():
    w = custom(130, 64, 70, 0, 2, 128, seed=3)
    log("attn empty history")
    st = wl.step_inputs(w, 0, 0, q_gain=2.0)
    scale = 1.0 / np.sqrt(128)
    gpu, _ = run_attention(st, scale)
    assert np.all(gpu["o_hist"] == 0)
    assert np.all(np.isneginf(gpu["lse_hist"]))
    np.testing.assert_array_equal(gpu["o_full"], gpu["o_local"])
    np.testing.assert_array_equal(gpu["lse_full"], gpu["lse_local"])
    assert np.all(gpu["d"] == 0)
    compare_attention(gpu, oracle_for(st, scale))


@pytest.mark.parametrize("outputs", [("o_full", "lse_full"), ("o_local",), ("o_local", "lse_local"),
                                     ("d",), ("o_hist", "lse_hist")])
def test_output_subsets(outputs):
    w = custom(150, 40, 90, 200, 2, 128, seed=4)
    log(f"attn subset {outputs}")
    st = wl.step_inputs(w, 0, 0, q_gain=3.0)
    scale = 1.0 / np.sqrt(128)
    gpu, _ = run_attention(st, scale, outputs=outputs)
    compare_attention(gpu, oracle_for(st, scale), keys=list(outputs))


@pytest.mark.parametrize("n_sink,n_cur", [(0, 90), (50, 0), (1, 1)])
def test_local_segment_edge_cases(n_sink, n_cur):
    w = custom(70, n_sink, n_cur, 65, 2, 128, seed=5 + n_sink)
    log(f"attn local edge sink={n_sink} cur={n_cur}")
    st = wl.step_inputs(w, 0, 0, q_gain=2.0)
    scale = 1.0 / np.sqrt(128)
    gpu, _ = run_attention(st, scale)
    compare_attention(gpu, oracle_for(st, scale))


def test_bitwise_deterministic():
    w = custom(256, 64, 128, 640, 4, 128, seed=9)
    log("attn determinism")
    st = wl.step_inputs(w, 0, 0)
    a, _ = run_attention(st, 1.0 / np.sqrt(128))
    b, _ = run_attention(st, 1.0 / np.sqrt(128))
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def _sampled_rows(w, step, n_rows=64, seed=0):
    st = wl.step_inputs(w, 0, step)
    log(f"attn full-size {w.name} step {step}: n_q={st.q.shape[0]} hist={st.k_hist.shape[0]}")
    gpu, _ = run_attention(st, w.sm_scale)
    rows = np.sort(np.random.default_rng(seed).choice(st.q.shape[0], n_rows, replace=False))
    ref = oracle_for(st, w.sm_scale, rows)
    sub = {}
    for k, v in gpu.items():
        sub[k] = v[:, rows] if k.startswith("lse") else v[rows]
    return compare_attention(sub, ref)


def test_wan13_layer_sampled_rows():
    _sampled_rows(wl.WAN13_LAYER, 0)


def test_wan14_headline_sampled_rows():
    """14B-class last warmup step: 40 heads, 4680 queries, 1560 + 4680 local
    keys and 56160 history keys."""
    _sampled_rows(wl.WAN14_WARMUP, 3, n_rows=32)


def test_wan14_stream_full_only_sampled_rows():
    """14B-class streaming chunk on an F-layer at the longest history (120 latent
    frames: 1560 + 4680 local and 187200 history keys, 40 heads): only O_full and
    LSE_full are requested, i.e. the single-pass full-only path, at its real size;
    sampled rows against full attention over the concatenated KV."""
    w = wl.WAN14_STREAM
    st = wl.step_inputs(w, 0, 0)
    log(f"attn 14B stream full-only: n_q={st.q.shape[0]} hist={st.k_hist.shape[0]}")
    gpu, _ = run_attention(st, w.sm_scale, outputs=("o_full", "lse_full"))
    rows = np.sort(np.random.default_rng(5).choice(st.q.shape[0], 32, replace=False))
    k_all = np.concatenate([st.k_sink, st.k_cur, st.k_hist])
    v_all = np.concatenate([st.v_sink, st.v_cur, st.v_hist])
    o_ref, lse_ref = orc.multihead_attention(st.q[rows], k_all, v_all, w.sm_scale)
    compare_attention({"o_full": gpu["o_full"][rows], "lse_full": gpu["lse_full"][:, rows]},
                      {"o_full": o_ref, "lse_full": lse_ref})

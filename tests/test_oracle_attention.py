"""Pins of the oracle's attention against what the pages and the mathematics fix.

The ISPA paper (§3.1 item 1, §3.4) defines A_loc as attention over current and
sink tokens, A_full as attention over the whole history, and obtains both from
the log-sum-exp states of one pass. These tests pin the oracle's plain
definitions with hand-derived values, brute force, the exact merge identity and
closed-form special cases.
"""
import math

import numpy as np
import pytest

from oracle import ispa_oracle as orc
from tests.conftest import read_golden
import workloads as wl


def _brute_attention(q, k, v, scale):
    """Explicit loops with math.exp: one head."""
    nq, n = len(q), len(k)
    outs, lses = [], []
    for i in range(nq):
        scores = [scale * sum(q[i][t] * k[j][t] for t in range(len(q[i])))
                  for j in range(n)]
        if n == 0:
            outs.append([0.0] * len(q[i]))
            lses.append(-math.inf)
            continue
        total = sum(math.exp(s) for s in scores)
        outs.append([sum(math.exp(scores[j]) * v[j][c] for j in range(n)) / total
                     for c in range(len(v[0]))])
        lses.append(math.log(total))
    return np.array(outs), np.array(lses)


def test_golden_hand_case():
    g = read_golden("attention_hand.txt")
    q = np.array(g["q"]).reshape(1, 1, 2)
    kv = {n: np.array(g[n]).reshape(1, 1, 2) for n in
          ("k_sink", "v_sink", "k_hist", "v_hist", "k_cur", "v_cur")}
    r = orc.decomposable_attention(q, kv["k_sink"], kv["v_sink"], kv["k_cur"],
                                   kv["v_cur"], kv["k_hist"], kv["v_hist"],
                                   g["scale"][0])
    for key in ("o_local", "o_hist", "o_full", "d"):
        np.testing.assert_allclose(r[key].ravel(), g[key], atol=1e-12)
    for key in ("lse_local", "lse_hist", "lse_full"):
        np.testing.assert_allclose(r[key].ravel(), g[key], atol=1e-12)


def test_brute_force_micro():
    rng = np.random.default_rng(3)
    nh, d = 2, 2
    q = rng.standard_normal((3, nh, d))
    ks, vs = rng.standard_normal((1, nh, d)), rng.standard_normal((1, nh, d))
    kc, vc = rng.standard_normal((2, nh, d)), rng.standard_normal((2, nh, d))
    kh, vh = rng.standard_normal((3, nh, d)), rng.standard_normal((3, nh, d))
    scale = 0.7
    r = orc.decomposable_attention(q, ks, vs, kc, vc, kh, vh, scale)
    for hd in range(nh):
        sets = {
            "local": (np.concatenate([ks, kc])[:, hd], np.concatenate([vs, vc])[:, hd]),
            "hist": (kh[:, hd], vh[:, hd]),
            "full": (np.concatenate([ks, kh, kc])[:, hd],
                     np.concatenate([vs, vh, vc])[:, hd]),
        }
        for name, (k, v) in sets.items():
            o_b, lse_b = _brute_attention(q[:, hd].tolist(), k.tolist(), v.tolist(), scale)
            np.testing.assert_allclose(r["o_" + name][:, hd * d:(hd + 1) * d], o_b,
                                       atol=1e-13)
            np.testing.assert_allclose(r["lse_" + name][hd], lse_b, atol=1e-13)
    np.testing.assert_allclose(r["d"], r["o_full"] - r["o_local"], atol=0)


def test_merge_identity_tiny_workload():
    st = wl.step_inputs(wl.TINY, 0, 0)
    r = orc.decomposable_attention(st.q, st.k_sink, st.v_sink, st.k_cur, st.v_cur,
                                   st.k_hist, st.v_hist, wl.TINY.sm_scale)
    o, lse = orc.merge_partials(r["o_local"], r["lse_local"], r["o_hist"], r["lse_hist"])
    assert np.max(np.abs(o - r["o_full"])) <= 1e-12
    assert np.max(np.abs(lse - r["lse_full"])) <= 1e-12


def test_merge_identity_peaked():
    rng = np.random.default_rng(11)
    nh, d = 3, 16
    q = 4.0 * rng.standard_normal((20, nh, d))
    mk = lambda n: rng.standard_normal((n, nh, d))
    ks, vs, kc, vc, kh, vh = mk(5), mk(5), mk(7), mk(7), mk(33), mk(33)
    r = orc.decomposable_attention(q, ks, vs, kc, vc, kh, vh, 0.5)
    o, lse = orc.merge_partials(r["o_local"], r["lse_local"], r["o_hist"], r["lse_hist"])
    np.testing.assert_allclose(o, r["o_full"], atol=1e-12)
    np.testing.assert_allclose(lse, r["lse_full"], atol=1e-12)


def test_zero_query_gives_mean_and_log_n():
    rng = np.random.default_rng(5)
    k, v = rng.standard_normal((9, 4)), rng.standard_normal((9, 4))
    o, lse = orc.softmax_attention_head(np.zeros((2, 4)), k, v, 1.3)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (2, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, np.log(9.0), atol=1e-14)


def test_single_key():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((4, 3)), rng.standard_normal((1, 3)), rng.standard_normal((1, 3))
    o, lse = orc.softmax_attention_head(q, k, v, 0.9)
    np.testing.assert_allclose(o, np.tile(v, (4, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, 0.9 * (q @ k[0]), atol=1e-14)


def test_uniform_score_shift():
    """Moving every key by t*q adds scale*t*|q|^2 to every score of that
    query: O unchanged, LSE shifted by the same constant."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 5))
    k, v = rng.standard_normal((12, 5)), rng.standard_normal((12, 5))
    scale, t = 0.4, 1.7
    o1, l1 = orc.softmax_attention_head(q, k, v, scale)
    o2, l2 = orc.softmax_attention_head(q, k + t * q, v, scale)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, scale * t * float((q @ q.T)[0, 0]), atol=1e-12)


def test_permutation_and_duplication():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((6, 4))
    k, v = rng.standard_normal((10, 4)), rng.standard_normal((10, 4))
    o1, l1 = orc.softmax_attention_head(q, k, v, 0.8)
    perm = rng.permutation(10)
    o2, l2 = orc.softmax_attention_head(q, k[perm], v[perm], 0.8)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)
    o3, l3 = orc.softmax_attention_head(q, np.concatenate([k, k]), np.concatenate([v, v]), 0.8)
    np.testing.assert_allclose(o3, o1, atol=1e-13)
    np.testing.assert_allclose(l3 - l1, math.log(2.0), atol=1e-13)


def test_empty_history():
    st = wl.step_inputs(wl.TINY, 0, 0, n_hist=0)
    r = orc.decomposable_attention(st.q, st.k_sink, st.v_sink, st.k_cur, st.v_cur,
                                   st.k_hist, st.v_hist, wl.TINY.sm_scale)
    assert np.all(r["o_hist"] == 0) and np.all(np.isneginf(r["lse_hist"]))
    np.testing.assert_array_equal(r["o_full"], r["o_local"])
    np.testing.assert_array_equal(r["lse_full"], r["lse_local"])
    assert np.all(r["d"] == 0)


def test_head_column_layout():
    """Column head*d + j of the flattened output belongs to head `head`:
    permuting heads of Q/K/V permutes the column blocks."""
    rng = np.random.default_rng(9)
    nh, d = 3, 4
    q, k, v = (rng.standard_normal((5, nh, d)), rng.standard_normal((7, nh, d)),
               rng.standard_normal((7, nh, d)))
    o, lse = orc.multihead_attention(q, k, v, 0.5)
    perm = [2, 0, 1]
    o2, lse2 = orc.multihead_attention(q[:, perm], k[:, perm], v[:, perm], 0.5)
    np.testing.assert_allclose(o2.reshape(5, nh, d), o.reshape(5, nh, d)[:, perm], atol=1e-14)
    np.testing.assert_allclose(lse2, lse[perm], atol=1e-14)
    o0, _ = orc.softmax_attention_head(q[:, 1], k[:, 1], v[:, 1], 0.5)
    np.testing.assert_allclose(o[:, d:2 * d], o0, atol=1e-14)

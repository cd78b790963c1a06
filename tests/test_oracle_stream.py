"""Pins of the oracle's streaming functions (ISPA paper §3.1 item 3, §3.3).

With every key zero all scores are equal, so attention is the plain mean of
the values in the attended set. Giving every chunk a constant value that
names it turns the output into a closed form of which chunks are attended,
which pins the history bookkeeping independently of the attention code.
Order invariance (a permutation of the keys leaves softmax attention
unchanged) is what lets a cache keep its chunks in ring-slot order.
"""
import numpy as np
import pytest

import oracle.ispa_oracle as orc

NH, D, NS, NC = 2, 4, 2, 3
SINK_VALUE = 100.0


def marked_inputs(n_chunks, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((5, NH, D))
    k_sink = np.zeros((NS, NH, D))
    v_sink = np.full((NS, NH, D), SINK_VALUE)
    k_chunks = [np.zeros((NC, NH, D)) for _ in range(n_chunks)]
    v_chunks = [np.full((NC, NH, D), float(i + 1)) for i in range(n_chunks)]
    return q, k_sink, v_sink, k_chunks, v_chunks


@pytest.mark.parametrize("c,cap,expected", [
    # full history: sink, chunks 0..c-1, chunk c
    (0, None, (2 * 100 + 3 * 1) / 5),
    (3, None, (2 * 100 + 3 * (1 + 2 + 3 + 4)) / 14),
    # capacity 2 chunks at chunk 5: chunks 3 and 4 plus the current chunk 5
    (5, 2, (2 * 100 + 3 * (4 + 5 + 6)) / 11),
    # capacity 2 at chunk 1: only chunk 0 exists before it
    (1, 2, (2 * 100 + 3 * (1 + 2)) / 8),
    # capacity 0: no history
    (4, 0, (2 * 100 + 3 * 5) / 5),
])
def test_full_layer_window_closed_form(c, cap, expected):
    q, ks, vs, kc, vc = marked_inputs(c + 1)
    wo = np.eye(NH * D)
    o, y = orc.stream_layer_chunk(q, ks, vs, kc, vc, c, wo, 0.5, local_only=False,
                                  capacity_chunks=cap)
    np.testing.assert_allclose(o, expected, rtol=1e-14)
    np.testing.assert_allclose(y, expected, rtol=1e-14)


@pytest.mark.parametrize("c", [0, 2, 6])
def test_local_layer_closed_form(c):
    q, ks, vs, kc, vc = marked_inputs(c + 1)
    wo = 2.0 * np.eye(NH * D)
    o, y = orc.stream_layer_chunk(q, ks, vs, kc, vc, c, wo, 0.5, local_only=True)
    expected = (2 * 100 + 3 * (c + 1)) / 5
    np.testing.assert_allclose(o, expected, rtol=1e-14)
    np.testing.assert_allclose(y, 2.0 * expected, rtol=1e-14)


def test_history_chunks_listing():
    assert orc.history_chunks(0) == []
    assert orc.history_chunks(4) == [0, 1, 2, 3]
    assert orc.history_chunks(4, 10) == [0, 1, 2, 3]
    assert orc.history_chunks(7, 3) == [4, 5, 6]
    assert orc.history_chunks(7, 0) == []


def test_attention_is_key_order_invariant():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((7, NH, D))
    k = rng.standard_normal((23, NH, D))
    v = rng.standard_normal((23, NH, D))
    perm = rng.permutation(23)
    o1, l1 = orc.multihead_attention(q, k, v, 0.7)
    o2, l2 = orc.multihead_attention(q, k[perm], v[perm], 0.7)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_projection_of_stream_output():
    """Y is O projected through the given weight, row by row."""
    rng = np.random.default_rng(5)
    q, ks, vs, kc, vc = marked_inputs(3)
    kc = [rng.standard_normal(x.shape) for x in kc]
    wo = rng.standard_normal((NH * D, NH * D))
    o, y = orc.stream_layer_chunk(q, ks, vs, kc, vc, 2, wo, 0.5, local_only=False)
    for r in range(o.shape[0]):
        for j in range(wo.shape[0]):
            assert abs(y[r, j] - sum(o[r, i] * wo[j, i] for i in range(wo.shape[1]))) < 1e-9

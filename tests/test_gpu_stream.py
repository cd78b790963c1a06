"""GPU parity of the streaming KV cache and the per-layer streaming step
(ISPA paper §3.1 item 3, §3.3) against the oracle's streaming functions.

Chunks are streamed through a cache: each chunk's K/V are written into the
current slot, every layer runs its attention (+ projection) over the cache,
then the cache advances. The oracle rebuilds each layer's attended key set
from the chunk list in time order (the cache keeps them in ring-slot order,
which attention does not see). Tolerances are those of the attention tests
(outputs max-abs 1e-2 scaled by max(1, max|O|), relative Frobenius 1e-2, LSE
max-abs 1e-3); the projection output Y = O W^T is a bf16 rounding of a
product of the bf16 O, so it is held to the same relative Frobenius bound.
"""
import numpy as np
import pytest
import torch

import kv_cache_absorption_attn_amd as ispa
import workloads as wl
from oracle import ispa_oracle as orc
from tests.gpu_helpers import O_RELFRO, compare_attention, dev_bf16, host, log

pytestmark = pytest.mark.gpu


class Stream:
    """Seeded chunks of one synthetic stream: per layer a sink, per (layer,
    chunk) the chunk's K/V and Q, per layer a projection W."""

    def __init__(self, n_layers, nh, d, n_sink, n_cur, n_q, seed):
        self.n_layers, self.nh, self.d = n_layers, nh, d
        self.n_sink, self.n_cur, self.n_q, self.seed = n_sink, n_cur, n_q, seed
        self.scale = 1.0 / np.sqrt(d)
        self.ks = [self._t((n_sink, nh, d), 1, l, 0) for l in range(n_layers)]
        self.vs = [self._t((n_sink, nh, d), 2, l, 0) for l in range(n_layers)]
        self.kc, self.vc, self.q = [[] for _ in range(n_layers)], [[] for _ in range(n_layers)], \
            [[] for _ in range(n_layers)]
        h = nh * d
        self.wo = [wl.random_bf16((h, h), 1.0 / np.sqrt(h), seed * 1000 + 900 + l)
                   for l in range(n_layers)]

    def _t(self, shape, kind, layer, chunk):
        return wl.random_bf16(shape, 1.0, self.seed * 1000003 + kind * 10007 + layer * 101 + chunk)

    def chunk(self, c):
        for l in range(self.n_layers):
            if len(self.kc[l]) == c:
                self.kc[l].append(self._t((self.n_cur, self.nh, self.d), 3, l, c))
                self.vc[l].append(self._t((self.n_cur, self.nh, self.d), 4, l, c))
                self.q[l].append(self._t((self.n_q, self.nh, self.d), 5, l, c))

    def oracle(self, l, c, local_only, cap, wo=None):
        return orc.stream_layer_chunk(self.q[l][c], self.ks[l], self.vs[l], self.kc[l],
                                      self.vc[l], c, self.wo[l] if wo is None else wo,
                                      self.scale, local_only=local_only, capacity_chunks=cap)

    def oracle_split(self, l, c, cap):
        hist = orc.history_chunks(c, cap)
        empty = np.zeros((0, self.nh, self.d))
        kh = np.concatenate([self.kc[l][i] for i in hist], axis=0) if hist else empty
        vh = np.concatenate([self.vc[l][i] for i in hist], axis=0) if hist else empty
        return orc.decomposable_attention(self.q[l][c], self.ks[l], self.vs[l], self.kc[l][c],
                                          self.vc[l][c], kh, vh, self.scale)


def relfro(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def run_layer(cache, s, l, c, wo_dev):
    h = s.nh * s.d
    o = torch.full((s.n_q, h), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(o, float("nan"))
    cache.layer_forward(l, dev_bf16(s.q[l][c]), s.scale, wo_dev, o, y)
    torch.cuda.synchronize()
    return host(o), host(y)


def check_forward(o, y, o_ref, y_ref, what):
    compare_attention({"o": o}, {"o": o_ref})
    err = relfro(y, y_ref)
    assert err <= O_RELFRO, f"{what}: y rel fro {err}"


def run_split(cache, s, l, c):
    h = s.nh * s.d
    out = {}
    kw = {}
    for name in ("o_local", "lse_local", "o_hist", "lse_hist", "o_full", "lse_full", "d"):
        if name.startswith("lse"):
            t = torch.full((s.nh, s.n_q), float("nan"), dtype=torch.float32, device="cuda")
        else:
            t = torch.full((s.n_q, h), float("nan"), dtype=torch.bfloat16, device="cuda")
        out[name] = t
        kw["d_out" if name == "d" else name] = t
    cache.attn(l, dev_bf16(s.q[l][c]), s.scale, **kw)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


@pytest.mark.parametrize("d", [128, 64])
def test_ring_of_full_layers(d):
    """Two F-layers, a history capacity of 3 chunks and 7 chunks: the ring
    fills, wraps, and keeps the 3 most recent chunks. Segment lengths end
    mid-tile (sink 40, chunk 100 keys; 150 queries). The split outputs match
    the oracle at every ring state, also when the wrapped history is in two
    pieces (the view's three segments then cover it only for full outputs)."""
    L, nh, ns, nc, nq, cap_chunks = 2, 2, 40, 100, 150, 3
    s = Stream(L, nh, d, ns, nc, nq, seed=d)
    cache = ispa.KVCache(L, nh, d, ns, nc, cap_chunks * nc)
    try:
        wo = [dev_bf16(w) for w in s.wo]
        for l in range(L):
            cache.write(l, dev_bf16(s.ks[l]), dev_bf16(s.vs[l]), sink=True)
        resident = []
        for c in range(7):
            log(f"stream ring d={d} chunk {c}")
            s.chunk(c)
            for l in range(L):
                cache.write(l, dev_bf16(s.kc[l][c]), dev_bf16(s.vc[l][c]))
            for l in range(L):
                v = cache.view(l)
                assert v.n_hist == min(c, cap_chunks) * nc and v.local_only == 0
                assert v.split_ok == (1 if c <= cap_chunks or c % (cap_chunks + 1) == 0 else 0)
                o, y = run_layer(cache, s, l, c, wo[l])
                o_ref, y_ref = s.oracle(l, c, False, cap_chunks)
                check_forward(o, y, o_ref, y_ref, f"layer {l} chunk {c}")
                compare_attention(run_split(cache, s, l, c), s.oracle_split(l, c, cap_chunks))
            resident.append(cache.resident_bytes())
            cache.advance()
        row = nh * d * 2
        # memory grows with the slots in use and stops once the ring is full
        assert all(b >= a for a, b in zip(resident, resident[1:]))
        assert resident[-1] == resident[cap_chunks]
        assert resident[-1] >= 2 * L * (ns + (cap_chunks + 1) * nc) * row
    finally:
        cache.close()


def test_eviction_makes_local_layers():
    """Three layers stream 2 chunks as F-layers; layer 1 then turns into an
    L-layer (history evicted, projected through a new weight) and the stream
    goes on for 3 chunks: layer 1 attends sink + current only, the others
    their whole history. The evicted layer's memory is released (a chunk is
    1.25 MiB of K and as much of V, so by then its history spans pieces
    beyond the first)."""
    L, nh, d, ns, nc, nq = 3, 8, 128, 64, 640, 130
    s = Stream(L, nh, d, ns, nc, nq, seed=7)
    cache = ispa.KVCache(L, nh, d, ns, nc, 16 * nc)
    try:
        wo = [dev_bf16(w) for w in s.wo]
        w_new = wl.random_bf16((nh * d, nh * d), 1.0 / np.sqrt(nh * d), 4242)
        for l in range(L):
            cache.write(l, dev_bf16(s.ks[l]), dev_bf16(s.vs[l]), sink=True)
        before = None
        for c in range(5):
            log(f"stream evict chunk {c}")
            if c == 2:
                before = cache.resident_bytes()
                cache.evict_history(1)
                cache.evict_history(1)          # idempotent
                wo[1] = dev_bf16(w_new)
                after = cache.resident_bytes()
                log(f"  resident bytes {before} -> {after}")
                assert after < before
            s.chunk(c)
            for l in range(L):
                cache.write(l, dev_bf16(s.kc[l][c]), dev_bf16(s.vc[l][c]))
            for l in range(L):
                local = l == 1 and c >= 2
                v = cache.view(l)
                assert v.local_only == int(local)
                assert v.n_hist == (0 if local else c * nc)
                o, y = run_layer(cache, s, l, c, wo[l])
                o_ref, y_ref = s.oracle(l, c, local, None, wo=w_new if local else None)
                check_forward(o, y, o_ref, y_ref, f"layer {l} chunk {c}")
            cache.advance()
        # the two F-layers kept growing; the L-layer holds its sink and one slot
        v1 = cache.view(1)
        assert v1.n_hist == 0 and v1.seg_n[2] == 0
    finally:
        cache.close()


def test_wan_shaped_chunks_with_wrap():
    """Frame-sized segments (sink 1560 keys, chunk 4680 keys = 3 frames) with
    a 2-chunk history ring over 5 chunks, 8 heads, 256 queries: the attention
    over the cache at the real segment lengths, including the wrapped ring's
    out-of-order slots, for the full and the split outputs."""
    L, nh, d, ns, nc, nq, cap = 1, 8, 128, 1560, 4680, 256, 2
    s = Stream(L, nh, d, ns, nc, nq, seed=11)
    cache = ispa.KVCache(L, nh, d, ns, nc, cap * nc)
    try:
        wo = dev_bf16(s.wo[0])
        cache.write(0, dev_bf16(s.ks[0]), dev_bf16(s.vs[0]), sink=True)
        for c in range(5):
            log(f"stream wan-shaped chunk {c}")
            s.chunk(c)
            cache.write(0, dev_bf16(s.kc[0][c]), dev_bf16(s.vc[0][c]))
            o, y = run_layer(cache, s, 0, c, wo)
            o_ref, y_ref = s.oracle(0, c, False, cap)
            check_forward(o, y, o_ref, y_ref, f"chunk {c}")
            # split outputs too (chunk 4: the history is slot 2, then slot 0)
            compare_attention(run_split(cache, s, 0, c), s.oracle_split(0, c, cap))
            cache.advance()
    finally:
        cache.close()

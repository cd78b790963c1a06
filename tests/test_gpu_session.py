"""GPU parity of the drift score and of the streaming session (warmup ->
absorption -> streaming, event-triggered recalibration; ISPA paper §3.1
items 1-3, §3.3 with its last paragraph) against the oracle.

The drift stage runs on the oracle's statistics and seeded probe tokens:
reference and score within 1e-4 / 1e-3 relative (fp32 factor and inverse
of G + lambda I on well-conditioned statistics).

The session test replays the whole life cycle with the oracle beside it:
the oracle keeps every chunk's K/V, rebuilds each layer's attended set,
accumulates its statistics over its own bf16-stored activations, solves,
selects and scores drift itself, and decides its own events. The GPU's
outputs, selections, events and drift scores must agree at the all-GPU
chain bounds (the GPU statistics come from the GPU's own attention output):
attention outputs at the attention bounds, Y relative Frobenius <= 1e-2,
selection and events identical, drift scores within 5e-2 relative.
"""
import numpy as np
import pytest
import torch

import kv_cache_absorption_attn_amd as ispa
import workloads as wl
from oracle import ispa_oracle as orc
from tests.gpu_helpers import O_RELFRO, compare_attention, dev_bf16, host, log

pytestmark = pytest.mark.gpu


def relfro(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("h,n_warm", [(256, 1200), (1536, 5000)])
def test_drift_prepare_and_score(h, n_warm):
    """Warmup statistics of seeded tokens (several 128-column factor blocks
    at h = 1536); probes from the warmup distribution, scaled by 3, and from
    a distribution with a new dominant direction."""
    lam = 1e-2
    log(f"drift h={h} n_warm={n_warm}")
    rng_basis = wl.random_bf16((h, h), 1.0 / np.sqrt(h), 71)
    warm = wl.random_bf16((n_warm, h), 0.3, 72) @ rng_basis
    g = orc.gram_statistics([warm], [np.zeros_like(warm)])[0]
    g = g.astype(np.float32).astype(np.float64)
    G = torch.from_numpy(g[None].astype(np.float32)).cuda()
    linv = torch.full((1, h, h), float("nan"), dtype=torch.float32, device="cuda")
    ref = torch.empty(1, dtype=torch.float64, device="cuda")
    info = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    n_tok, stride = 700, 3
    ws = torch.empty(ispa.ispa_drift_workspace_bytes(1, h, (n_tok + stride - 1) // stride),
                     dtype=torch.uint8, device="cuda")
    ispa.ispa_drift_prepare(G, lam, n_warm, linv, ref, info, ws)
    torch.cuda.synchronize()
    assert int(info[0]) == 0
    ref_o = orc.drift_reference(g, lam, n_warm)
    log(f"  ref {float(ref[0]):.6e} oracle {ref_o:.6e}")
    assert abs(float(ref[0]) - ref_o) <= 1e-4 * ref_o
    li = host(linv[0])
    assert np.count_nonzero(np.triu(li, 1)) == 0
    # the same from the factor a ridge solve on G leaves in its workspace
    rws = torch.empty(ispa.ispa_ridge_workspace_bytes(1, h), dtype=torch.uint8, device="cuda")
    wo = dev_bf16(wl.random_bf16((1, h, h), 0.02, 76))
    dw = torch.empty((1, h, h), dtype=torch.float32, device="cuda")
    rinfo = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    ispa.ispa_ridge_solve(G, torch.zeros_like(G), wo, lam, dw, rinfo, rws)
    linv_f = torch.full_like(linv, float("nan"))
    ref_f = torch.empty_like(ref)
    ispa.ispa_drift_prepare_factored(1, h, lam, n_warm, linv_f, ref_f, rws)
    torch.cuda.synchronize()
    assert int(rinfo[0]) == 0
    assert torch.equal(linv_f, linv) and torch.equal(ref_f, ref)
    same = wl.random_bf16((n_tok, h), 0.3, 73) @ rng_basis
    spike = wl.random_bf16((n_tok, 1), 2.0, 74) * wl.random_bf16((1, h), 1.0, 75)
    probes = {"same": same, "scaled": 3.0 * same, "new direction": same + spike}
    scores = {}
    for name, p in probes.items():
        p = orc.bf16_round(p)
        sc = torch.empty(1, dtype=torch.float64, device="cuda")
        ispa.ispa_drift_score(linv, ref, dev_bf16(p), stride, sc, ws)
        torch.cuda.synchronize()
        exp = orc.drift_score(p[::stride], g, lam, n_warm)
        scores[name] = float(sc[0])
        log(f"  {name}: score {float(sc[0]):.5f} oracle {exp:.5f}")
        assert abs(float(sc[0]) - exp) <= 1e-3 * exp
    assert scores["scaled"] > 8.0 * scores["same"]
    assert scores["new direction"] > 5.0 * scores["same"]


class OracleSession:
    """The oracle's replay of the session: the same life cycle, decided on
    the oracle's own numbers."""

    def __init__(self, wo, n_sink, scale, lam, k_select, t_warm, tau, quant=False, cap=None):
        self.quant = quant                   # W8A8 projections, E4M3 attention when streaming
        self.cap = cap                       # history capacity in chunks (None: unbounded)
        self.mu = {}
        self.wo = [np.asarray(w, dtype=np.float64) for w in wo]
        self.L = len(wo)
        self.scale, self.lam, self.k, self.t_warm, self.tau = scale, lam, k_select, t_warm, tau
        self.phase, self.warm = "warmup", 0
        self.first = [0] * self.L            # first chunk of each layer's history
        self.local = [False] * self.L
        self.w = list(self.wo)
        self.xs = [[] for _ in range(self.L)]
        self.ds = [[] for _ in range(self.L)]
        self.stats = None
        self.drift = [0.0] * self.L

    def proj(self, o, l):
        if self.quant:
            # the projection quantizes the bf16 activations the attention
            # stores (its input is bf16): E4M3 codes amplify a bf16-level
            # difference of their input into whole code steps
            wq, ws = orc.quantize_rows(self.w[l])
            return orc.project_w8a8(orc.bf16_round(o), wq, ws)
        return orc.project(o, self.w[l])

    def layer(self, l, c, q, ks, vs, kc, vc):
        empty = np.zeros((0,) + kc[c].shape[1:])
        streaming_fp8 = self.quant and self.phase == "stream"
        if streaming_fp8 and l not in self.mu:
            self.mu[l] = orc.bf16_round(orc.key_mean(ks))   # the sink's mean key, fixed
        if self.local[l]:
            if streaming_fp8:
                o = orc.decomposable_attention_fp8(q, ks, vs, kc[c], vc[c], empty, empty,
                                                   self.scale, self.mu[l])["o_local"]
            else:
                k = np.concatenate([ks, kc[c]])
                v = np.concatenate([vs, vc[c]])
                o, _ = orc.multihead_attention(q, k, v, self.scale)
            x = orc.bf16_round(o)
            g, n_warm = self.stats[l]
            self.drift[l] = orc.drift_score(x, g, self.lam, n_warm)
            return o, self.proj(o, l)
        hist = [i for i in range(self.first[l], c) if self.cap is None or i >= c - self.cap]
        kh = np.concatenate([kc[i] for i in hist]) if hist else empty
        vh = np.concatenate([vc[i] for i in hist]) if hist else empty
        if streaming_fp8:
            r = orc.decomposable_attention_fp8(q, ks, vs, kc[c], vc[c], kh, vh, self.scale,
                                               self.mu[l])
        else:
            r = orc.decomposable_attention(q, ks, vs, kc[c], vc[c], kh, vh, self.scale)
        if self.phase == "warmup":
            x, d = orc.stored_activations(r["o_local"], r["o_full"])
            self.xs[l].append(x)
            self.ds[l].append(d)
        return r["o_full"], self.proj(r["o_full"], l)

    def end_chunk(self, c):
        if self.phase == "warmup":
            self.warm += 1
            if self.warm < self.t_warm:
                return 0
            eps, dws, self.stats = [], [], []
            for l in range(self.L):
                g, cc, e = orc.gram_statistics(self.xs[l], self.ds[l])
                dw = orc.ridge_delta_w(g, cc, self.wo[l], self.lam)
                eps.append(orc.layer_error_from_stats(g, cc, e, self.wo[l], dw, self.lam)[1])
                dws.append(dw)
                self.stats.append((g, sum(x.shape[0] for x in self.xs[l])))
            sel = orc.select_layers(np.array(eps), self.k)
            self.eps = eps
            for l in range(self.L):
                self.local[l] = bool(sel[l])
                self.w[l] = orc.apply_delta(self.wo[l], dws[l]) if sel[l] else self.wo[l]
                self.xs[l], self.ds[l] = [], []
            self.phase = "stream"
            return 1
        if any(self.local[l] and self.drift[l] > self.tau for l in range(self.L)):
            for l in range(self.L):
                if self.local[l]:
                    self.local[l] = False
                    self.first[l] = c + 1
                self.w[l] = self.wo[l]
            self.phase, self.warm = "warmup", 0
            self.drift = [0.0] * self.L
            return 2
        return 0


def test_session_life_cycle_with_recalibration():
    """Three layers (query temperatures 1, 0.5, 2 separate their errors; the
    absorbed layer is layer 1, whose per-layer entries sit off 16-byte
    boundaries),
    2 warmup chunks, K = 1, drift threshold 4. The stream is temporally
    coherent: a chunk's K, V and Q are its scene's tensors plus small
    per-chunk noise. Chunks 0-1 warm up, 2-3 stream in the same scene,
    chunk 4 starts a new scene, which drives the L-layer's drift score past
    the threshold; chunks 5-6 warm up again and chunk 7 streams under the
    new calibration."""
    life_cycle(nh=2, d=64, flags=0, y_tol=O_RELFRO)


def test_session_quantized_life_cycle():
    """The same life cycle with W8A8 projections (E4M3 weights requantized
    at creation, absorption and recalibration) and E4M3 attention in the
    streaming phase (one head of 128), against the oracle's replay with its
    own quantized attention and W8A8 projection: the same selections, events
    and drift bounds. Y is held to 3e-2 relative Frobenius: the E4M3 codes
    of the activations turn the attention's own bf16-level differences into
    whole code steps (2^-3 relative) wherever a value sits near a rounding
    boundary, and a row's scale moves with its largest element; on this
    case that alone moves Y by up to ~2 % between two correct chains."""
    life_cycle(nh=1, d=128, flags=ispa.SESSION_W8A8 | ispa.SESSION_FP8_ATTN, y_tol=3e-2)


def test_session_recalibrates_after_ring_wrap():
    """The life cycle with a history capacity of 3 chunks: the F-layers'
    rings have wrapped by the time the drift event re-enters the warmup, so
    the warmup's split attention runs over a history in two pieces (chunks
    5 and 6: slots after the current one, then before it), against the
    oracle's replay over the 3 most recent chunks."""
    life_cycle(nh=2, d=64, flags=0, y_tol=O_RELFRO, cap_chunks=3)


def life_cycle(nh, d, flags, y_tol, cap_chunks=16):
    L, ns, nc = 3, 64, 256
    h = nh * d
    scale, lam, K, t_warm, tau = 1.0 / np.sqrt(d), 1e-2, 1, 2, 4.0
    temps = [1.0, 0.5, 2.0]
    n_chunks, shift_at = 8, 4
    rnd = lambda shape, seed, std=1.0: wl.random_bf16(shape, std, 5000 + seed)
    ks = [rnd((ns, nh, d), 10 * l + 1) for l in range(L)]
    vs = [rnd((ns, nh, d), 10 * l + 2) for l in range(L)]
    wo = [rnd((h, h), 10 * l + 3, 1.0 / np.sqrt(h)) for l in range(L)]
    # per scene and layer: base K, V, Q of a chunk
    scene = [[{t: rnd((nc, nh, d), 300 * sc + 10 * l + t) for t in (4, 5, 6)}
              for l in range(L)] for sc in range(2)]
    kc = [[] for _ in range(L)]
    vc = [[] for _ in range(L)]
    sess = ispa.Session(dev_bf16(np.stack(wo)), n_heads=nh, head_dim=d, n_sink=ns, n_cur=nc,
                        hist_capacity=cap_chunks * nc, k_select=K, t_warm=t_warm, sm_scale=scale,
                        lam=lam, drift_threshold=tau, drift_stride=1, flags=flags)
    ref = OracleSession(wo, ns, scale, lam, K, t_warm, tau, quant=flags != 0,
                        cap=cap_chunks if cap_chunks < n_chunks else None)
    try:
        for l in range(L):
            sess.cache.write(l, dev_bf16(ks[l]), dev_bf16(vs[l]), sink=True)
        events = []
        worst = 0.0
        y = torch.empty((nc, h), dtype=torch.bfloat16, device="cuda")
        for c in range(n_chunks):
            sc = scene[1 if c >= shift_at else 0]
            noise = lambda l, t: rnd((nc, nh, d), 1000 + 100 * c + 10 * l + t, 0.1)
            for l in range(L):
                kc[l].append(orc.bf16_round(sc[l][4] + noise(l, 4)))
                vc[l].append(orc.bf16_round(sc[l][5] + noise(l, 5)))
                sess.cache.write(l, dev_bf16(kc[l][c]), dev_bf16(vc[l][c]))
            for l in range(L):
                q = orc.bf16_round(temps[l] * (sc[l][6] + 3.0 * noise(l, 6)))
                sess.layer(l, dev_bf16(q), y)
                torch.cuda.synchronize()
                o_ref, y_ref = ref.layer(l, c, q, ks[l], vs[l], kc[l], vc[l])
                err = relfro(host(y), y_ref)
                worst = max(worst, err)
                assert err <= y_tol, f"chunk {c} layer {l}: y rel fro {err}"
            st, _, _, drift_run = sess.state()
            drift_ref = list(ref.drift)
            ev = sess.end_chunk()
            ev_ref = ref.end_chunk(c)
            st, loc, eps, _ = sess.state()
            log(f"chunk {c}: event {ev} (oracle {ev_ref}), local {loc}, drift "
                f"{[round(x, 3) for x in drift_run]} (oracle {[round(x, 3) for x in drift_ref]})")
            assert ev == ev_ref
            events.append(ev)
            if ev == 1:
                assert loc == [int(x) for x in ref.local]
                for l in range(L):
                    assert abs(eps[l] - ref.eps[l]) <= 5e-2 * ref.eps[l] + 1e-6
        log(f"largest y rel fro over the chunks and layers: {worst:.4f}")
        assert events == [0, 1, 0, 0, 2, 0, 1, 0]
        st, loc, _, _ = sess.state()
        assert st.n_calibrations == 2 and st.chunk == n_chunks and st.phase == 1
    finally:
        sess.close()

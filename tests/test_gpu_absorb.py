"""GPU parity of the warmup statistics, ridge solve, layer score, selection,
weight update and projection against the fp64 oracle.

Every input of a GPU stage comes from the seeded generator or from the
oracle, never from another GPU stage: the Gram runs on the oracle's
bf16-stored X and D (oracle.stored_activations), the solve and the score on
the oracle's statistics rounded to fp32. Stage tolerances: Gram relative
Frobenius <= 1e-5 (fp32 accumulation of exact bf16 products), dW relative
Frobenius <= 1e-3, eps relative <= 1e-4, selection identical, weight update
bit-exact.

The all-GPU chain (attention -> Gram -> solve -> score) is compared with the
oracle's chain separately. There the GPU's X and D differ from the oracle's
stored ones by the attention error and by bf16 rounding flips, errors of the
size of the bf16 storage itself; on the tiny case that storage moves dW by
under 2e-3 and the statistics by a few 1e-4 (pinned in the oracle tests), so
the chain bounds are 5x those: statistics 1e-2, dW 1e-2, eps 5e-2 relative.

The error eps_rel is a difference of traces (tr(W^T E W) minus the explained
part) built from fp32 GEMMs, so when the fit is very good (eps_rel << 1) the
fp32 rounding of those traces dominates: the bound is 1e-4 relative plus an
absolute floor of 4 * 2^-24 * sqrt(h) in units of ||Z W||^2.
"""
import numpy as np
import pytest
import torch

import kv_cache_absorption_attn_amd as ispa
import workloads as wl
from oracle import ispa_oracle as orc
from tests.gpu_helpers import dev_bf16, host, log, oracle_chain, run_attention

pytestmark = pytest.mark.gpu

GRAM_REL = 1e-5
DW_REL = 1e-3
EPS_REL = 1e-4


def eps_tol(ref, h):
    return EPS_REL * abs(ref) + 4.0 * 2.0 ** -24 * np.sqrt(h)


def relfro(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))


CHAIN_STATS_REL = 1e-2
CHAIN_DW_REL = 1e-2
CHAIN_EPS_REL = 5e-2


def gpu_chain_stats(w, layer=0):
    """The all-GPU warmup of one layer: GPU attention for every step, its X
    and D straight into the GPU Gram. Returns the GPU G, C, E tensors."""
    h = w.hidden
    G = torch.empty((1, h, h), dtype=torch.float32, device="cuda")
    C = torch.empty_like(G)
    E = torch.empty_like(G)
    for s in range(w.n_steps):
        st = wl.step_inputs(w, layer, s)
        _, dev = run_attention(st, w.sm_scale, outputs=("o_local", "d"))
        ispa.ispa_gram_accumulate(dev["o_local"], dev["d"], G[0], C[0], E[0], zero_first=(s == 0))
    torch.cuda.synchronize()
    return G, C, E


def gram_of(xs, ds, h):
    """GPU Gram accumulated over the given per-step bf16 X and D (host)."""
    G = torch.full((1, h, h), float("nan"), dtype=torch.float32, device="cuda")
    C, E = torch.full_like(G, float("nan")), torch.full_like(G, float("nan"))
    for s, (x, d) in enumerate(zip(xs, ds)):
        ispa.ispa_gram_accumulate(dev_bf16(x), dev_bf16(d), G[0], C[0], E[0], zero_first=(s == 0))
    torch.cuda.synchronize()
    return G, C, E


def f32_dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() for a in arrays]


def ridge_gpu(G, C, Wo, lam):
    L, h, _ = G.shape
    dW = torch.empty((L, h, h), dtype=torch.float32, device="cuda")
    info = torch.full((L,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(ispa.ispa_ridge_workspace_bytes(L, h), dtype=torch.uint8, device="cuda")
    ispa.ispa_ridge_solve(G, C, Wo, lam, dW, info, ws)
    torch.cuda.synchronize()
    return dW, info, ws


def score_gpu(G, C, E, Wo, dW, lam, info, K, ws):
    L = G.shape[0]
    ea = torch.empty(L, dtype=torch.float64, device="cuda")
    er = torch.empty(L, dtype=torch.float64, device="cuda")
    sel = torch.full((L,), -1, dtype=torch.int32, device="cuda")
    ispa.ispa_layer_score(G, C, E, Wo, dW, lam, info, K, ws, ea, er, sel)
    torch.cuda.synchronize()
    return ea.cpu().numpy(), er.cpu().numpy(), sel.cpu().numpy()


# ------------------------------------------------------------------ Gram

def test_gram_tiny_warmup():
    """The Gram over the three warmup steps of the oracle's stored X, D."""
    log("gram tiny warmup")
    ref = oracle_chain(wl.TINY)
    G, C, E = gram_of(ref["xs"], ref["ds"], wl.TINY.hidden)
    g, c, e = ref["g"], ref["c"], ref["e"]
    Gh, Ch, Eh = host(G[0]), host(C[0]), host(E[0])
    assert relfro(Gh, g) <= GRAM_REL and relfro(Ch, c) <= GRAM_REL and relfro(Eh, e) <= GRAM_REL
    np.testing.assert_array_equal(Gh, Gh.T)
    np.testing.assert_array_equal(Eh, Eh.T)


@pytest.mark.parametrize("n_tok,h,batch", [(100, 192, 2), (1, 64, 1), (333, 256, 3), (200, 512, 2)])
def test_gram_ragged(n_tok, h, batch):
    log(f"gram ragged n={n_tok} h={h} b={batch}")
    x = wl.random_bf16((batch, n_tok, h), 0.5, 11 + h)
    d = wl.random_bf16((batch, n_tok, h), 0.2, 12 + h)
    xg, dg = dev_bf16(x), dev_bf16(d)
    G = torch.full((batch, h, h), float("nan"), dtype=torch.float32, device="cuda")
    C, E = torch.full_like(G, float("nan")), torch.full_like(G, float("nan"))
    ispa.ispa_gram_accumulate(xg, dg, G, C, E, zero_first=True)
    ispa.ispa_gram_accumulate(xg, dg, G, C, E)           # second step: accumulate
    torch.cuda.synchronize()
    for b in range(batch):
        g, c, e = orc.gram_statistics([x[b], x[b]], [d[b], d[b]])
        assert relfro(host(G[b]), g) <= GRAM_REL
        assert relfro(host(C[b]), c) <= GRAM_REL
        assert relfro(host(E[b]), e) <= GRAM_REL
        np.testing.assert_array_equal(host(G[b]), host(G[b]).T)


def test_gram_without_e_and_deterministic():
    x = wl.random_bf16((300, 128), 0.5, 21)
    d = wl.random_bf16((300, 128), 0.2, 22)
    xg, dg = dev_bf16(x), dev_bf16(d)
    outs = []
    for _ in range(2):
        G = torch.empty((128, 128), dtype=torch.float32, device="cuda")
        C = torch.empty_like(G)
        ispa.ispa_gram_accumulate(xg, dg, G, C, None, zero_first=True)
        torch.cuda.synchronize()
        outs.append((host(G), host(C)))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    g, c, _ = orc.gram_statistics([x], [d])
    assert relfro(outs[0][0], g) <= GRAM_REL and relfro(outs[0][1], c) <= GRAM_REL


@pytest.mark.parametrize("n_tok,h,batch,with_e", [(200, 5120, 1, True), (130, 1024, 16, False)])
def test_gram_hidden_5120_and_batched(n_tok, h, batch, with_e):
    """Production shapes: the 14B hidden size (h = 5120, 3240 output tiles)
    with a ragged last stage (200 = 3 x 64 + 8 tokens), and a batched case
    without E; two accumulating calls."""
    log(f"gram n={n_tok} h={h} b={batch} E={with_e}")
    x = wl.random_bf16((batch, n_tok, h), 0.5, 41 + h)
    d = wl.random_bf16((batch, n_tok, h), 0.2, 42 + h)
    xg, dg = dev_bf16(x), dev_bf16(d)
    G = torch.full((batch, h, h), float("nan"), dtype=torch.float32, device="cuda")
    C = torch.full_like(G, float("nan"))
    E = torch.full_like(G, float("nan")) if with_e else None
    ispa.ispa_gram_accumulate(xg, dg, G, C, E, zero_first=True)
    ispa.ispa_gram_accumulate(xg, dg, G, C, E)
    torch.cuda.synchronize()
    for b in range(batch):
        g, c, e = orc.gram_statistics([x[b], x[b]], [d[b], d[b]])
        Gh = host(G[b])
        assert relfro(Gh, g) <= GRAM_REL
        assert relfro(host(C[b]), c) <= GRAM_REL
        if with_e:
            assert relfro(host(E[b]), e) <= GRAM_REL
            np.testing.assert_array_equal(host(E[b]), host(E[b]).T)
        np.testing.assert_array_equal(Gh, Gh.T)


def test_gram_solve_score_hidden_5120():
    """The 14B hidden size over 2 layers with 7000 tokens each (full-rank
    statistics, cond(G + lambda I) ~ 2e2): the GPU Gram of the seeded
    activations, then the solve and the layer score (W_o^T W_o by the G-only
    Gram launch batched over layers) on the oracle's statistics; dW, the
    errors and the selection against the oracle's."""
    L, h, n, lam = 2, 5120, 7000, 1e-2
    log("gram + solve + score h=5120")
    gs, cs, es, wos, refs = [], [], [], [], []
    for l in range(L):
        x = wl.random_bf16((n, h), 0.3, 51 + 10 * l)
        d = wl.random_bf16((n, h), 0.05 * (l + 1), 52 + 10 * l)
        g, c, e = orc.gram_statistics([x], [d])
        if l == 0:
            G0, C0, E0 = gram_of([x], [d], h)
            for name, t, r in (("G", G0, g), ("C", C0, c), ("E", E0, e)):
                assert relfro(host(t[0]), r) <= GRAM_REL, name
            del G0, C0, E0
        g, c, e = (a.astype(np.float32).astype(np.float64) for a in (g, c, e))
        wo = wl.random_bf16((h, h), 1.0 / np.sqrt(h), 53 + 10 * l)
        dw = orc.ridge_delta_w(g, c, wo, lam)
        refs.append((dw, orc.layer_error_from_stats(g, c, e, wo, dw, lam)))
        gs.append(g); cs.append(c); es.append(e); wos.append(wo)
    G, C, E = f32_dev(np.stack(gs), np.stack(cs), np.stack(es))
    Wo = dev_bf16(np.stack(wos))
    dW, info, ws = ridge_gpu(G, C, Wo, lam)
    assert np.all(info.cpu().numpy() == 0)
    ea, er, sel = score_gpu(G, C, E, Wo, dW, lam, info, 1, ws)
    for l in range(L):
        dw_ref, (ea_ref, er_ref) = refs[l]
        err = relfro(host(dW[l]), dw_ref)
        log(f"  layer {l}: dW rel fro {err:.2e}, eps_rel {er[l]:.6e} oracle {er_ref:.6e}")
        assert err <= DW_REL
        assert abs(er[l] - er_ref) <= eps_tol(er_ref, h), (er[l], er_ref)
    np.testing.assert_array_equal(sel, orc.select_layers(np.array([r[1][1] for r in refs]), 1))


@pytest.mark.parametrize("h,n", [(1024, 200), (5120, 200)])
def test_rank_deficient_statistics(h, n):
    """Fewer tokens than features (n = 200 < h): G + lambda I has eigenvalues
    lambda outside the span of the tokens (cond ~2e4 at h = 1024), so an
    fp32 Cholesky solve alone is off by ~3e-3 and a C W formed before the
    solve by more. The solve refines once with an fp64-accumulated residual;
    dW itself, the fitted output X dW and the error against the oracle's
    fp64 solve of the same fp32 statistics."""
    lam = 1e-2
    log(f"rank-deficient statistics h={h} n={n}")
    x = wl.random_bf16((n, h), 0.3, 61)
    d = wl.random_bf16((n, h), 0.1, 62)
    g, c, e = (a.astype(np.float32).astype(np.float64) for a in orc.gram_statistics([x], [d]))
    wo = wl.random_bf16((h, h), 1.0 / np.sqrt(h), 63)
    dw_ref = orc.ridge_delta_w(g, c, wo, lam)
    _, er_ref = orc.layer_error_from_stats(g, c, e, wo, dw_ref, lam)
    G, C, E = f32_dev(g[None], c[None], e[None])
    Wo = dev_bf16(wo[None])
    dW, info, ws = ridge_gpu(G, C, Wo, lam)
    assert int(info[0]) == 0
    got = host(dW[0])
    dw_err = relfro(got, dw_ref)
    fit_err = relfro(x @ got.T, x @ dw_ref.T)
    log(f"  dW rel fro {dw_err:.2e}, X dW rel fro {fit_err:.2e}")
    assert dw_err <= DW_REL
    assert fit_err <= DW_REL
    ea, er, sel = score_gpu(G, C, E, Wo, dW, lam, info, 1, ws)
    log(f"  eps_rel {er[0]:.3e} oracle {er_ref:.3e}")
    assert ea[0] >= 0.0 and er[0] >= 0.0
    assert abs(er[0] - er_ref) <= eps_tol(er_ref, h), (er[0], er_ref)


def test_refinement_decided_per_layer():
    """One batched solve over layers that need the refinement step (200
    tokens at h = 1024: the fp32 solve alone is off by ~3e-3) and a layer that
    does not (4000 tokens, well conditioned): every layer's dW within 1e-3 of
    the oracle, so a refinement skipped where it was needed, or applied to the
    wrong layer, fails."""
    lam, h = 1e-2, 1024
    log("per-layer refinement h=1024: rank-deficient, full-rank, rank-deficient")
    stats = []
    for l, n in enumerate((200, 4000, 200)):
        x = wl.random_bf16((n, h), 0.3, 161 + 7 * l)
        d = wl.random_bf16((n, h), 0.1, 162 + 7 * l)
        stats.append(tuple(a.astype(np.float32).astype(np.float64)
                           for a in orc.gram_statistics([x], [d])))
    wo = np.stack([wl.random_bf16((h, h), 1.0 / np.sqrt(h), 163 + 7 * l) for l in range(3)])
    G, C, _ = f32_dev(*(np.stack([st[i] for st in stats]) for i in range(3)))
    dW, info, _ = ridge_gpu(G, C, dev_bf16(wo), lam)
    assert np.all(info.cpu().numpy() == 0)
    for l, (g, c, _) in enumerate(stats):
        err = relfro(host(dW[l]), orc.ridge_delta_w(g, c, wo[l], lam))
        log(f"  layer {l}: dW rel fro {err:.2e}")
        assert err <= DW_REL


# ------------------------------------------------------------------ ridge + score

def _synthetic_stats(L, h, n, seed):
    """Per-layer statistics from random activations with layer-dependent
    history strength (so the errors separate)."""
    Gs, Cs, Es, Ws = [], [], [], []
    for l in range(L):
        x = wl.random_bf16((n, h), 0.3, seed + 10 * l)
        dd = wl.random_bf16((n, h), 0.05 * (l + 1), seed + 10 * l + 1) + 0.3 * x * (l % 2)
        dd = wl.bf16_bits_to_f32(wl.round_to_bf16_bits(dd.astype(np.float32)))
        g, c, e = orc.gram_statistics([x], [dd])
        Gs.append(g); Cs.append(c); Es.append(e)
        Ws.append(wl.random_bf16((h, h), 1.0 / np.sqrt(h), seed + 10 * l + 2))
    f32 = lambda a: np.stack(a).astype(np.float32)
    hostside = (f32(Gs).astype(np.float64), f32(Cs).astype(np.float64),
                f32(Es).astype(np.float64), np.stack(Ws).astype(np.float64))
    G, C, E = f32_dev(*hostside[:3])
    return G, C, E, dev_bf16(np.stack(Ws)), hostside


@pytest.mark.parametrize("L,h,n", [(1, 128, 300), (3, 320, 500), (2, 64, 50), (2, 256, 400),
                                   (2, 200, 300), (2, 136, 300), (1, 160, 250)])
def test_ridge_and_score(L, h, n):
    log(f"ridge L={L} h={h} n={n}")
    lam = 1e-2
    G, C, E, Wo, (gh, ch, eh, wh) = _synthetic_stats(L, h, n, 100 + h)
    dW, info, ws = ridge_gpu(G, C, Wo, lam)
    assert np.all(info.cpu().numpy() == 0)
    eps_ref = []
    for l in range(L):
        ref = orc.ridge_delta_w(gh[l], ch[l], wh[l], lam)
        err = relfro(host(dW[l]), ref)
        log(f"  layer {l}: dW rel fro {err:.2e}")
        assert err <= DW_REL
        eps_ref.append(orc.layer_error_from_stats(gh[l], ch[l], eh[l], wh[l], ref, lam))
    ea, er, sel = score_gpu(G, C, E, Wo, dW, lam, info, max(1, L // 2), ws)
    assert np.all(ea >= 0.0) and np.all(er >= 0.0)
    for l in range(L):
        assert abs(er[l] - eps_ref[l][1]) <= eps_tol(eps_ref[l][1], h), (er[l], eps_ref[l])
        scale = eps_ref[l][0] / eps_ref[l][1] if eps_ref[l][1] > 0 else 1.0
        assert abs(ea[l] - eps_ref[l][0]) <= eps_tol(eps_ref[l][1], h) * scale
    np.testing.assert_array_equal(sel, orc.select_layers(np.array([e[1] for e in eps_ref]),
                                                         max(1, L // 2)))


def test_ridge_info_reports_failures():
    log("ridge info")
    h = 128
    G, C, E, Wo, _ = _synthetic_stats(3, h, 200, 7)
    G[1] = -torch.eye(h, device="cuda")          # not positive definite at the first pivot
    G[2, 5, 5] = float("nan")
    dW, info, ws = ridge_gpu(G, C, Wo, 0.0)
    inf = info.cpu().numpy()
    assert inf[0] == 0 and inf[1] == 1 and inf[2] != 0
    ea, er, sel = score_gpu(G, C, E, Wo, dW, 0.0, info, 3, ws)
    assert np.isinf(er[1]) and np.isinf(er[2]) and np.isfinite(er[0])
    np.testing.assert_array_equal(sel, [1, 0, 0])


def test_no_history_gives_zero_update():
    log("ridge zero history")
    h = 128
    x = wl.random_bf16((200, h), 0.3, 31)
    g, _, _ = orc.gram_statistics([x], [np.zeros_like(x)])
    G = torch.from_numpy(g[None].astype(np.float32)).cuda()
    C = torch.zeros_like(G)
    Wo = dev_bf16(wl.random_bf16((1, h, h), 0.1, 32))
    dW, info, ws = ridge_gpu(G, C, Wo, 1e-2)
    assert int(info[0]) == 0
    assert torch.count_nonzero(dW).item() == 0
    ea, er, sel = score_gpu(G, C, torch.zeros_like(G), Wo, dW, 1e-2, info, 1, ws)
    assert ea[0] == 0.0 and er[0] == 0.0 and sel[0] == 1


def test_warmup_tiny_stages():
    """Tiny case, stage by stage on the oracle's warmup: the solve and score
    on its statistics (fp32), the update and the projection of its last X."""
    w = wl.TINY
    log("warmup tiny stages")
    ref = oracle_chain(w)
    g, c, e = (a.astype(np.float32).astype(np.float64) for a in (ref["g"], ref["c"], ref["e"]))
    dw_ref = orc.ridge_delta_w(g, c, ref["wo"], w.lam)
    _, er_ref = orc.layer_error_from_stats(g, c, e, ref["wo"], dw_ref, w.lam)
    G, C, E = f32_dev(g[None], c[None], e[None])
    Wo = dev_bf16(ref["wo"][None])
    dW, info, ws = ridge_gpu(G, C, Wo, w.lam)
    assert relfro(host(dW[0]), dw_ref) <= DW_REL
    ea, er, sel = score_gpu(G, C, E, Wo, dW, w.lam, info, 1, ws)
    assert abs(er[0] - er_ref) <= eps_tol(er_ref, w.hidden)
    assert sel[0] == 1
    ispa.ispa_apply_dW(torch.from_numpy(sel).cuda(), dW, Wo)
    y = torch.empty((w.n_q, w.hidden), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_project(dev_bf16(ref["xs"][-1]), Wo[0], y)
    torch.cuda.synchronize()
    new_ref = orc.apply_delta(ref["wo"], dw_ref)
    # the GPU rounds W + its own dW: each stored element is within one bf16
    # rounding (unit roundoff 2^-8) of each exact sum, and the two sums differ
    # by the difference of the dW
    got_w, dw_got = host(Wo[0]), host(dW[0])
    bound = 2.0 ** -8 * (np.abs(ref["wo"] + dw_got) + np.abs(ref["wo"] + dw_ref)) + \
        np.abs(dw_got - dw_ref)
    assert np.all(np.abs(got_w - new_ref) <= bound)
    yref = orc.project(ref["xs"][-1], new_ref)
    assert relfro(host(y), yref) <= 4e-3


def test_warmup_tiny_gpu_chain():
    """The all-GPU warmup of the tiny case (attention output into the Gram,
    its statistics into the solve and the score) against the oracle's chain,
    at the chain bounds of the module docstring."""
    w = wl.TINY
    log("warmup tiny GPU chain")
    ref = oracle_chain(w)
    G, C, E = gpu_chain_stats(w)
    for name, t in (("G", G), ("C", C), ("E", E)):
        err = relfro(host(t[0]), ref[name.lower()])
        log(f"  {name} rel fro {err:.2e}")
        assert err <= CHAIN_STATS_REL, name
    Wo = dev_bf16(ref["wo"][None])
    dW, info, ws = ridge_gpu(G, C, Wo, w.lam)
    err = relfro(host(dW[0]), ref["dw"])
    ea, er, sel = score_gpu(G, C, E, Wo, dW, w.lam, info, 1, ws)
    log(f"  dW rel fro {err:.2e}, eps_rel {er[0]:.6e} oracle {ref['eps_rel']:.6e}")
    assert err <= CHAIN_DW_REL
    assert abs(er[0] - ref["eps_rel"]) <= CHAIN_EPS_REL * ref["eps_rel"]
    assert sel[0] == 1


# ------------------------------------------------------------------ apply + project

def test_apply_bit_exact():
    log("apply")
    L, h = 3, 256
    Wo_h = wl.random_bf16((L, h, h), 0.05, 41)
    dw_h = (np.random.default_rng(42).standard_normal((L, h, h)) * 1e-3).astype(np.float32)
    # plant exact fp32 ties: W + dW lands halfway between two bf16 values
    dw_h[0, 0, :8] = (np.ldexp(1.0, np.frexp(Wo_h[0, 0, :8])[1] - 9)).astype(np.float32)
    Wo = dev_bf16(Wo_h)
    dW = torch.from_numpy(dw_h).cuda()
    sel = torch.tensor([1, 0, 1], dtype=torch.int32, device="cuda")
    ispa.ispa_apply_dW(sel, dW, Wo)
    torch.cuda.synchronize()
    got = host(Wo)
    for l in range(L):
        exp = orc.apply_delta(Wo_h[l], dw_h[l]) if l != 1 else Wo_h[l]
        np.testing.assert_array_equal(got[l], exp)


@pytest.mark.parametrize("n,h_in,h_out", [(200, 128, 192), (4680, 1536, 1536), (7, 64, 64),
                                         (4680, 5120, 5120), (1000, 200, 72), (4700, 5120, 4096),
                                         (4680, 5088, 5120)])
def test_project(n, h_in, h_out):
    log(f"project {n}x{h_in}->{h_out}")
    x = wl.random_bf16((n, h_in), 0.5, 51)
    wt = wl.random_bf16((h_out, h_in), 1.0 / np.sqrt(h_in), 52)
    y = torch.empty((n, h_out), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_project(dev_bf16(x), dev_bf16(wt), y)
    torch.cuda.synchronize()
    ref = orc.project(x, wt)
    got = host(y)
    # bf16 output: each element within half a bf16 ulp of the fp32-accumulated value
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 1e-3)) <= 2 ** -8 + 1e-3
    assert relfro(got, ref) <= 4e-3


def test_project_input_above_2gib():
    """X above 2^31 bytes (220000 tokens x 5120, 2.25 GB): buffer offsets are
    32-bit, so the launch runs in row blocks below 2^31 bytes. The rows repeat
    1021 seeded rows (a prime period, so a block that read from the wrong
    offset would meet different rows); every 1021st-period row, and the rows
    around each block boundary, against the oracle."""
    n, h = 220000, 5120
    period = 1021
    log(f"project {n}x{h}->{h} (input above 2 GiB)")
    base = wl.random_bf16((period, h), 0.5, 53)
    wt = wl.random_bf16((h, h), 1.0 / np.sqrt(h), 54)
    idx = torch.arange(n, device="cuda") % period
    x = dev_bf16(base).index_select(0, idx)
    y = torch.empty((n, h), dtype=torch.bfloat16, device="cuda")
    ispa.ispa_project(x, dev_bf16(wt), y)
    torch.cuda.synchronize()
    del x
    ref = orc.project(base, wt)
    block = (2 ** 31 - 1) // (h * 2) // 256 * 256          # rows per launch
    rows = sorted(set(range(0, n, 997)) | {r for b in range(block, n, block)
                                          for r in (b - 1, b, b + 1) if r < n} | {n - 1})
    got = host(y[torch.tensor(rows, device="cuda")])
    exp = ref[np.array(rows) % period]
    assert np.max(np.abs(got - exp) / (np.abs(exp) + 1e-3)) <= 2 ** -8 + 1e-3


# ------------------------------------------------------------------ realistic conditioning

def test_wan13_layer_warmup_ridge():
    """1.3B-class layer (hidden 1536, history growing to 18 frames): the
    oracle's attention over 512 sampled query rows of each of the 4 warmup
    steps gives X and D with the spectrum of real attention outputs; the GPU
    Gram of those and the GPU solve of the oracle's statistics against the
    oracle's."""
    w = wl.WAN13_LAYER
    log("wan1.3b layer warmup + ridge")
    rows = np.linspace(0, w.n_q - 1, 512).astype(np.int64)
    ref = oracle_chain(w, rows=rows)
    G, C, _ = gram_of(ref["xs"], ref["ds"], w.hidden)
    assert relfro(host(G[0]), ref["g"]) <= GRAM_REL and relfro(host(C[0]), ref["c"]) <= GRAM_REL
    gh, ch = (a.astype(np.float32).astype(np.float64) for a in (ref["g"], ref["c"]))
    G, C = f32_dev(gh[None], ch[None])
    Wo = dev_bf16(ref["wo"][None])
    dW, info, ws = ridge_gpu(G, C, Wo, w.lam)
    assert int(info[0]) == 0
    ev = np.linalg.eigvalsh(gh + w.lam * np.eye(w.hidden))
    ref = orc.ridge_delta_w(gh, ch, ref["wo"], w.lam)
    err = relfro(host(dW[0]), ref)
    log(f"  cond(G+lam I) = {ev[-1] / ev[0]:.3e}, dW rel fro {err:.2e}")
    assert err <= DW_REL

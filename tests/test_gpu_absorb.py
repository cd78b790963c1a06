"""GPU parity of the warmup statistics, ridge solve, layer score, selection,
weight update and projection against the fp64 oracle.

Checks are stage-wise: each stage's oracle is fed the GPU's own inputs to
that stage (e.g. the oracle Gram sums the GPU-emitted bf16 X and D), so the
tolerance measures that stage alone. Tolerances: Gram relative Frobenius
<= 1e-5 (fp32 accumulation of exact bf16 products), dW relative Frobenius
<= 1e-3, eps relative <= 1e-4, selection identical, weight update
bit-exact.

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
from tests.gpu_helpers import dev_bf16, host, log, run_attention

pytestmark = pytest.mark.gpu

GRAM_REL = 1e-5
DW_REL = 1e-3
EPS_REL = 1e-4


def eps_tol(ref, h):
    return EPS_REL * abs(ref) + 4.0 * 2.0 ** -24 * np.sqrt(h)


def relfro(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))


def gpu_warmup_stats(w, layer=0, steps=None):
    """GPU attention for every warmup step of one layer, then the GPU Gram.
    Returns host X/D per step (bf16 values) and the GPU G, C, E tensors."""
    h = w.hidden
    G = torch.empty((1, h, h), dtype=torch.float32, device="cuda")
    C = torch.empty_like(G)
    E = torch.empty_like(G)
    xs, ds = [], []
    for s in range(w.n_steps if steps is None else steps):
        st = wl.step_inputs(w, layer, s)
        _, dev = run_attention(st, w.sm_scale, outputs=("o_local", "d"))
        ispa.ispa_gram_accumulate(dev["o_local"], dev["d"], G[0], C[0], E[0], zero_first=(s == 0))
        xs.append(host(dev["o_local"]))
        ds.append(host(dev["d"]))
    torch.cuda.synchronize()
    return xs, ds, G, C, E


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
    log("gram tiny warmup")
    xs, ds, G, C, E = gpu_warmup_stats(wl.TINY)
    g, c, e = orc.gram_statistics(xs, ds)
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


def test_score_hidden_5120():
    """Layer score at the 14B hidden size over 3 layers (W_o^T W_o by the
    G-only Gram launch batched over layers). Statistics, solve and score on
    the GPU; the error is checked against the oracle's formula on the GPU's
    G, C, E and dW."""
    L, h, n, lam = 3, 5120, 200, 1e-2
    log("score h=5120")
    x = wl.random_bf16((L, n, h), 0.3, 51)
    d = wl.random_bf16((L, n, h), 0.1, 52)
    G = torch.empty((L, h, h), dtype=torch.float32, device="cuda")
    C, E = torch.empty_like(G), torch.empty_like(G)
    ispa.ispa_gram_accumulate(dev_bf16(x), dev_bf16(d), G, C, E, zero_first=True)
    Wo = dev_bf16(wl.random_bf16((L, h, h), 1.0 / np.sqrt(h), 53))
    dW, info, ws = ridge_gpu(G, C, Wo, lam)
    assert np.all(info.cpu().numpy() == 0)
    ea, er, sel = score_gpu(G, C, E, Wo, dW, lam, info, 1, ws)
    for l in range(L):
        ref = orc.layer_error_from_stats(host(G[l]), host(C[l]), host(E[l]), host(Wo[l]),
                                         host(dW[l]), lam)
        log(f"  layer {l}: eps_rel {er[l]:.6e} oracle {ref[1]:.6e}")
        assert abs(er[l] - ref[1]) <= eps_tol(ref[1], h), (er[l], ref)


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
    f32 = lambda a: torch.from_numpy(np.stack(a).astype(np.float32)).cuda()
    return f32(Gs), f32(Cs), f32(Es), dev_bf16(np.stack(Ws))


@pytest.mark.parametrize("L,h,n", [(1, 128, 300), (3, 320, 500), (2, 64, 50), (2, 256, 400)])
def test_ridge_and_score(L, h, n):
    log(f"ridge L={L} h={h} n={n}")
    lam = 1e-2
    G, C, E, Wo = _synthetic_stats(L, h, n, 100 + h)
    dW, info, ws = ridge_gpu(G, C, Wo, lam)
    assert np.all(info.cpu().numpy() == 0)
    eps_ref = []
    for l in range(L):
        ref = orc.ridge_delta_w(host(G[l]), host(C[l]), host(Wo[l]), lam)
        err = relfro(host(dW[l]), ref)
        log(f"  layer {l}: dW rel fro {err:.2e}")
        assert err <= DW_REL
        eps_ref.append(orc.layer_error_from_stats(host(G[l]), host(C[l]), host(E[l]),
                                                  host(Wo[l]), ref, lam))
    ea, er, sel = score_gpu(G, C, E, Wo, dW, lam, info, max(1, L // 2), ws)
    for l in range(L):
        assert abs(er[l] - eps_ref[l][1]) <= eps_tol(eps_ref[l][1], h), (er[l], eps_ref[l])
        scale = eps_ref[l][0] / eps_ref[l][1] if eps_ref[l][1] > 0 else 1.0
        assert abs(ea[l] - eps_ref[l][0]) <= eps_tol(eps_ref[l][1], h) * scale
    np.testing.assert_array_equal(sel, orc.select_layers(np.array([e[1] for e in eps_ref]),
                                                         max(1, L // 2)))


def test_ridge_info_reports_failures():
    log("ridge info")
    h = 128
    G, C, E, Wo = _synthetic_stats(3, h, 200, 7)
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


def test_warmup_tiny_end_to_end():
    """Tiny case through every stage; selection, update and projection."""
    w = wl.TINY
    log("warmup tiny end to end")
    xs, ds, G, C, E = gpu_warmup_stats(w)
    Wo = dev_bf16(wl.output_projection(w, 0)[None])
    dW, info, ws = ridge_gpu(G, C, Wo, w.lam)
    ref = orc.ridge_delta_w(host(G[0]), host(C[0]), host(Wo[0]), w.lam)
    assert relfro(host(dW[0]), ref) <= DW_REL
    ea, er, sel = score_gpu(G, C, E, Wo, dW, w.lam, info, 1, ws)
    _, er_ref = orc.layer_error_from_stats(host(G[0]), host(C[0]), host(E[0]), host(Wo[0]), ref,
                                           w.lam)
    assert abs(er[0] - er_ref) <= eps_tol(er_ref, w.hidden)
    # the error of the GPU update on the stored activations, directly
    x_all, z_all = np.concatenate(xs), np.concatenate(xs) + np.concatenate(ds)
    _, er_direct = orc.layer_error_direct(x_all, z_all, host(Wo[0]), host(dW[0]))
    assert abs(er[0] - er_direct) <= 1e-3 * er_direct + eps_tol(0.0, w.hidden)


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


@pytest.mark.parametrize("n,h_in,h_out", [(200, 128, 192), (4680, 1536, 1536), (7, 64, 64)])
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


# ------------------------------------------------------------------ realistic conditioning

def test_wan13_layer_warmup_ridge():
    """1.3B-class layer: 4 warmup steps of 4680 tokens (hidden 1536, history
    18 frames), statistics and solve on the GPU, oracle solve on the GPU's
    statistics."""
    w = wl.WAN13_LAYER
    log("wan1.3b layer warmup + ridge")
    xs, ds, G, C, E = gpu_warmup_stats(w)
    g, c, e = orc.gram_statistics(xs, ds)
    assert relfro(host(G[0]), g) <= GRAM_REL and relfro(host(C[0]), c) <= GRAM_REL
    Wo = dev_bf16(wl.output_projection(w, 0)[None])
    dW, info, ws = ridge_gpu(G, C, Wo, w.lam)
    assert int(info[0]) == 0
    Gh = host(G[0])
    ev = np.linalg.eigvalsh(Gh + w.lam * np.eye(w.hidden))
    ref = orc.ridge_delta_w(Gh, host(C[0]), host(Wo[0]), w.lam)
    err = relfro(host(dW[0]), ref)
    log(f"  cond(G+lam I) = {ev[-1] / ev[0]:.3e}, dW rel fro {err:.2e}")
    assert err <= DW_REL

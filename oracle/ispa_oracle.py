"""Plain fp64 CPU oracle for the ISPA hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module:
only the test suite, the smoke check and the CPU-baseline leg of the benchmark
use it. It shares no code with the HIP library (no kernels, helpers or
constants); both sides only take their seeded inputs from ``workloads``.

Source: the ISPA paper, "Towards Memory-Efficient Autoregressive Video
Generation via Instance-Specific Parametric Absorption" (page text at
paperpeel.com), and the reading notes on it at paper.gecl.asia ("Core Idea",
"Method"). Everything here is the plain definition of what the method
computes, written out directly in float64 with numpy:

* attention over a KV set is ordinary softmax attention, computed separately
  for the local set (sink + current), the history and the concatenated full
  set. The full output is *not* obtained by merging partial results: the merge
  is what the fast path does, and the oracle checks it instead of using it;
* warmup statistics are plain sums over all warmup tokens;
* the absorbed update is the closed-form ridge solution solved densely with
  ``numpy.linalg.solve``;
* the layer error is the residual of the absorbed reconstruction;
* selection is a stable ascending sort.

Conventions (row vectors): an attention output X = A_loc and Z = A_full are
[N, h] with column head*d + j; the output projection is Y = X @ W_o^T with
W_o stored as nn.Linear [out, in]. Inside the math W = W_o^T ([in, out]).

Where the pages are silent the readings used are:
  lambda is added unscaled to the summed statistics; LSE is natural log;
  the softmax scale is 1/sqrt(d); no masking inside a chunk; an empty KV set
  gives O = 0 and LSE = -inf; a layer whose solve failed or whose error is
  NaN gets error +inf and is never selected; equal errors keep the lower
  layer index first.

Every function below is pinned by tests under ``tests/test_oracle_*.py``
against closed forms, brute force and independent library routines.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_BLOCK_Q = 512


# ---------------------------------------------------------------------------
# Attention (ISPA paper §3.1 item 1: A_full uses the whole history, A_loc
# uses only current and sink tokens; §3.4: both come from one forward pass)
# ---------------------------------------------------------------------------

def softmax_attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one head over one KV set.

    q [nq, d], k [n, d], v [n, d] -> (O [nq, d], LSE [nq]) with
    s = scale * q k^T, m = max_j s, l = sum_j exp(s - m), O = sum_j
    exp(s_j - m) v_j / l and LSE = m + ln l (natural log). n = 0 gives O = 0,
    LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, d = q.shape
    n = k.shape[0]
    out = np.zeros((nq, v.shape[1] if v.ndim == 2 else d), dtype=np.float64)
    lse = np.full(nq, -np.inf, dtype=np.float64)
    if n == 0:
        return out, lse
    for q0 in range(0, nq, _BLOCK_Q):
        qb = q[q0:q0 + _BLOCK_Q]
        s = scale * (qb @ k.T)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[q0:q0 + _BLOCK_Q] = (p @ v) / l
        lse[q0:q0 + _BLOCK_Q] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def multihead_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                        scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """q [nq, nh, d], k/v [n, nh, d] -> O [nq, nh*d] (column head*d + j),
    LSE [nh, nq]."""
    nq, nh, d = q.shape
    o = np.zeros((nq, nh, d), dtype=np.float64)
    lse = np.zeros((nh, nq), dtype=np.float64)
    for hd in range(nh):
        o[:, hd, :], lse[hd] = softmax_attention_head(q[:, hd, :], k[:, hd, :],
                                                      v[:, hd, :], scale)
    return o.reshape(nq, nh * d), lse


def decomposable_attention(q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist,
                           scale: float) -> Dict[str, np.ndarray]:
    """The three attention results the warmup needs, each computed directly.

    local = attention over sink + current (A_loc), hist = attention over the
    history alone, full = attention over the concatenated sink + history +
    current (A_full). D = O_full - O_local is the discrepancy the absorption
    fits (gecl.asia notes, "Method": the full-local output difference is the
    supervision signal).
    """
    k_loc = np.concatenate([k_sink, k_cur], axis=0)
    v_loc = np.concatenate([v_sink, v_cur], axis=0)
    k_full = np.concatenate([k_sink, k_hist, k_cur], axis=0)
    v_full = np.concatenate([v_sink, v_hist, v_cur], axis=0)
    o_l, lse_l = multihead_attention(q, k_loc, v_loc, scale)
    o_h, lse_h = multihead_attention(q, k_hist, v_hist, scale)
    o_f, lse_f = multihead_attention(q, k_full, v_full, scale)
    return {"o_local": o_l, "lse_local": lse_l, "o_hist": o_h,
            "lse_hist": lse_h, "o_full": o_f, "lse_full": lse_f,
            "d": o_f - o_l}


def merge_partials(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Combine attention results over two disjoint KV sets (ISPA paper §3.4,
    online-softmax decomposition via the log-sum-exp states).

    o_* [nq, nh*d], lse_* [nh, nq]. Returns the result over the union. Used by
    the tests to check the identity the fast path relies on; the oracle never
    produces O_full this way.
    """
    nh, nq = lse_a.shape
    d = o_a.shape[1] // nh
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - lse))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - lse))
    oa = o_a.reshape(nq, nh, d)
    ob = o_b.reshape(nq, nh, d)
    o = wa.T[:, :, None] * oa + wb.T[:, :, None] * ob
    return o.reshape(nq, nh * d), lse


# ---------------------------------------------------------------------------
# Warmup statistics (ISPA paper §3.1 item 2: "the accumulated dual-stream
# activations serve as the basis for weight adaption")
# ---------------------------------------------------------------------------

def gram_statistics(xs: Sequence[np.ndarray], ds: Sequence[np.ndarray]
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Sums over every warmup step of G = X^T X, C = X^T D, E = D^T D.

    xs, ds: per-step [N_s, h] local outputs and full-minus-local
    differences. These three sums are all the solve and the error need.
    """
    h = xs[0].shape[1]
    g = np.zeros((h, h))
    c = np.zeros((h, h))
    e = np.zeros((h, h))
    for x, dd in zip(xs, ds):
        x = np.asarray(x, dtype=np.float64)
        dd = np.asarray(dd, dtype=np.float64)
        g += x.T @ x
        c += x.T @ dd
        e += dd.T @ dd
    return g, c, e


# ---------------------------------------------------------------------------
# Layer absorb (ISPA paper §3.1 item 2 and §3.2: a least-squares fit of a
# modulation of the output projection so that the local output through
# W + dW reproduces the full output through W; §4.1: a ridge parameter
# lambda balances keeping the pre-trained weights; gecl.asia notes, "Method":
# ridge regression on the attention output projection)
# ---------------------------------------------------------------------------

def ridge_delta_w(g: np.ndarray, c: np.ndarray, wo: np.ndarray, lam: float
                  ) -> np.ndarray:
    """dW minimising ||X (W + dW) - Z W||_F^2 + lam ||dW||_F^2.

    With Z = X + D the minimiser is dW = (G + lam I)^{-1} C W (W = wo^T,
    [in, out]). Returned in nn.Linear layout [out, in] (i.e. dW^T), like wo.
    """
    g = np.asarray(g, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    w = np.asarray(wo, dtype=np.float64).T
    h = g.shape[0]
    dw = np.linalg.solve(g + lam * np.eye(h), c @ w)
    return dw.T.copy()


def layer_error_from_stats(g, c, e, wo, dwo, lam: float) -> Tuple[float, float]:
    """Reconstruction error of the absorbed layer from the statistics.

    eps_abs = ||X (W + dW) - Z W||_F^2 over all warmup tokens
            = tr(dW^T G dW) - 2 tr(dW^T C W) + tr(W^T E W)
    eps_rel = eps_abs / ||Z W||_F^2, with Z^T Z = G + C + C^T + E.
    (ISPA paper §3.3: the error metric used to rank layers; its definition is
    lost from the page text, this is the residual of the reconstruction named
    in the §3.2 title.)
    """
    g = np.asarray(g, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    w = np.asarray(wo, dtype=np.float64).T
    dw = np.asarray(dwo, dtype=np.float64).T
    quad = np.sum(dw * (g @ dw))
    cross = np.sum(dw * (c @ w))
    tew = np.sum(w * (e @ w))
    eps_abs = quad - 2.0 * cross + tew
    zz = g + c + c.T + e
    denom = np.sum(w * (zz @ w))
    eps_rel = eps_abs / denom if denom > 0 else (0.0 if eps_abs == 0 else math.inf)
    return float(eps_abs), float(eps_rel)


def layer_error_direct(x_all, z_all, wo, dwo) -> Tuple[float, float]:
    """The same error evaluated on the stacked warmup activations."""
    w = np.asarray(wo, dtype=np.float64).T
    dw = np.asarray(dwo, dtype=np.float64).T
    x_all = np.asarray(x_all, dtype=np.float64)
    z_all = np.asarray(z_all, dtype=np.float64)
    target = z_all @ w
    r = x_all @ (w + dw) - target
    eps_abs = float(np.sum(r * r))
    denom = float(np.sum(target * target))
    return eps_abs, (eps_abs / denom if denom > 0 else
                     (0.0 if eps_abs == 0 else math.inf))


# ---------------------------------------------------------------------------
# Dynamic layer selection (ISPA paper §3.3: rank layers by ascending error,
# the K lowest become L-layers)
# ---------------------------------------------------------------------------

def select_layers(eps: np.ndarray, k: int,
                  valid: Optional[np.ndarray] = None) -> np.ndarray:
    """int32 [L] with 1 for the min(K, #valid) lowest-error layers.

    Invalid layers (failed solve) and NaN errors count as +inf and are never
    selected; equal errors keep the lower layer index first.
    """
    eps = np.array(eps, dtype=np.float64)
    n = eps.shape[0]
    if valid is None:
        valid = np.ones(n, dtype=bool)
    key = np.where(valid & ~np.isnan(eps), eps, np.inf)
    order = np.argsort(key, kind="stable")
    sel = np.zeros(n, dtype=np.int32)
    taken = 0
    for idx in order:
        if taken >= k or not np.isfinite(key[idx]):
            break
        sel[idx] = 1
        taken += 1
    return sel


# ---------------------------------------------------------------------------
# Weight injection (ISPA paper §3.3: W_new = W + dW, updated in place in the
# weight's own storage type, bf16 here)
# ---------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Correctly rounded fp64 -> bf16 (nearest, ties to even), returned as
    fp64 values.

    A bf16 has an 8-bit significand: for |x| = m * 2^ex with m in [0.5, 1)
    the representable spacing is 2^(ex-8) (never below the subnormal spacing
    2^-133). Dividing by that power of two is exact in fp64, so rounding the
    quotient to an integer with ties-to-even (numpy.rint) and scaling back is
    the exact rounding. Magnitudes that round to 2^128 or more overflow to
    inf.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, ex = np.frexp(ax)
    ulp = np.ldexp(1.0, np.maximum(ex - 8, -133))
    mag = np.rint(ax / ulp) * ulp
    mag = np.where(mag >= 2.0 ** 128, np.inf, mag)
    out = np.copysign(mag, x)
    keep = (ax == 0.0) | ~np.isfinite(x)
    return np.where(keep, x, out)


def apply_delta(wo: np.ndarray, dwo: np.ndarray) -> np.ndarray:
    """bf16 storage of W_o + dW (both [out, in])."""
    return bf16_round(np.asarray(wo, dtype=np.float64) +
                      np.asarray(dwo, dtype=np.float64))


def project(x: np.ndarray, wo: np.ndarray) -> np.ndarray:
    """L-layer output projection Y = X W^T for x [N, in], wo [out, in]
    (ISPA paper §3.1 item 3: L-layers use local attention with W_new)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(wo, dtype=np.float64).T


# ---------------------------------------------------------------------------
# Whole warmup (ISPA paper §3.1 items 1-3) for small cases
# ---------------------------------------------------------------------------

def stored_activations(o_local, o_full) -> Tuple[np.ndarray, np.ndarray]:
    """The warmup activations as a bf16 model keeps them: X = bf16(O_local)
    and D = bf16(O_full - O_local), each the rounding of its exact value, so
    that D = 0 exactly when there is no history. (Reading: the pages do not
    fix the precision of the collected activations; they are kept in the
    model's bf16 activation dtype.)"""
    o_local = np.asarray(o_local, dtype=np.float64)
    return bf16_round(o_local), bf16_round(np.asarray(o_full, dtype=np.float64) - o_local)


def run_warmup_layer(steps, wo, lam: float, scale: float, store_bf16: bool = False):
    """steps: iterable of workloads.StepInputs for one layer. With
    store_bf16 the statistics are taken over stored_activations (bf16 X and
    D) instead of the exact fp64 ones. Returns dict with stacked X/Z,
    statistics, dW and the error."""
    xs, ds, zs = [], [], []
    for st in steps:
        r = decomposable_attention(st.q, st.k_sink, st.v_sink, st.k_cur,
                                   st.v_cur, st.k_hist, st.v_hist, scale)
        if store_bf16:
            x, d = stored_activations(r["o_local"], r["o_full"])
        else:
            x, d = r["o_local"], r["d"]
        xs.append(x)
        ds.append(d)
        zs.append(x + d)
    g, c, e = gram_statistics(xs, ds)
    dw = ridge_delta_w(g, c, wo, lam)
    eps_abs, eps_rel = layer_error_from_stats(g, c, e, wo, dw, lam)
    return {"x_all": np.concatenate(xs), "z_all": np.concatenate(zs),
            "d_all": np.concatenate(ds), "g": g, "c": c, "e": e, "dw": dw,
            "eps_abs": eps_abs, "eps_rel": eps_rel}


# ---------------------------------------------------------------------------
# Streaming after the transition (ISPA paper §3.1 item 3 and §3.3: the K
# selected layers take W + dW and permanently drop their history KV, so they
# attend the sink and current tokens only; the other layers keep attending
# the whole history through the original W)
# ---------------------------------------------------------------------------

def history_chunks(c: int, capacity_chunks: Optional[int] = None) -> list:
    """Indices of the earlier chunks that a full-history layer attends while
    chunk c (0-based, counted from the first chunk the cache saw) is
    current. The paper keeps the whole history (capacity None); a finite
    capacity keeps the `capacity_chunks` most recent chunks, dropping the
    oldest first."""
    lo = 0 if capacity_chunks is None else max(0, c - capacity_chunks)
    return list(range(lo, c))


def stream_layer_chunk(q, k_sink, v_sink, k_chunks, v_chunks, c: int, wo,
                       scale: float, *, local_only: bool,
                       capacity_chunks: Optional[int] = None):
    """One layer while chunk c is current. k_chunks / v_chunks hold the
    [n_cur, nh, d] keys / values of chunks 0..c in order (chunk c is the
    current one). An L-layer (local_only) attends sink + current; an F-layer
    attends sink + its history chunks + current, the keys concatenated in
    time order. Returns (O [nq, h], Y = O wo^T)."""
    hist = [] if local_only else history_chunks(c, capacity_chunks)
    k = np.concatenate([k_sink] + [k_chunks[i] for i in hist] + [k_chunks[c]], axis=0)
    v = np.concatenate([v_sink] + [v_chunks[i] for i in hist] + [v_chunks[c]], axis=0)
    o, _ = multihead_attention(q, k, v, scale)
    return o, project(o, wo)


# ---------------------------------------------------------------------------
# Event-triggered recalibration (ISPA paper §3.3, last paragraph: on a large
# scene transition or temporal distribution shift the warmup-to-absorption
# procedure is re-entered: dual-stream warmup again, errors recomputed, the
# absorbed layer set and dW refreshed for the new context). The pages give no
# trigger; the reading used here is a drift score of an L-layer's local
# outputs against the warmup statistics its dW was fitted on.
# ---------------------------------------------------------------------------

def drift_reference(g: np.ndarray, lam: float, n_warm: int) -> float:
    """Expected leverage x (G + lam I)^{-1} x^T of a warmup token:
    tr((G + lam I)^{-1} G) / N, N the number of warmup tokens in G."""
    g = np.asarray(g, dtype=np.float64)
    m = g + lam * np.eye(g.shape[0])
    return float(np.trace(np.linalg.solve(m, g)) / n_warm)


def drift_score(x: np.ndarray, g: np.ndarray, lam: float, n_warm: int) -> float:
    """Mean leverage of the rows of x (a sample of a chunk's local outputs
    X = O_local of one layer) under the warmup statistics, divided by its
    warmup expectation: 1 on average for tokens like the warmup ones, large
    when the chunk's activations leave the span the ridge fit was supported
    on (there the absorbed dW extrapolates)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = g + lam * np.eye(g.shape[0])
    lev = np.einsum("ij,ji->i", x, np.linalg.solve(m, x.T))
    return float(lev.mean() / drift_reference(g, lam, n_warm))


# ---------------------------------------------------------------------------
# W8A8 output projection (ISPA paper §4.4, "Compatibility with Post-Training
# Quantization": 8-bit weights and activations for the linear layers; here
# the L-layer's W + dW is quantized after the update is folded in). Format:
# OCP 8-bit floating point E4M3 (the "fn" variant: bias 7, no infinities,
# S.1111.111 is NaN, largest finite 448). Readings: per-output-channel
# weight scales and per-token activation scales, each absmax / 448, with
# round-to-nearest-even codes saturated at +-448; the scale and the scaled
# value are formed in fp32 (as the kernel forms them), so both sides take
# the same code decisions.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """Value of E4M3 codes (uint8): sign, 4 exponent bits (bias 7) and 3
    mantissa bits; exponent field 0 holds the subnormals m * 2^-9; code
    0x7F / 0xFF is NaN."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), values beyond
    +-448 saturated to +-448; NaN maps to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), E4M3_MAX)
    # quantum of the binade holding ax: 2^(e-3) for normal values, 2^-9 below 2^-6
    ex = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    q = np.where(ax < 2.0 ** -6, 2.0 ** -9, 2.0 ** (ex - 3))
    n = ax / q
    r = np.floor(n)
    frac = n - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (r % 2 == 1)), r + 1, r)
    mag = r * q
    # magnitude -> code: exponent field and mantissa field
    e_f = np.where(mag < 2.0 ** -6, 0, np.floor(np.log2(np.where(mag > 0, mag, 1.0))) + 7)
    m_f = np.where(e_f == 0, np.round(mag / 2.0 ** -9), np.round((mag / 2.0 ** (e_f - 7) - 1) * 8))
    code = (e_f.astype(np.int64) << 3) | m_f.astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return np.where(np.isnan(x), 0x7F, code).astype(np.uint8)


def quantize_rows(a):
    """Per-row E4M3 quantization of a [rows, k] matrix: absmax a = max |row|
    (fp32), scale = a / 448 and inv = 448 / a (fp32 divisions; both 0 for an
    all-zero row), codes = e4m3(fp32(value * inv)). Returns (codes uint8,
    scale float32)."""
    a32 = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(a32), axis=1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    scale = np.where(nz, safe / np.float32(E4M3_MAX), np.float32(0)).astype(np.float32)
    inv = np.where(nz, np.float32(E4M3_MAX) / safe, np.float32(0)).astype(np.float32)
    scaled = (a32 * inv[:, None]).astype(np.float32)
    return e4m3_encode(scaled), scale


def project_w8a8(x, wq, w_scale) -> np.ndarray:
    """W8A8 projection: the activations x [N, in] are quantized per token,
    then Y[m][o] = s_x[m] s_w[o] sum_k dq(Xq[m][k]) dq(Wq[o][k]) (exact)."""
    xq, x_scale = quantize_rows(x)
    acc = e4m3_decode(xq) @ e4m3_decode(wq).T
    return acc * np.asarray(x_scale, dtype=np.float64)[:, None] * \
        np.asarray(w_scale, dtype=np.float64)[None, :]


# ---------------------------------------------------------------------------
# Quantized decomposable attention (the ISPA paper's §3.4 builds on
# FlashAttention-style LSE states and cites SageAttention's 8-bit attention;
# §4.4 pairs ISPA with 8-bit quantization). Q K^T on E4M3 codes: each query
# row (token, head) has its own scale; the keys are first smoothed by a
# vector mu per head (subtracting the same vector from every key shifts all
# of a query's scores by the same amount, so the softmax is unchanged and
# only the LSE moves, by scale * q . mu, which is added back), then quantized
# with one scale per head and per run of KEY_TILE keys from the start of
# each KV segment. V, P and P V stay at bf16 precision.
# ---------------------------------------------------------------------------

KEY_TILE = 64


def quantize_key_tiles(k, mu=None, tile: int = KEY_TILE):
    """E4M3 quantization of one key segment k [n, nh, d] after smoothing:
    r = fp32(k - mu) (mu [nh, d], the same for every key; None = 0), then for
    each head and each run of `tile` keys from the segment start, the absmax
    a of r over the run's tile x d values, scale = a / 448 and codes =
    e4m3(fp32(r * (448 / a))) as in quantize_rows. Returns (codes [n, nh, d]
    uint8, scales [n_tiles, nh] float32)."""
    k32 = np.asarray(k, dtype=np.float32)
    n, nh, d = k32.shape
    m32 = np.zeros((nh, d), dtype=np.float32) if mu is None else \
        np.asarray(mu, dtype=np.float32).reshape(nh, d)
    r = (k32 - m32[None]).astype(np.float32)
    n_tiles = (n + tile - 1) // tile
    codes = np.zeros((n, nh, d), dtype=np.uint8)
    scales = np.zeros((n_tiles, nh), dtype=np.float32)
    for t in range(n_tiles):
        blk = r[t * tile:(t + 1) * tile]                      # [rows, nh, d]
        per_head = blk.transpose(1, 0, 2).reshape(nh, -1)     # one row per head
        c, s = quantize_rows(per_head)
        codes[t * tile:(t + 1) * tile] = c.reshape(nh, blk.shape[0], d).transpose(1, 0, 2)
        scales[t] = s
    return codes, scales


def quantize_queries(q):
    """Per-(token, head) E4M3 quantization of q [nq, nh, d]: codes [nq, nh, d],
    scales [nh, nq] (the layout of the LSE outputs)."""
    nq, nh, d = np.shape(q)
    c, s = quantize_rows(np.asarray(q).reshape(nq * nh, d))
    return c.reshape(nq, nh, d), s.reshape(nq, nh).T.copy()


def dequantized_keys(k, mu=None, tile: int = KEY_TILE) -> np.ndarray:
    """The smoothed keys as the quantized attention sees them: dq(codes) x the
    scale of their tile and head (exact in fp64)."""
    k = np.asarray(k)
    if k.shape[0] == 0:
        return np.zeros(k.shape, dtype=np.float64)
    c, s = quantize_key_tiles(k, mu, tile)
    per_row = np.repeat(s.astype(np.float64), tile, axis=0)[:k.shape[0]]
    return e4m3_decode(c) * per_row[:, :, None]


def key_mean(*segments) -> np.ndarray:
    """Mean over all keys of the given segments [n_s, nh, d] -> [nh, d]
    (fp64); a smoothing vector for quantize_key_tiles."""
    ks = [np.asarray(k, dtype=np.float64) for k in segments if np.shape(k)[0] > 0]
    allk = np.concatenate(ks, axis=0)
    return allk.mean(axis=0)


def decomposable_attention_fp8(q, k_sink, v_sink, k_cur, v_cur, k_hist, v_hist,
                               scale: float, mu=None) -> Dict[str, np.ndarray]:
    """decomposable_attention with the scores formed from E4M3 codes: queries
    quantized per (token, head), keys smoothed by mu and quantized per
    (segment tile, head); the scores are scale * dq(q) . dq(k - mu) with the
    products exact, V unquantized, and every LSE output shifted back by
    scale * q . mu (the unquantized q)."""
    qc, qs = quantize_queries(q)
    q_dq = e4m3_decode(qc) * qs.T.astype(np.float64)[:, :, None]
    r = decomposable_attention(q_dq, dequantized_keys(k_sink, mu), v_sink,
                               dequantized_keys(k_cur, mu), v_cur,
                               dequantized_keys(k_hist, mu), v_hist, scale)
    if mu is not None:
        nh, d = np.shape(q)[1], np.shape(q)[2]
        m64 = np.asarray(mu, dtype=np.float64).reshape(nh, d)
        shift = scale * np.einsum("qhd,hd->hq", np.asarray(q, dtype=np.float64), m64)
        for key in ("lse_local", "lse_hist", "lse_full"):
            r[key] = r[key] + shift
    return r

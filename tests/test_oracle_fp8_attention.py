"""Pins of the oracle's quantized decomposable attention (ISPA paper §3.4:
decomposable attention on LSE states, citing SageAttention's 8-bit attention;
§4.4: 8-bit quantization on top of ISPA).

Pinned against exact special cases and properties, not against a retyping:
* inputs already on the E4M3 grid with per-block absmax 448 quantize with
  scale 1 and decode to themselves, so the quantized attention must equal the
  plain one exactly; with keys shifted by a smoothing vector mu the same holds
  only if the smoothing, its sign and the LSE shift back are all right;
* tiles run from each segment's start: editing one tile changes only it;
* scaling by a power of two scales the scales and leaves the codes alone;
* the reconstruction error stays inside E4M3's half-ulp bound;
* smoothing by the key mean cuts the error when keys share a large bias
  (the case SageAttention's smoothing is for).
"""
import numpy as np

import oracle.ispa_oracle as orc
import workloads as wl


def grid_blocks(shape, block_axes_last, rng):
    """E4M3 grid values with one element of every block (the product of the
    trailing `block_axes_last` axes) set to +-448."""
    codes = rng.integers(0, 0x7E, size=shape, dtype=np.int64)
    codes |= rng.integers(0, 2, size=shape) << 7
    vals = orc.e4m3_decode(codes.astype(np.uint8))
    flat = vals.reshape(-1, int(np.prod(shape[-block_axes_last:])))
    flat[:, 0] = np.where(rng.integers(0, 2, size=flat.shape[0]) == 1, 448.0, -448.0)
    return flat.reshape(shape)


def test_queries_on_grid_quantize_exactly():
    rng = np.random.default_rng(1)
    q = grid_blocks((50, 3, 64), 1, rng)
    c, s = orc.quantize_queries(q)
    assert s.shape == (3, 50) and np.all(s == 1.0)
    np.testing.assert_array_equal(orc.e4m3_decode(c), q)


def test_key_tiles_exact_grid_with_smoothing():
    """K = K0 + mu with K0 on the grid (multiples of 32, absmax 448 in every
    64-key tile of every head) and mu multiples of 32: k - mu is exact, so
    every scale is 1 and the codes decode to K0."""
    rng = np.random.default_rng(2)
    n, nh, d = 150, 2, 32
    k0 = 32.0 * rng.integers(-13, 14, size=(n, nh, d))
    for t in range(0, n, 64):
        k0[t, :, 0] = 448.0
    mu = 32.0 * rng.integers(-2, 3, size=(nh, d))
    c, s = orc.quantize_key_tiles(k0 + mu[None], mu)
    assert s.shape == (3, nh) and np.all(s == 1.0)
    np.testing.assert_array_equal(orc.e4m3_decode(c), k0)
    # without the smoothing the scales differ (the check above is not vacuous)
    _, s0 = orc.quantize_key_tiles(k0 + mu[None], None)
    assert np.any(s0 != 1.0)


def test_quantized_attention_equals_plain_on_grid_inputs():
    """On-grid queries and smoothed keys: the quantized attention is the plain
    attention of the same inputs (O and every LSE), history empty or not."""
    rng = np.random.default_rng(3)
    nh, d, nq = 2, 32, 40
    scale = 1.0 / (448.0 * 448.0)
    q = grid_blocks((nq, nh, d), 1, rng)
    mu = 32.0 * rng.integers(-2, 3, size=(nh, d))

    def keys(n):
        k0 = 32.0 * rng.integers(-13, 14, size=(n, nh, d))
        for t in range(0, n, 64):
            k0[t, :, 0] = -448.0
        return k0 + mu[None]

    ks, kc, kh = keys(20), keys(70), keys(130)
    vs, vc, vh = (wl.random_bf16((n, nh, d), 1.0, 40 + n) for n in (20, 70, 130))
    for hist in (True, False):
        kh_, vh_ = (kh, vh) if hist else (kh[:0], vh[:0])
        ref = orc.decomposable_attention(q, ks, vs, kc, vc, kh_, vh_, scale)
        got = orc.decomposable_attention_fp8(q, ks, vs, kc, vc, kh_, vh_, scale, mu)
        for key in ref:
            a, b = got[key], ref[key]
            fin = np.isfinite(b)
            assert np.array_equal(np.isfinite(a), fin), key
            np.testing.assert_allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12, err_msg=key)
    # a wrong smoothing sign or a missing LSE shift breaks the equality
    bad = orc.decomposable_attention_fp8(q, ks, vs, kc, vc, kh, vh, scale, -mu)
    ref = orc.decomposable_attention(q, ks, vs, kc, vc, kh, vh, scale)
    assert np.max(np.abs(bad["lse_full"] - ref["lse_full"])) > 1e-3


def test_tiles_start_at_segment_start_and_are_independent():
    k = wl.random_bf16((200, 2, 64), 1.0, 11)
    c, s = orc.quantize_key_tiles(k)
    k2 = k.copy()
    k2[64:128] *= 4.0                           # tile 1 only
    c2, s2 = orc.quantize_key_tiles(k2)
    for t in (0, 2, 3):
        rows = slice(64 * t, 64 * (t + 1))
        np.testing.assert_array_equal(c2[rows], c[rows])
        assert np.array_equal(s2[t], s[t])
    np.testing.assert_array_equal(c2[64:128], c[64:128])   # power of two: same codes
    np.testing.assert_array_equal(s2[1], 4.0 * s[1])
    # the last, partial tile (8 keys) has its own scale
    assert s.shape == (4, 2)
    last = np.max(np.abs(k[192:].astype(np.float32)), axis=(0, 2)) / np.float32(448)
    np.testing.assert_array_equal(s[3], last)


def test_reconstruction_within_half_ulp():
    k = wl.random_bf16((300, 3, 128), 1.0, 12) + 2.0 * wl.random_bf16((1, 3, 128), 1.0, 13)
    mu = orc.bf16_round(orc.key_mean(k))
    r = k.astype(np.float32) - mu.astype(np.float32)[None]
    deq = orc.dequantized_keys(k, mu)
    c, s = orc.quantize_key_tiles(k, mu)
    srow = np.repeat(s.astype(np.float64), 64, axis=0)[:300][:, :, None]
    # half an E4M3 ulp: 2^-4 relative for normal codes, 2^-10 absolute (in code
    # units) for subnormal ones, plus the fp32 rounding of the scaled value
    bound = 2.0 ** -4 * np.abs(r) + 2.0 ** -10 * srow + 1e-6 * np.abs(r)
    assert np.all(np.abs(deq - r) <= bound)
    # and the codes are the nearest: one code step further is never closer
    q = wl.random_bf16((100, 3, 128), 1.0, 14)
    qc, qs = orc.quantize_queries(q)
    dq = orc.e4m3_decode(qc) * qs.T[:, :, None]
    assert np.all(np.abs(dq - q) <= 2.0 ** -4 * np.abs(q) + 2.0 ** -10 * qs.T[:, :, None] + 1e-7)


def test_smoothing_reduces_error_for_biased_keys():
    """Keys with a common bias 20x their spread: smoothing by the key mean
    recovers the plain attention far better than no smoothing."""
    nh, d, nq = 2, 64, 64
    scale = 1.0 / np.sqrt(d)
    q = wl.random_bf16((nq, nh, d), 1.0, 20)
    bias = 20.0 * wl.random_bf16((1, nh, d), 1.0, 21)
    ks = orc.bf16_round(wl.random_bf16((32, nh, d), 1.0, 22) + bias)
    kc = orc.bf16_round(wl.random_bf16((96, nh, d), 1.0, 23) + bias)
    kh = orc.bf16_round(wl.random_bf16((256, nh, d), 1.0, 24) + bias)
    vs, vc, vh = (wl.random_bf16((n, nh, d), 1.0, 30 + n) for n in (32, 96, 256))
    ref = orc.decomposable_attention(q, ks, vs, kc, vc, kh, vh, scale)
    mu = orc.bf16_round(orc.key_mean(ks, kc, kh))
    err = {}
    for name, m in (("none", None), ("mean", mu)):
        got = orc.decomposable_attention_fp8(q, ks, vs, kc, vc, kh, vh, scale, m)
        err[name] = np.linalg.norm(got["o_full"] - ref["o_full"]) / np.linalg.norm(ref["o_full"])
        assert np.max(np.abs(got["lse_full"] - ref["lse_full"])) < 2.0
    assert err["mean"] < 0.2 * err["none"]
    assert err["mean"] < 0.05


def test_key_mean_is_the_mean():
    a = wl.random_bf16((10, 2, 8), 1.0, 30)
    b = wl.random_bf16((5, 2, 8), 1.0, 31)
    m = orc.key_mean(a, b[:0], b)
    np.testing.assert_allclose(m * 15, a.sum(0) + b.sum(0), rtol=1e-13)

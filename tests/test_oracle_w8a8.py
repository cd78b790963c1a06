"""Pins of the oracle's W8A8 projection pieces (ISPA paper §4.4: 8-bit
weights and activations for the linear layers; OCP 8-bit floating point
E4M3, the "fn" variant).

The E4M3 decoding and encoding are checked against torch's own float8_e4m3fn
conversion (an independent implementation of the same format) over every
code and over random values inside the format's range, plus the rounding
cases by hand; quantization and the projection against brute force.
"""
import numpy as np
import torch

import oracle.ispa_oracle as orc


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2      # 0x7F, 0xFF
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * np.exp(rng.uniform(-12, 5, 20000)),
                        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.e4m3_encode(x.astype(np.float64)), ref)


def test_encode_rounding_cases():
    cases = {
        1.0 + 1 / 16: 0x38,           # halfway 1.0 / 1.125 -> even mantissa 0
        1.0 + 3 / 16: 0x3A,           # halfway 1.125 / 1.25 -> even mantissa 2
        1.0 + 1 / 16 + 1e-9: 0x39,    # just above halfway
        2.0 ** -10: 0x00,             # half the smallest subnormal -> 0 (even)
        3 * 2.0 ** -11: 0x01,         # 0.75 of the smallest subnormal -> it
        464.0: 0x7E,                  # beyond the largest finite value: saturates
        1e6: 0x7E,
        -1e6: 0xFE,
        -0.0: 0x80,
    }
    for v, c in cases.items():
        assert int(orc.e4m3_encode(np.array([v]))[0]) == c, (v, c)


def test_quantize_rows():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((5, 33)).astype(np.float32)
    a[2] = 0.0
    codes, scale = orc.quantize_rows(a)
    assert scale.dtype == np.float32 and scale[2] == 0 and np.all(codes[2] == 0)
    for r in (0, 1, 3, 4):
        k = int(np.argmax(np.abs(a[r])))
        assert codes[r, k] & 0x7F == 0x7E                 # the absmax lands on 448
        assert scale[r] == np.float32(np.max(np.abs(a[r])) / np.float32(448))
        # every dequantized value is within half a quantum (E4M3 has 3
        # mantissa bits: relative 2^-4) of the scaled input, or of a
        # subnormal quantum
        deq = orc.e4m3_decode(codes[r]) * scale[r]
        err = np.abs(deq - a[r])
        bound = np.maximum(2.0 ** -4 * np.abs(a[r]), 2.0 ** -10 * scale[r]) * (1 + 1e-6)
        assert np.all(err <= bound)


def test_project_w8a8_brute():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 16)).astype(np.float32)
    w = rng.standard_normal((4, 16)).astype(np.float32)
    wq, ws = orc.quantize_rows(w)
    y = orc.project_w8a8(x, wq, ws)
    xq, xs = orc.quantize_rows(x)
    for m in range(3):
        for o in range(4):
            acc = sum(float(orc.e4m3_decode(xq[m, k])) * float(orc.e4m3_decode(wq[o, k]))
                      for k in range(16))
            assert abs(y[m, o] - acc * float(xs[m]) * float(ws[o])) <= 1e-12 * max(1, abs(acc))

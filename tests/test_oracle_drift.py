"""Pins of the oracle's drift score (event-triggered recalibration, ISPA
paper §3.3 last paragraph; the pages give no trigger, so the score is a
reading of them).

The score is the mean leverage x (G + lam I)^{-1} x^T of a chunk's local
outputs over its warmup expectation tr((G + lam I)^{-1} G) / N. Pinned by
identities that do not retype it: over the warmup tokens themselves the mean
leverage is exactly the expectation (score 1); a token orthogonal to every
warmup token has leverage |x|^2 / lam; the score is quadratic in x; and a
2 x 2 case by hand.
"""
import numpy as np

import oracle.ispa_oracle as orc


def test_warmup_tokens_score_one():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 40)) @ rng.standard_normal((40, 40))
    g = x.T @ x
    assert abs(orc.drift_score(x, g, 0.3, 300) - 1.0) < 1e-12


def test_orthogonal_token_leverage():
    """Warmup tokens span the first 5 coordinates; a probe on coordinate 7
    sees only lam: leverage |x|^2 / lam, and the reference is the warmup's
    sum of s / (s + lam) over its nonzero eigenvalues s, over N."""
    rng = np.random.default_rng(2)
    h, n, lam = 12, 50, 0.5
    x = np.zeros((n, h))
    x[:, :5] = rng.standard_normal((n, 5))
    g = x.T @ x
    s = np.linalg.eigvalsh(g[:5, :5])
    ref = float(np.sum(s / (s + lam)) / n)
    assert abs(orc.drift_reference(g, lam, n) - ref) < 1e-12
    probe = np.zeros((1, h))
    probe[0, 7] = 3.0
    assert abs(orc.drift_score(probe, g, lam, n) - (9.0 / lam) / ref) < 1e-9


def test_quadratic_in_x():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((80, 10))
    g = x.T @ x
    probe = rng.standard_normal((7, 10))
    s1 = orc.drift_score(probe, g, 0.1, 80)
    s3 = orc.drift_score(3.0 * probe, g, 0.1, 80)
    assert abs(s3 - 9.0 * s1) < 1e-9 * s3


def test_hand_case():
    """G = diag(4, 1), lam = 1, N = 2: (G + I)^{-1} = diag(1/5, 1/2),
    tr((G + I)^{-1} G) = 4/5 + 1/2 = 1.3, reference 0.65; the probe (1, 1)
    has leverage 1/5 + 1/2 = 0.7, score 0.7 / 0.65."""
    g = np.diag([4.0, 1.0])
    assert abs(orc.drift_reference(g, 1.0, 2) - 0.65) < 1e-15
    assert abs(orc.drift_score(np.array([[1.0, 1.0]]), g, 1.0, 2) - 0.7 / 0.65) < 1e-14


def test_shift_raises_score():
    """Tokens from a rotated distribution (new directions) score far above
    tokens from the warmup distribution."""
    rng = np.random.default_rng(4)
    h = 32
    basis = rng.standard_normal((8, h))
    warm = rng.standard_normal((400, 8)) @ basis + 0.05 * rng.standard_normal((400, h))
    g = warm.T @ warm
    same = rng.standard_normal((64, 8)) @ basis + 0.05 * rng.standard_normal((64, h))
    other = rng.standard_normal((64, 8)) @ rng.standard_normal((8, h))
    s_same = orc.drift_score(same, g, 1e-2, 400)
    s_other = orc.drift_score(other, g, 1e-2, 400)
    assert 0.5 < s_same < 2.0
    assert s_other > 20.0 * s_same

"""Pins of the oracle's unclipped four-channel kernel (SANATAN reading notes §2.5: Phi_4 = [1, r, r cos, r sin]
per dim, one dim contributing 1 + r_q r_k (1 + cos dtheta)), independent of the GPU path.

- Hard roots, as the notes print them: matched labels give 2 + cos dtheta per dim, mismatched ones -cos dtheta.
- Dropping the cos and sin channels removes exactly sum_a cos dtheta_a from the six-channel kernel.
- The direct quadratic form on the four-channel kernel equals the normalised sum built pair by pair from kappa4.
"""
import math

import numpy as np
import pytest

import oracle


def theta(u):
    return math.pi * u / (1 + abs(u))


@pytest.mark.parametrize("match", [True, False])
def test_hard_roots_match_the_printed_values(match):
    """d = 1, gamma huge: the label is the sign of cos(theta + omega) - sin(theta + omega)."""
    gamma, om = 1e6, np.array([0.0])
    uq, uk = 0.3, (-0.1 if match else 2.5)  # theta: 0.72 and -0.29 (cos > sin, label +1) or 2.24 (label -1)
    lq = np.sign(math.cos(theta(uq)) - math.sin(theta(uq)))
    lk = np.sign(math.cos(theta(uk)) - math.sin(theta(uk)))
    assert (lq == lk) == match
    for t, s in [(0, 0), (5, 2)]:
        dth = theta(uq) - theta(uk) + (t - s) * 1.0  # lambda_0 = 1
        want = 2 + math.cos(dth) if match else -math.cos(dth)
        got = oracle.kappa4(np.array([uq]), np.array([uk]), t, s, om, gamma=gamma)
        assert got == pytest.approx(want, abs=1e-12)


def test_dropping_cos_sin_channels_removes_sum_cos():
    rng = np.random.default_rng(31)
    d = 64
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    om = rng.uniform(-math.pi, math.pi, d)
    for t, s in [(0, 0), (9, 3), (1000, 17)]:
        lam = 10000.0 ** (-np.arange(d) / d)
        sum_cos = sum(math.cos(theta(q[a]) - theta(k[a]) + (t - s) * lam[a]) for a in range(d))
        k6 = oracle.kappa(q, k, t, s, om)
        k4 = oracle.kappa4(q, k, t, s, om)
        assert k6 - k4 == pytest.approx(sum_cos, abs=1e-9)


@pytest.mark.parametrize("p", [1, 2])
def test_direct_form_equals_pairwise_sum(p):
    rng = np.random.default_rng(32 + p)
    T, d, dv = 7, 64, 5
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-math.pi, math.pi, d)
    c, eps = 4.0 * d, 1e-6
    got = oracle.attention_direct(q, k, v, om, p=p, four_channel=True)
    for t in range(T):
        w = np.array([(oracle.kappa4(q[t], k[s], t, s, om) / c) ** p for s in range(t + 1)])
        want = (w[:, None] * v[:t + 1]).sum(0) / (w.sum() + eps)
        np.testing.assert_allclose(got[t], want, rtol=1e-12, atol=1e-12)
    # and the six-channel default is untouched by the flag
    np.testing.assert_array_equal(oracle.attention_direct(q, k, v, om, p=p),
                                  oracle.attention_direct(q, k, v, om, p=p, four_channel=False))

"""Pins of the oracle's spectral-harmonic kernel (CPU only).

Reading of the notes' Appendix B outlook (harmonics cos(n theta), sin(n theta) added per dim; at p = 1 the map
stays explicit and the state grows with the harmonic count): harmonics n = 1..nh of the rotated angle, each
gated by the root label, so kappa_h = sum_a (1 + r_q r_k)(1 + sum_n cos(n x_a)).  The pins do not re-type that
formula:
  * nh = 1 is the six-channel kernel (features, kappa and the attention output against the six-channel code);
  * the factorisation <Phi_h(q), Phi_h(k)> = kappa_h, the identity the outlook relies on;
  * the recurrent form equals the direct form (p = 1 stays an exact recurrence);
  * the angular factor against the textbook Dirichlet closed form 1 + sum_{n<=N} cos(n x) =
    1/2 + sin((N + 1/2) x) / (2 sin(x / 2));
  * special values: all-matched hard roots at zero difference give 2 d (1 + nh); gamma = 0 gives r = 0;
  * the kernel can be negative for nh >= 2 (documented, not clipped); position shifts leave outputs unchanged.
"""
import math

import numpy as np
import pytest

import oracle

PI = math.pi


def _inputs(seed, T, d, dv=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv)),
            rng.uniform(-PI, PI, d))


def test_one_harmonic_is_the_six_channel_kernel():
    q, k, v, om = _inputs(1, 12, 5)
    np.testing.assert_array_equal(oracle.features_h(q, 7, om, 1), oracle.features(q, 7, om))
    for t, s in ((3, 0), (11, 11), (9, 4)):
        assert oracle.kappa_h(q[t], k[s], t, s, om, 1) == pytest.approx(oracle.kappa(q[t], k[s], t, s, om),
                                                                         rel=1e-14)
    np.testing.assert_allclose(oracle.attention_direct_h(q, k, v, om, 1), oracle.attention_direct(q, k, v, om),
                               rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("nh", [2, 3, 5])
def test_factorisation_identity(nh):
    q, k, _, om = _inputs(2 + nh, 10, 6)
    fq = oracle.features_h(q, 100, om, nh)
    fk = oracle.features_h(k, 100, om, nh)
    assert fq.shape == (10, (2 + 4 * nh) * 6)
    for t in range(10):
        for s in range(10):
            kap = oracle.kappa_h(q[t], k[s], 100 + t, 100 + s, om, nh)
            assert float(fq[t] @ fk[s]) == pytest.approx(kap, rel=1e-12, abs=1e-12 * 6 * (1 + nh))


@pytest.mark.parametrize("nh,d", [(2, 1), (2, 4), (3, 3)])
def test_recurrent_equals_direct(nh, d):
    q, k, v, om = _inputs(10 + nh + d, 14, d)
    want = oracle.attention_direct_h(q, k, v, om, nh, c=2.0 * d * (1 + nh))
    got, S, z = oracle.recurrent_h(q, k, v, om, nh, c=2.0 * d * (1 + nh))
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)
    # the state is sum Phi_h(k_s) v_s^T and sum Phi_h(k_s)
    fk = oracle.features_h(k, 0, om, nh)
    np.testing.assert_allclose(S, fk.T @ v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, fk.sum(0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nh", [1, 2, 4, 7])
def test_angular_factor_matches_dirichlet_closed_form(nh):
    """gamma = 0 (r = 0) and d = 1: kappa_h = 1 + sum_{n<=nh} cos(n x), with x = theta_q - theta_k + (t - s)."""
    for uq, uk, dt in ((0.3, -1.1, 0), (2.0, 0.5, 3), (-0.7, 0.9, 7), (1.5, 1.5, 1)):
        thq, thk = PI * uq / (1 + abs(uq)), PI * uk / (1 + abs(uk))
        x = thq - thk + dt * 1.0  # d = 1: lambda_0 = 1
        closed = 0.5 + math.sin((nh + 0.5) * x) / (2 * math.sin(x / 2))
        got = oracle.kappa_h([uq], [uk], dt, 0, [0.4], nh, gamma=0.0)
        assert got == pytest.approx(closed, rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("nh", [1, 2, 3])
def test_hard_roots_matched_at_zero_difference(nh):
    """Hard roots (|r| -> 1) and q = k at s = t: every label matches itself (r_q r_k = r^2 = 1) and x = 0, so
    every dim gives 2 (1 + nh)."""
    d = 8
    q = np.linspace(0.2, 2.0, d)
    om = np.full(d, -PI / 4 - 0.3)
    r = [oracle.root(u, w, 1e4) for u, w in zip(q, om)]
    assert all(abs(abs(x) - 1) < 1e-12 for x in r)
    assert oracle.kappa_h(q, q, 5, 5, om, nh, gamma=1e4) == pytest.approx(2 * d * (1 + nh), rel=1e-12)


def test_gamma_zero():
    """r = 0: kappa_h = d + sum_a sum_n cos(n x_a); at q = k, s = t it is d (1 + nh)."""
    q, k, _, om = _inputs(30, 4, 6)
    for nh in (2, 3):
        assert oracle.kappa_h(q[1], q[1], 2, 2, om, nh, gamma=0.0) == pytest.approx(6 * (1 + nh), rel=1e-13)


def test_kernel_can_be_negative_for_two_harmonics():
    """1 + cos x + cos 2x < 0 near x = 2: with gamma = 0 and d = 1 the kernel is negative (no clipping)."""
    uq = 0.0
    # x = theta_q - theta_k + (t - s) lambda_0 = 2 with theta_k = 0 and t - s = 2
    assert oracle.kappa_h([uq], [0.0], 2, 0, [0.1], 2, gamma=0.0) < 0
    assert oracle.kappa_h([uq], [0.0], 2, 0, [0.1], 1, gamma=0.0) > 0


def test_position_shift_leaves_recurrent_outputs():
    q, k, v, om = _inputs(40, 16, 4)
    a, _, _ = oracle.recurrent_h(q, k, v, om, 2, pos0=0)
    b, _, _ = oracle.recurrent_h(q, k, v, om, 2, pos0=12345)
    np.testing.assert_allclose(b, a, rtol=1e-9, atol=1e-10)

"""Pins of the oracle's gradient of the direct form (CPU only).

The gradient is needed because omega is learned and the method is trained (SANATAN reading notes §2.2
root equation; §4.1 two-stage training).  None of these re-types the oracle's chain rule:
  * central finite differences of the oracle's forward direct form (an independent route: it calls only the
    forward), for every coordinate of q, k, v and omega, at p = 1 and p = 2;
  * exact identities: with eps = 0 every output row is a convex combination of the values, so the value
    gradients sum to the output gradients, and shifting every value by one vector leaves the q, k and omega
    gradients unchanged; a single token with eps = 0 outputs its own value;
  * symmetries of the method: omega -> omega + pi negates every root label and leaves kappa unchanged
    (§2.2), so the q, k, v and omega gradients are unchanged; gamma = 0 makes r = 0, so omega has no effect.
"""
import math

import numpy as np
import pytest

import oracle


def _inputs(seed, T, d, dv, away_from_zero=1e-3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    # the angle map is only C^1 at u = 0: keep the finite-difference steps away from that kink
    q[np.abs(q) < away_from_zero] += 0.01
    k[np.abs(k) < away_from_zero] += 0.01
    v = rng.standard_normal((T, dv))
    g = rng.standard_normal((T, dv))
    om = rng.uniform(-math.pi, math.pi, d)
    return q, k, v, g, om


def _loss(q, k, v, g, om, **kw):
    return float((oracle.attention_direct(q, k, v, om, **kw) * g).sum())


@pytest.mark.parametrize("p", [1, 2])
@pytest.mark.parametrize("gamma,eps", [(4.0, 1e-6), (1.5, 0.05)])
def test_gradient_matches_central_differences(p, gamma, eps):
    T, d, dv = 9, 4, 3
    q, k, v, g, om = _inputs(100 + p, T, d, dv)
    kw = dict(p=p, gamma=gamma, eps=eps, c=4.0 * d)
    dq, dk, dvv, dom = oracle.attention_direct_grad(q, k, v, g, om, **kw)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dvv), ("omega", om, dom)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v, "omega": om}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], g, args["omega"], **kw)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], g, args["omega"], **kw)
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(np.abs(fd).max(), 1e-3)
        assert np.abs(grad - fd).max() <= 2e-6 * scale, (name, np.abs(grad - fd).max(), scale)


@pytest.mark.parametrize("p", [1, 2])
def test_value_gradients_sum_to_output_gradients(p):
    """eps = 0: o_t is a convex combination of v_s, so sum_s dL/dv_s = sum_t g_t exactly."""
    q, k, v, g, om = _inputs(7, 40, 8, 5)
    _, _, dvv, _ = oracle.attention_direct_grad(q, k, v, g, om, p=p, eps=0.0)
    np.testing.assert_allclose(dvv.sum(0), g.sum(0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("p", [1, 2])
def test_value_shift_leaves_other_gradients(p):
    """eps = 0: v -> v + b shifts every output by b, so the q, k, omega gradients do not change."""
    q, k, v, g, om = _inputs(8, 30, 6, 4)
    b = np.array([0.7, -1.3, 2.0, 0.25])
    a = oracle.attention_direct_grad(q, k, v, g, om, p=p, eps=0.0)
    s = oracle.attention_direct_grad(q, k, v + b, g, om, p=p, eps=0.0)
    for x, y in zip(a[:2] + a[3:], s[:2] + s[3:]):
        np.testing.assert_allclose(y, x, rtol=1e-9, atol=1e-11)


def test_single_token_without_eps():
    """T = 1, eps = 0: o_0 = v_0, so dv = g and the other gradients vanish."""
    q, k, v, g, om = _inputs(9, 1, 5, 3)
    dq, dk, dvv, dom = oracle.attention_direct_grad(q, k, v, g, om, eps=0.0)
    np.testing.assert_allclose(dvv, g, rtol=1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15 and np.abs(dom).max() < 1e-15


@pytest.mark.parametrize("p", [1, 2])
def test_omega_plus_pi_symmetry(p):
    """omega -> omega + pi negates every r (cos and sin both change sign) and leaves kappa unchanged."""
    q, k, v, g, om = _inputs(10, 25, 6, 4)
    a = oracle.attention_direct_grad(q, k, v, g, om, p=p)
    b = oracle.attention_direct_grad(q, k, v, g, om + math.pi, p=p)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=1e-9, atol=1e-12)


def test_gamma_zero_omega_gradient_vanishes():
    """gamma = 0 gives r = 0 for every component: omega does not enter the output."""
    q, k, v, g, om = _inputs(11, 20, 5, 3)
    _, _, _, dom = oracle.attention_direct_grad(q, k, v, g, om, gamma=0.0)
    assert np.abs(dom).max() == 0.0

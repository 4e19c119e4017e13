"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks a special value, closed form,
invariant, bound, or an independent computation route (brute force / tensor powers / the
feature-map factorisation) -- so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))
PI = math.pi


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- angle / root / frequency
def test_angle_special_points():
    # phi(u) = pi u / (1+|u|)  (reading notes §2.2): 0 -> 0, +-1 -> +-pi/2, 3 -> 3pi/4, |u|->inf -> pi
    assert oracle.angle(0.0) == 0.0
    assert oracle.angle(1.0) == pytest.approx(PI / 2, abs=1e-15)
    assert oracle.angle(-1.0) == pytest.approx(-PI / 2, abs=1e-15)
    assert oracle.angle(3.0) == pytest.approx(3 * PI / 4, abs=1e-15)
    assert oracle.angle(1e12) == pytest.approx(PI, abs=1e-9)
    assert abs(oracle.angle(1e12)) < PI


def test_root_at_omega_pi_over_4_closed_form():
    # reading notes §2.2: omega = pi/4 gives coefficient -sqrt(2) sin(theta); root sign opposite to theta's.
    g = 3.0
    for u in (-2.5, -0.3, 0.2, 0.9, 7.0):
        th = PI * u / (1 + abs(u))
        assert oracle.root(u, PI / 4, g) == pytest.approx(math.tanh(-math.sqrt(2) * g * math.sin(th)), abs=1e-14)
        assert np.sign(oracle.root(u, PI / 4, g)) == -np.sign(u)


def test_root_at_omega_zero_and_sign_convention():
    # omega = 0: r = tanh(gamma (cos th - sin th)); u = 1 -> th = pi/2 -> tanh(-gamma) (minus, not plus, sin)
    assert oracle.root(1.0, 0.0, 2.0) == pytest.approx(math.tanh(-2.0), abs=1e-15)
    assert oracle.root(0.0, 0.0, 2.0) == pytest.approx(math.tanh(2.0), abs=1e-15)
    assert oracle.root(-1.0, 0.0, 2.0) == pytest.approx(math.tanh(2.0), abs=1e-15)


def test_frequency_ladder():
    assert oracle.freq(0, 64) == 1.0
    assert oracle.freq(32, 64) == pytest.approx(0.01, rel=1e-14)
    assert oracle.freq(63, 64) == pytest.approx(10000 ** (-63 / 64), rel=1e-14)
    f = [oracle.freq(a, 64) for a in range(64)]
    assert all(f[i] > f[i + 1] for i in range(63))


# ---------------------------------------------------------------- factorisation identity (P1)
@pytest.mark.parametrize("d", [1, 3, 64])
def test_feature_inner_product_equals_kappa(d):
    # reading notes §2.3: <Phi_a(q), Phi_a(k)> = (1 + r_q r_k)(1 + cos dtheta_a), summed over a
    rng = _rng(10 + d)
    om = rng.uniform(-PI, PI, d)
    for trial in range(20):
        q = rng.standard_normal(d) * 2
        k = rng.standard_normal(d) * 2
        t = int(rng.integers(0, 40000))
        s = int(rng.integers(0, t + 1))
        fq = oracle.features(q[None], t, om)[0]
        fk = oracle.features(k[None], s, om)[0]
        kap = oracle.kappa(q, k, t, s, om)
        assert abs(float(fq @ fk) - kap) <= 1e-12 * 4 * d


def test_feature_layout_channel_major():
    d = 4
    om = np.array([0.1, -0.5, 1.0, 2.0])
    u = np.array([[0.0, 1.0, -1.0, 3.0]])
    f = oracle.features(u, 0, om, gamma=2.0).reshape(6, d)
    assert np.all(f[0] == 1.0)
    th = np.array([0, PI / 2, -PI / 2, 3 * PI / 4])
    np.testing.assert_allclose(f[1], np.cos(th), atol=1e-15)
    np.testing.assert_allclose(f[2], np.sin(th), atol=1e-15)
    r = np.tanh(2.0 * (np.cos(th + om) - np.sin(th + om)))
    np.testing.assert_allclose(f[3], r, atol=1e-15)
    np.testing.assert_allclose(f[4], r * np.cos(th), atol=1e-15)
    np.testing.assert_allclose(f[5], r * np.sin(th), atol=1e-15)


def test_rotation_direction_hand_case():
    # d=1, u_q=1 (theta=pi/2), u_k=0, omega=0, t-s=1, lambda_0=1:
    # dtheta_rot = pi/2 - 0 + 1 -> cos = -sin(1);  gate = 1 + tanh(-g) tanh(g)
    g = 1.5
    kap = oracle.kappa([1.0], [0.0], 1, 0, [0.0], gamma=g)
    assert kap == pytest.approx((1 - math.tanh(g) ** 2) * (1 - math.sin(1.0)), abs=1e-15)


# ---------------------------------------------------------------- bounds and gates (P2, P3)
def test_kappa_bounds_random():
    rng = _rng(2)
    d = 64
    om = rng.uniform(-PI, PI, d)
    ub = GOLD["score_upper_bound_per_dim"]["value"] * d
    for _ in range(200):
        q, k = rng.standard_normal(d) * 3, rng.standard_normal(d) * 3
        t = int(rng.integers(0, 5000))
        s = int(rng.integers(0, t + 1))
        kap = oracle.kappa(q, k, t, s, om)
        assert 0.0 <= kap <= ub


def test_hard_roots_gate_values():
    # Huge gamma saturates tanh to exactly +-1 in fp64: the per-dim gate is exactly 0 or 2.
    g = 1e6
    om = PI / 4  # r = sign opposite to theta
    for uq in (-2.0, -0.5, 0.5, 2.0):
        for uk in (-3.0, -0.1, 0.1, 3.0):
            gate = 1 + oracle.root(uq, om, g) * oracle.root(uk, om, g)
            assert gate in GOLD["hard_gate_values"]["value"]


def test_hard_roots_all_mismatched_and_all_matched():
    g = 1e6
    d = 64
    rng = _rng(3)
    om = np.full(d, PI / 4)
    q = np.abs(rng.standard_normal(d)) + 0.1   # theta > 0 -> r = -1
    k = -(np.abs(rng.standard_normal(d)) + 0.1)  # theta < 0 -> r = +1
    assert oracle.kappa(q, k, 7, 3, om, gamma=g) == 0.0
    # all matched with zero rotated difference (q = k at the same position): 4d
    assert oracle.kappa(q, q, 5, 5, om, gamma=g) == pytest.approx(4 * d, abs=1e-12)
    # m matched dims: kappa in [0, 4m]
    for m in (1, 10, 40):
        kk = k.copy()
        kk[:m] = np.abs(kk[:m])
        kap = oracle.kappa(q, kk, 9, 2, om, gamma=g)
        lo, hi = GOLD["matched_dims_range_per_dim"]["value"]
        assert lo * m <= kap <= hi * m + 1e-12


def test_label_flip_invariance():
    # reading notes §2.2: swapping all labels (omega -> omega + pi negates r) leaves r_q r_k unchanged
    rng = _rng(4)
    d = 16
    om = rng.uniform(-PI, PI, d)
    for _ in range(10):
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        assert oracle.kappa(q, k, 11, 4, om + PI) == pytest.approx(oracle.kappa(q, k, 11, 4, om), abs=1e-12)
        assert oracle.root(q[0], om[0] + PI) == pytest.approx(-oracle.root(q[0], om[0]), abs=1e-14)


def test_gamma_zero_is_three_channel_kernel():
    # gamma = 0 -> r = 0 -> kappa = d + sum_a cos(dtheta_a)  (reading notes §4.4, s3 in [0, 2d])
    rng = _rng(5)
    d = 8
    om = rng.uniform(-PI, PI, d)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    t, s = 9, 3
    th = lambda u: PI * u / (1 + np.abs(u))
    lam = 10000.0 ** (-np.arange(d) / d)
    want = d + np.sum(np.cos(th(q) - th(k) + (t - s) * lam))
    kap = oracle.kappa(q, k, t, s, om, gamma=0.0)
    assert kap == pytest.approx(want, abs=1e-13)
    lo, hi = GOLD["three_channel_range_per_dim"]["value"]
    assert lo * d <= kap <= hi * d


def test_relative_position_invariance_of_features():
    # Only t - s enters the kernel (reading notes §2.2): shift both positions by a large offset.
    rng = _rng(6)
    d = 64
    om = rng.uniform(-PI, PI, d)
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    base = float(oracle.features(q, 12, om)[0] @ oracle.features(k, 5, om)[0])
    shifted = float(oracle.features(q, 10**6 + 12, om)[0] @ oracle.features(k, 10**6 + 5, om)[0])
    assert shifted == pytest.approx(base, abs=1e-8)


# ---------------------------------------------------------------- attention forms (P4-P8, P12, P13)
@pytest.mark.parametrize("d,dv,T", [(1, 5, 9), (2, 3, 16), (3, 7, 12), (64, 64, 16)])
def test_quadratic_equals_recurrent_p1(d, dv, T):
    rng = _rng(100 + d)
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-PI, PI, d)
    a = oracle.attention_direct(q, k, v, om, pos0=3)
    b, S, z = oracle.recurrent(q, k, v, om, pos0=3)
    # Rounding bound: both forms sum |terms| of size |Phi_q||Phi_k||v| over s <= t, divided by
    # the denominator sum_s kappa (which can be small at tiny d when gates mismatch).
    Fq, Fk = oracle.features(q, 3, om), oracle.features(k, 3, om)
    absk = np.abs(Fq) @ np.abs(Fk).T                       # [t, s] sum_f |Phi_q,f Phi_k,f|
    den = np.tril(Fq @ Fk.T).sum(1)                          # sum_{s<=t} kappa
    scale = (np.tril(absk) @ np.abs(v)).max(1) / den + np.abs(a).max(1) * np.tril(absk).sum(1) / den
    assert np.all(np.abs(a - b).max(1) <= 64 * 2.3e-16 * scale)


def test_recurrent_resume_equals_direct_on_concatenation():
    rng = _rng(7)
    d, dv, T1, T2 = 4, 6, 7, 9
    q, k, v = rng.standard_normal((T1 + T2, d)), rng.standard_normal((T1 + T2, d)), rng.standard_normal((T1 + T2, dv))
    om = rng.uniform(-PI, PI, d)
    _, S, z = oracle.recurrent(q[:T1], k[:T1], v[:T1], om, pos0=20)
    b, _, _ = oracle.recurrent(q[T1:], k[T1:], v[T1:], om, pos0=20 + T1, S=S, z=z)
    a = oracle.attention_direct(q, k, v, om, pos0=20)
    assert np.max(np.abs(a[T1:] - b)) <= 1e-12


def test_recurrent_state_is_sum_of_outer_products():
    # The state after T tokens is sum_s Phi(k_s) v_s^T and sum_s Phi(k_s) (reading notes §2.7).
    rng = _rng(8)
    d, dv, T = 3, 4, 10
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-PI, PI, d)
    _, S, z = oracle.recurrent(q, k, v, om, pos0=0)
    F = oracle.features(k, 0, om)
    np.testing.assert_allclose(S, F.T @ v, atol=1e-12)
    np.testing.assert_allclose(z, F.sum(0), atol=1e-12)


def test_first_row_and_epsilon():
    rng = _rng(9)
    d, dv, T = 64, 8, 5
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-PI, PI, d)
    o = oracle.attention_direct(q, k, v, om, eps=0.0)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-14, atol=1e-15)
    eps = 0.05
    o = oracle.attention_direct(q, k, v, om, eps=eps)
    w = oracle.kappa(q[0], k[0], 0, 0, om) / (4 * d)
    np.testing.assert_allclose(o[0], v[0] * w / (w + eps), rtol=1e-13)


@pytest.mark.parametrize("p", [1, 2])
def test_convex_hull_and_constant_values(p):
    rng = _rng(11 + p)
    d, dv, T = 16, 5, 30
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-PI, PI, d)
    o = oracle.attention_direct(q, k, v, om, eps=0.0, p=p)
    for t in range(T):
        assert np.all(o[t] >= v[: t + 1].min(0) - 1e-12) and np.all(o[t] <= v[: t + 1].max(0) + 1e-12)
    vc = np.tile(np.array([[1.5, -2.0, 0.25, 3.0, -0.5]]), (T, 1))
    o = oracle.attention_direct(q, k, vc, om, eps=0.0, p=p)
    np.testing.assert_allclose(o, vc, rtol=1e-13)


def test_position_shift_recurrent():
    # The recurrent form uses absolute positions; shifting pos0 by 1e6 must not change outputs.
    rng = _rng(12)
    d, dv, T = 64, 8, 12
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-PI, PI, d)
    a, _, _ = oracle.recurrent(q, k, v, om, pos0=0)
    b, _, _ = oracle.recurrent(q, k, v, om, pos0=10**6)
    assert np.max(np.abs(a - b)) <= 1e-8


def test_hand_case_d1_zero_inputs():
    # d=1, q=k=0 (theta=0), T=2: kappa_00 = kappa_11 = 2(1+r^2), kappa_10 = (1+r^2)(1+cos 1),
    # with r = tanh(gamma (cos omega - sin omega)).  c = 4d = 4.
    g, om, eps = 2.5, 0.7, 1e-3
    r = math.tanh(g * (math.cos(om) - math.sin(om)))
    k11 = 2 * (1 + r * r)
    k10 = (1 + r * r) * (1 + math.cos(1.0))
    v = np.array([[2.0], [-1.0]])
    o = oracle.attention_direct(np.zeros((2, 1)), np.zeros((2, 1)), v, [om], gamma=g, eps=eps)
    c = 4.0
    assert o[0, 0] == pytest.approx(2.0 * (k11 / c) / (k11 / c + eps), rel=1e-14)
    assert o[1, 0] == pytest.approx((k10 * 2.0 + k11 * -1.0) / c / ((k10 + k11) / c + eps), rel=1e-14)


def test_power_ratio_page_example():
    # reading notes §2.6: normalised scores 0.8 vs 0.4 (ratio 2) give weights 2:1, 4:1, 16:1 for p=1,2,4.
    # Build d=1, hard matched roots, key s=1 at the query's own position and angle (kappa = 4),
    # key s=0 one step back with rotated difference pi/2 (kappa = 2).
    g = 1e6
    om = PI / 4
    uq = 0.8
    thq = PI * uq / (1 + uq)
    th0 = thq + 1.0 - PI / 2          # dtheta_rot(t=1, s=0) = thq - th0 + 1 = pi/2
    u0 = th0 / (PI - abs(th0))        # inverse of the angle map
    assert oracle.angle(u0) == pytest.approx(th0, abs=1e-14)
    assert oracle.root(uq, om, g) == oracle.root(u0, om, g)   # matched hard labels
    q = np.array([[uq], [uq]])
    k = np.array([[u0], [uq]])
    v = np.array([[1.0], [0.0]])
    assert oracle.kappa(q[1], k[0], 1, 0, [om], gamma=g) == pytest.approx(2.0, abs=1e-12)
    assert oracle.kappa(q[1], k[1], 1, 1, [om], gamma=g) == pytest.approx(4.0, abs=1e-12)
    ex = GOLD["power_ratio_example"]
    for p, ratio in ex["weight_ratio_by_p"].items():
        o = oracle.attention_direct(q, k, v, [om], gamma=g, eps=0.0, p=int(p))[1, 0]
        # o = w0 / (w0 + w1) with w1/w0 = ratio (the own-position key scores twice as high)
        assert o == pytest.approx(1.0 / (1.0 + ratio), rel=1e-12)


@pytest.mark.parametrize("d", [1, 2])
def test_p2_equals_tensor_power_recurrence(d):
    # reading notes §2.6: kappa^p = <Phi^{(x)p}(q), Phi^{(x)p}(k)>; with p=2 a (6d)^2-feature
    # constant-state recurrence reproduces the normalised quadratic p=2 attention.
    rng = _rng(200 + d)
    T, dv = 11, 3
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-PI, PI, d)
    eps = 1e-3
    c = 4.0 * d
    Fq = oracle.features(q, 0, om)
    Fk = oracle.features(k, 0, om)
    D2 = (6 * d) ** 2
    S2 = np.zeros((D2, dv))
    z2 = np.zeros(D2)
    want = np.empty((T, dv))
    for t in range(T):
        fk2 = np.outer(Fk[t], Fk[t]).ravel() / c ** 2
        S2 += np.outer(fk2, v[t])
        z2 += fk2
        fq2 = np.outer(Fq[t], Fq[t]).ravel()
        want[t] = (fq2 @ S2) / (fq2 @ z2 + eps)
    got = oracle.attention_direct(q, k, v, om, eps=eps, p=2)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_rows_subset_matches_full():
    rng = _rng(13)
    d, dv, T = 8, 4, 40
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv))
    om = rng.uniform(-PI, PI, d)
    full = oracle.attention_direct(q, k, v, om, p=2)
    rows = [0, 7, 39, 13]
    np.testing.assert_array_equal(oracle.attention_direct(q, k, v, om, p=2, rows=rows), full[rows])


def test_recurrent_heads_matches_single_heads():
    rng = _rng(14)
    NH, T, d, dv = 5, 6, 4, 3
    q, k, v = rng.standard_normal((NH, T, d)), rng.standard_normal((NH, T, d)), rng.standard_normal((NH, T, dv))
    om = rng.uniform(-PI, PI, (2, d))
    out, S, z = oracle.recurrent_heads(q, k, v, om, pos0=4)
    for j in range(NH):
        o1, S1, z1 = oracle.recurrent(q[j], k[j], v[j], om[j % 2], pos0=4)
        np.testing.assert_array_equal(out[j], o1)
        np.testing.assert_array_equal(S[j], S1)
        np.testing.assert_array_equal(z[j], z1)


def test_state_size_formula_from_pages():
    d = dv = 64
    per_head = (6 * d * dv + 6 * d) * 4
    assert per_head == GOLD["state_bytes_per_head_d64"]["value"]
    assert 12 * 12 * per_head == GOLD["state_bytes_12layers_12heads_d64"]["value"]

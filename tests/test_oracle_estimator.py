"""Pins of oracle.estimator (latency-estimator fitting, ConfluxServe §6.2 and App. D)
-- CPU only.

The fits are pinned by exact recovery from noiseless data, closed forms (a line
through two points, the intercept-only minimizer), the first-order optimality
condition of the relative-error loss, and recovery of known contention factors.
"""
import random

import numpy as np
import pytest

from oracle import estimator as est


def _rel_loss(a, b, x, t):
    x, t = np.asarray(x, float), np.asarray(t, float)
    return float(np.sum(((a * x + b) / t - 1.0) ** 2))


def test_noiseless_affine_data_is_recovered():
    rnd = random.Random(1)
    for _ in range(50):
        a, b = rnd.uniform(1e-9, 1e-6), rnd.uniform(1e-6, 1e-4)
        x = [rnd.uniform(1, 1e6) for _ in range(rnd.randint(2, 30))]
        t = [a * v + b for v in x]
        ga, gb = est.fit_affine(x, t)
        assert ga == pytest.approx(a, rel=1e-9) and gb == pytest.approx(b, rel=1e-9)


def test_two_points_give_the_line_through_them():
    ga, gb = est.fit_affine([100.0, 300.0], [2.0, 5.0])
    assert ga == pytest.approx(0.015, rel=1e-12) and gb == pytest.approx(0.5, rel=1e-12)


def test_equal_workloads_fit_the_intercept_only():
    t = [2.0, 4.0, 5.0]
    ga, gb = est.fit_affine([7.0, 7.0, 7.0], t)
    # minimizer of sum (b/t - 1)^2: b = sum(1/t) / sum(1/t^2)
    s1 = sum(1 / v for v in t)
    s2 = sum(1 / v ** 2 for v in t)
    assert ga == 0.0 and gb == pytest.approx(s1 / s2, rel=1e-12)
    assert est.fit_affine([], []) == (0.0, 0.0)


def test_fit_minimizes_relative_not_absolute_error():
    rnd = random.Random(2)
    x = [rnd.uniform(10, 1e5) for _ in range(40)]
    t = [(3e-8 * v + 2e-5) * rnd.uniform(0.8, 1.25) for v in x]
    a, b = est.fit_affine(x, t)
    base = _rel_loss(a, b, x, t)
    for da, db in ((1, 0), (-1, 0), (0, 1), (0, -1), (1, 1), (1, -1)):
        assert _rel_loss(a * (1 + 1e-4 * da), b * (1 + 1e-4 * db), x, t) > base
    # an absolute-error fit (ordinary least squares) is a different, worse point here
    A = np.stack([np.asarray(x), np.ones(len(x))], axis=1)
    (oa, ob), *_ = np.linalg.lstsq(A, np.asarray(t), rcond=None)
    assert _rel_loss(oa, ob, x, t) > base


def test_known_contention_factors_are_recovered():
    model = dict(gamma=2e-7, gamma0=3e-5, a_d=1e-9, a_d0=1e-5, a_p=5e-11, a_p0=8e-6, a_comm=0.0, a_comm0=0.0)
    alpha, beta = 1 + 23 / 64, 1 + 40 / 64
    rnd = random.Random(4)
    mixed = []
    for _ in range(60):
        g = rnd.randint(64, 8192)
        d = rnd.choice([-1.0, float(rnd.randint(1000, 2_000_000))])
        p = rnd.choice([-1.0, float(rnd.randint(1000, 50_000_000))])
        tg = model["gamma"] * g + model["gamma0"]
        td = 0.0 if d < 0 else model["a_d"] * d + model["a_d0"]
        tp = 0.0 if p < 0 else model["a_p"] * p + model["a_p0"]
        mixed.append((g, d, p, 0.0, 2 * (tg + max(beta * tp, alpha * td))))
    assert est.fit_contention(model, mixed, 2, 3.0) == (alpha, beta)
    # with no decode anywhere alpha is not identifiable and stays at 1
    only_p = [m for m in mixed if m[1] < 0]
    assert est.fit_contention(model, only_p, 2, 3.0)[0] == 1.0


def test_whole_fit_on_synthetic_profiles():
    rnd = random.Random(5)
    truth = dict(gamma=1.5e-7, gamma0=2.5e-5, a_d=8e-10, a_d0=1.2e-5, a_p=6e-11, a_p0=9e-6, a_comm=0.0,
                 a_comm0=0.0, alpha=1.25, beta=1.5)

    def prof(a, b, lo, hi):
        x = [rnd.uniform(lo, hi) for _ in range(25)]
        return x, [a * v + b for v in x]

    gemm = prof(truth["gamma"], truth["gamma0"], 16, 10000)
    dec = prof(truth["a_d"], truth["a_d0"], 1000, 2e6)
    pre = prof(truth["a_p"], truth["a_p0"], 500, 5e7)
    mixed = []
    for _ in range(40):
        g, d, p = rnd.randint(64, 10000), float(rnd.randint(1000, 2_000_000)), float(rnd.randint(500, 50_000_000))
        tg = truth["gamma"] * g + truth["gamma0"]
        mixed.append((g, d, p, 0.0, tg + max(1.5 * (truth["a_p"] * p + truth["a_p0"]),
                                              1.25 * (truth["a_d"] * d + truth["a_d0"]))))
    m = est.fit_model(gemm, dec, pre, ([], []), mixed, n_layers=1, ab_max=3.0)
    for k in ("gamma", "gamma0", "a_d", "a_d0", "a_p", "a_p0"):
        assert m[k] == pytest.approx(truth[k], rel=1e-9)
    assert (m["alpha"], m["beta"], m["a_comm"], m["a_comm0"]) == (1.25, 1.5, 0.0, 0.0)


def test_mape_closed_form():
    assert est.mape([1.1, 0.9, 2.0], [1.0, 1.0, 2.0]) == pytest.approx((0.1 + 0.1 + 0.0) / 3, rel=1e-12)

"""Fitting the latency estimator from profiles (test infrastructure).

ConfluxServe §6.2 ("Estimator construction") and App. D (Eq. 7-11): every base
function is affine in its workload metric, fitted from isolated profiles; the
contention factors alpha, beta >= 1 of Eq. 4 are calibrated on heterogeneous
iterations.  fp64 NumPy; ``numpy.linalg.lstsq`` is the least-squares step.

Readings of points the pages leave open:

* The pages name no loss; their accuracy figure is a mean absolute percentage error
  (§8.5, Table 4), so each fit minimizes the squared relative error
  sum_i ((a x_i + b) / t_i - 1)^2.  No samples give a = b = 0 (a path that was never
  profiled contributes nothing); samples that all share one x fit the intercept alone.
* alpha and beta are searched exhaustively on the grid 1 + k/64 up to ``ab_max``; on
  equal error the smaller alpha, then the smaller beta, is kept.
"""
from __future__ import annotations

import numpy as np

__all__ = ["fit_affine", "fit_contention", "fit_model", "mape"]


def fit_affine(x, t):
    """(slope, intercept) of t ~ slope * x + intercept, least squares on relative error."""
    x = np.asarray(x, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    if x.size == 0:
        return 0.0, 0.0
    ones = np.ones_like(t)
    if np.all(x == x[0]):
        (b,), *_ = np.linalg.lstsq((1.0 / t)[:, None], ones, rcond=None)
        return 0.0, float(b)
    design = np.stack([x / t, 1.0 / t], axis=1)     # (a x + b) / t = a (x/t) + b (1/t)
    (a, b), *_ = np.linalg.lstsq(design, ones, rcond=None)
    return float(a), float(b)


def _terms(model, gemm_x, decode_x, prefill_x, comm_x):
    """Eq. 3, 5, 6 per iteration under the base functions of ``model`` (a path with no
    work contributes 0)."""
    tg = model["gamma"] * gemm_x + model["gamma0"]
    td = 0.0 if decode_x < 0 else model["a_d"] * decode_x + model["a_d0"]
    tp = 0.0 if prefill_x < 0 else (model["a_comm"] * comm_x + model["a_comm0"]) + \
        (model["a_p"] * prefill_x + model["a_p0"])
    return tg, td, tp


def fit_contention(model, mixed, n_layers, ab_max):
    """(alpha, beta) on the grid minimizing the squared relative error of Eq. 2/4."""
    terms = [_terms(model, g, d, p, c) for g, d, p, c, _ in mixed]
    grid = [1.0 + k / 64.0 for k in range(int(np.floor((ab_max - 1.0) * 64.0 + 1e-9)) + 1)]
    best, pick = np.inf, (1.0, 1.0)
    for alpha in grid:
        for beta in grid:
            err = 0.0
            for (tg, td, tp), (*_, t) in zip(terms, mixed):
                pred = n_layers * (tg + max(beta * tp, alpha * td))
                err += (pred / t - 1.0) ** 2
            if err < best:
                best, pick = err, (alpha, beta)
    return pick


def fit_model(gemm, decode, prefill, comm, mixed, n_layers=1, ab_max=3.0) -> dict:
    """The estimator: ``gemm``/``decode``/``prefill``/``comm`` are (x list, t list) profiles,
    ``mixed`` a list of (gemm_x, decode_x, prefill_x, comm_x, t) iterations."""
    m = {}
    m["gamma"], m["gamma0"] = fit_affine(*gemm)
    m["a_d"], m["a_d0"] = fit_affine(*decode)
    m["a_p"], m["a_p0"] = fit_affine(*prefill)
    m["a_comm"], m["a_comm0"] = fit_affine(*comm)
    m["alpha"], m["beta"] = fit_contention(m, mixed, n_layers, ab_max)
    m["n_layers"] = n_layers
    return m


def mape(pred, meas) -> float:
    """Mean absolute percentage error (§8.5), as a fraction."""
    pred = np.asarray(pred, dtype=np.float64)
    meas = np.asarray(meas, dtype=np.float64)
    return float(np.mean(np.abs(pred - meas) / meas))

"""Pins for the schedule, the Step rate lambda and the temperature (CPU only).

The Step derivation is pinned by transporting exact distributions: one Step
with the exact posterior must move the forward marginal p_t to p_{t-dt}
up to O(dt^2), and iterating Step from pure noise must recover the data law.
"""
import math
import os

import numpy as np
import pytest

from oracle import schedule_terms, step_lambda, temperature, inv_temperature


def _constants(golden_dir):
    out = {}
    with open(os.path.join(golden_dir, "tr_summary_constants.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


@pytest.mark.parametrize("sched", ["linear", "cosine"])
def test_kappa_endpoints_and_monotone(sched):
    assert schedule_terms(0.0, sched)[0] == pytest.approx(1.0, abs=1e-15)
    assert schedule_terms(1.0, sched)[0] == pytest.approx(0.0, abs=1e-15)
    ts = np.linspace(0, 1, 1001)
    k = np.array([schedule_terms(t, sched)[0] for t in ts])
    assert np.all(np.diff(k) <= 1e-15)
    # the rate is -dkappa/dt: compare with a central difference
    for t in [0.1, 0.37, 0.5, 0.9]:
        h = 1e-6
        fd = -(schedule_terms(t + h, sched)[0] - schedule_terms(t - h, sched)[0]) / (2 * h)
        assert schedule_terms(t, sched)[1] == pytest.approx(fd, rel=1e-7)
        kap, _, om = schedule_terms(t, sched)
        assert kap + om == pytest.approx(1.0, abs=1e-15)


def test_lambda_closed_forms():
    for t in [1.0, 0.75, 0.5, 0.2, 0.125]:
        assert step_lambda(t, 0.125, "linear") == pytest.approx(min(1.0, 0.125 / t), rel=1e-14)
    for t in [0.9, 0.5, 0.3]:
        dt = 1 / 12
        want = dt * math.pi / math.tan(math.pi * t / 2)
        assert step_lambda(t, dt, "cosine") == pytest.approx(min(1.0, want), rel=1e-12)
    # cosine: the first step (t = 1) moves no token; the last is clamped to 1
    assert step_lambda(1.0, 1 / 12, "cosine") < 2.0 ** -24
    assert step_lambda(1 / 12, 1 / 12, "cosine") == 1.0
    assert step_lambda(1 / 8, 1 / 8, "linear") == 1.0


def test_temperature_matches_page_constants(golden_dir):
    c = _constants(golden_dir)
    assert temperature(1.0) == pytest.approx(c["tau_max"])
    assert temperature(0.0) == pytest.approx(c["tau_min"])
    assert temperature(0.5) == pytest.approx(0.5 * (c["tau_max"] + c["tau_min"]))
    assert inv_temperature(1.0) == np.float32(1 / 0.8)
    assert inv_temperature(1.0).dtype == np.float32


def _forward_marginal(q, kappa):
    V = q.size
    return kappa * q + (1 - kappa) / V


def _posterior(q, kappa):
    """Exact P(x0 = y | x_t = x) as a [x, y] matrix for the uniform path."""
    V = q.size
    lik = kappa * np.eye(V) + (1 - kappa) / V      # lik[x, y] = P(x_t = x | x0 = y)
    post = lik * q[None, :]
    return post / post.sum(axis=1, keepdims=True)


def _step_kernel(q, t, dt, sched):
    """Transition matrix T[x, y] = (1 - lambda) delta(x, y) + lambda post(y | x)."""
    lam = step_lambda(t, dt, sched)
    kappa = schedule_terms(t, sched)[0]
    V = q.size
    return (1 - lam) * np.eye(V) + lam * _posterior(q, kappa)


@pytest.mark.parametrize("sched", ["linear", "cosine"])
def test_step_transports_forward_marginal_to_second_order(sched):
    q = np.array([0.5, 0.2, 0.15, 0.1, 0.05])
    t = 0.6
    errs = []
    for dt in [0.02, 0.01, 0.005]:
        p_t = _forward_marginal(q, schedule_terms(t, sched)[0])
        p_next = p_t @ _step_kernel(q, t, dt, sched)
        want = _forward_marginal(q, schedule_terms(t - dt, sched)[0])
        errs.append(np.abs(p_next - want).max())
    if sched == "linear":
        # the marginal is linear in t, so the Euler step is exact
        assert max(errs) < 1e-14
    else:
        # local error is O(dt^2): halving dt divides it by about 4
        assert errs[0] / errs[1] == pytest.approx(4.0, rel=0.1)
        assert errs[1] / errs[2] == pytest.approx(4.0, rel=0.1)
        assert errs[2] < 1e-5


def test_reversed_rate_breaks_transport():
    """A plausible slip (lambda built from kappa instead of 1 - kappa) fails at first order."""
    q = np.array([0.5, 0.2, 0.15, 0.1, 0.05])
    t, dt = 0.6, 0.01
    kappa, rate, om = schedule_terms(t, "linear")
    bad = dt * rate / kappa
    from oracle.schedule import step_lambda as good_lambda
    assert abs(bad - good_lambda(t, dt, "linear")) > 1e-3
    V = q.size
    lik = kappa * np.eye(V) + om / V
    post = lik * q[None, :]
    post /= post.sum(axis=1, keepdims=True)
    T = (1 - bad) * np.eye(V) + bad * post
    p_next = _forward_marginal(q, kappa) @ T
    want = _forward_marginal(q, schedule_terms(t - dt, "linear")[0])
    assert np.abs(p_next - want).max() > 1e-4


@pytest.mark.parametrize("sched", ["linear", "cosine"])
def test_iterated_step_recovers_data_law(sched):
    q = np.array([0.6, 0.25, 0.1, 0.05])
    steps = 1000
    p = np.full(q.size, 1.0 / q.size)          # t = 1: pure uniform noise
    for k in range(steps):
        t = 1.0 - k / steps
        T = _step_kernel(q, t, 1.0 / steps, sched)
        assert np.all(T >= -1e-15) and np.allclose(T.sum(axis=1), 1.0)
        p = p @ T
    assert np.abs(p - q).max() < 2e-3

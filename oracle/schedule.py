"""Noise schedule, Step rate and temperature.

TR summary, Method, forward path equation: kappa_t goes smoothly and
monotonically from kappa_0 = 1 to kappa_1 = 0. The pages give no formula;
the workloads use linear (kappa = 1 - t) and cosine (kappa = cos^2(pi t/2)).

Step (our derivation; the pages stop at the Step relation): the rate
  u(y | x; x0) = kappa'/(1 - kappa) [delta(y, x0) - delta(y, x)]
(kappa' = d kappa / d s with s = 1 - t) generates the forward path;
replacing delta(y, x0) by the posterior p0 and taking one Euler step of
size dt gives (1 - lambda) delta(y, x_t) + lambda p0(y) with
  lambda = dt * (-dkappa/dt) / (1 - kappa_t), clamped to [0, 1].

Temperature (TR summary, Method, sampler paragraph): linear anneal from
tau_max = 0.8 to tau_min = 0.4 over denoising time, read as
tau_t = 0.4 + 0.4 t (t = 1 at the start of generation).
"""
import math
import numpy as np


def schedule_terms(t, schedule):
    """Return (kappa, -dkappa/dt, 1 - kappa) in float64 for a scalar t."""
    t = float(t)
    if schedule == "linear":
        return 1.0 - t, 1.0, t
    if schedule == "cosine":
        c = math.cos(0.5 * math.pi * t)
        s = math.sin(0.5 * math.pi * t)
        # -d/dt cos^2(pi t / 2) = pi sin(pi t / 2) cos(pi t / 2); 1 - kappa = sin^2
        return c * c, math.pi * s * c, s * s
    raise ValueError(schedule)


def step_lambda(t, dt, schedule):
    """lambda in float64, clamped to [0, 1]."""
    _, rate, one_minus = schedule_terms(t, schedule)
    if one_minus <= 0.0:
        return 1.0
    lam = dt * rate / one_minus
    return min(1.0, max(0.0, lam))


def temperature(t):
    return 0.4 + 0.4 * float(t)


def inv_temperature(t):
    """1/tau_t rounded to float32: the value both sides multiply logits by."""
    return np.float32(1.0 / temperature(t))

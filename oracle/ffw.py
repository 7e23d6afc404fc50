"""Self-conditioning feed-forward block, z = FFW(p0 E) -- TEST INFRASTRUCTURE.

TR summary, Method, three-line update: the next self-conditioning signal is
a standard feed-forward network applied to the expected embedding p0 E
(a [C, d] tensor); the Experiments paragraph on the model adds that this
self-conditioning block costs little next to the rest of the network.

The pages give neither the structure nor the width of the block. Reading
taken here: the gated feed-forward layer of the Gemma family that the model
is initialised from,

    FFW(u) = W_down (gelu(W_gate u) * (W_up u)),

with W_gate, W_up [F, d], W_down [d, F], no biases and no residual, GELU in
its tanh form gelu(a) = a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))), and
the hidden width F a parameter. The identity block (F = 0) is the reading
used by the standard workloads.

Rounding points: the input u is the act-rounded p0 E of the step; the hidden
activations gelu(g) * v are rounded to act; the output z is rounded to act.
Sums run in float64.
"""
import numpy as np

from .rounding import round_act

_GELU_C = np.sqrt(2.0 / np.pi)


def gelu_tanh(a):
    """a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))), float64."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * (1.0 + np.tanh(_GELU_C * (a + 0.044715 * a ** 3)))


def ffw_hidden(u, W_gate, W_up, act):
    """Hidden activations [R, F] = round(gelu(u W_gate^T) * (u W_up^T))."""
    d = np.shape(u)[-1]
    x = np.asarray(u, dtype=np.float64).reshape(-1, d)
    g = x @ np.asarray(W_gate, dtype=np.float64).T
    v = x @ np.asarray(W_up, dtype=np.float64).T
    return round_act(gelu_tanh(g) * v, act)


def ffw(u, W_gate, W_up, W_down, act):
    """z = round(hidden W_down^T), same leading shape as u."""
    u = np.asarray(u, dtype=np.float64)
    hid = ffw_hidden(u, W_gate, W_up, act)
    z = hid @ np.asarray(W_down, dtype=np.float64).T
    return round_act(z, act).reshape(u.shape[:-1] + (np.shape(W_down)[0],))

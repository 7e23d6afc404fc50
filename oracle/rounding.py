"""Rounding of oracle tensors to the activation dtype.

bf16 rounding is round-to-nearest, ties-to-even, applied directly to the
float64 value: the significand is kept to 8 bits with numpy's rint (which
rounds half to even). Valid for normal-range values (|x| >= 2^-126) and 0,
which is all the workloads produce.
"""
import numpy as np


def round_bf16(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                   # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_act(x, dtype):
    """Round to the activation dtype; "f64" leaves values unrounded (pin tests)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)

"""The corruption kernel's keep test in integers: u01(w) < kappa holds iff
(w >> 9) < ceil((kappa 2^24 - 1) / 2), with that bound formed in fp32 as the
kernel forms it. Checked here against the float rule (u01(w) is
(2 (w >> 9) + 1) 2^-24) for random and edge values of kappa; the GPU tests
check the kernel itself bit for bit against the oracle."""
import numpy as np


def _float_rule_count(kap):
    # number of k in [0, 2^23) with (2k + 1) 2^-24 < kap in float32: the
    # rule is monotone in k, so bisect
    lo, hi = 0, 2 ** 23
    while lo < hi:
        mid = (lo + hi) // 2
        if np.float32(2 * mid + 1) * np.float32(2.0 ** -24) < kap:
            lo = mid + 1
        else:
            hi = mid
    return lo


def test_integer_keep_bound_matches_the_float_rule():
    rng = np.random.default_rng(1)
    edge = np.array([0.0, 1.0, 0.5, 2.0 ** -24, 2.0 ** -23, 3 * 2.0 ** -25, 1 - 2.0 ** -24,
                     np.nextafter(np.float32(1), np.float32(0)), 1e-30, 0.999999, 0.1, 1 / 3], np.float32)
    kaps = np.concatenate([rng.random(4000).astype(np.float32), edge])
    t = kaps * np.float32(16777216.0)
    bound = np.ceil((t - np.float32(1.0)) * np.float32(0.5)).astype(np.int64)
    for kap, b in zip(kaps, bound):
        assert min(max(int(b), 0), 2 ** 23) == _float_rule_count(kap), float(kap)

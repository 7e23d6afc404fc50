"""Philox4x32-10 counter-based generator and the uniform map.

Philox4x32 is defined in Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11): a 4-word counter and a 2-word key go
through 10 rounds; each round multiplies counter words 0 and 2 by two fixed
odd constants, keeps the high and low halves of both 64-bit products, and
mixes the high halves with the other two counter words and the key; the key
is advanced by two Weyl constants between rounds. The pages fix no RNG;
the library and this oracle both implement this published generator.

Counter map (ours; the pages are silent):
  key     = (low 32 bits of seed, high 32 bits of seed)
  counter = (c0, c1, c2, c3), c3 selects the stream:
    stream 0, Gumbel noise:  (16 (v >> 6) + (v & 15), i, b, 0), word (v >> 4) & 3
                             (vocab id v: block j of each aligned group of 64
                             ids holds ids j, j+16, j+32, j+48)
    stream 1, Step Bernoulli: (0, i, b, 1), word 0
    stream 2, corruption:    (i >> 1, 0, b, 2), words 2*(i&1) (keep draw)
                             and 2*(i&1)+1 (replacement token)
    stream 3, entropy-step re-noise: (0, i, b, 3), word 0
with i the canvas position and b the canvas index.
"""
import numpy as np

MUL0 = 0xD2511F53
MUL1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9
WEYL1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox_scalar(ctr, key, rounds=10):
    """Plain-integer Philox4x32 of one counter; returns a tuple of 4 ints."""
    c0, c1, c2, c3 = (int(v) & MASK32 for v in ctr)
    k0, k1 = (int(v) & MASK32 for v in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + WEYL0) & MASK32
            k1 = (k1 + WEYL1) & MASK32
        p0 = MUL0 * c0
        p1 = MUL1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & MASK32, (p0 >> 32) ^ c3 ^ k1, p0 & MASK32)
    return c0, c1, c2, c3


def philox4x32_10(c0, c1, c2, c3, seed):
    """Vectorised Philox4x32-10 over broadcastable uint32 counter arrays.

    `seed` is a Python int in [0, 2**64); returns four uint32 arrays.
    """
    c = [np.asarray(v, dtype=np.uint64) & np.uint64(MASK32) for v in (c0, c1, c2, c3)]
    c = np.broadcast_arrays(*c)
    c = [a.copy() for a in c]
    k0 = int(seed) & MASK32
    k1 = (int(seed) >> 32) & MASK32
    m32 = np.uint64(MASK32)
    for r in range(10):
        if r:
            k0 = (k0 + WEYL0) & MASK32
            k1 = (k1 + WEYL1) & MASK32
        p0 = np.uint64(MUL0) * c[0]
        p1 = np.uint64(MUL1) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0),
             p1 & m32,
             (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1),
             p0 & m32]
    return tuple(a.astype(np.uint32) for a in c)


def uniform01(w):
    """32-bit word -> float32 uniform in the open interval (0, 1).

    U = (2 * (w >> 9) + 1) * 2^-24: the top 23 bits pick one of 2^23 cells,
    and the value is the cell centre, so every U is exact in float32 and
    neither 0 nor 1 (log(U) and log(-log(U)) are always finite).
    """
    w = np.asarray(w, dtype=np.uint32)
    k = (w >> np.uint32(9)).astype(np.int64) * 2 + 1
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def mulhi_token(w, V):
    """floor(w * V / 2^32): a token id uniform over [0, V) when V divides 2^32."""
    return ((np.asarray(w, dtype=np.uint64) * np.uint64(V)) >> np.uint64(32)).astype(np.int64)

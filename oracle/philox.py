"""Seeded Gaussian draws from a counter-based generator (test oracle only).

When a caller gives the library only a seed, the method's random matrices
(the Gaussian matrix the dense rotation is built from, the Rademacher signs
of the Hadamard variant, the QJL matrix S) are drawn inside the library.
This module is the test side's own implementation of the same published
generator, written from its definition, so the two can be compared:

* Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
  As Easy as 1, 2, 3", SC 2011): a 128-bit counter and a 64-bit key; each of
  ten rounds multiplies counter words 0 and 2 by 0xD2511F53 and 0xCD9E8D57
  (full 64-bit products), and the new counter is (hi1 ^ c1 ^ k0, lo1,
  hi0 ^ c3 ^ k1, lo0); between rounds the key grows by (0x9E3779B9,
  0xBB67AE85).
* Stream layout (this library's choice): draws 2j and 2j+1 of stream s come
  from the block with counter (j mod 2^32, j div 2^32, s, 0) and key
  (seed mod 2^32, seed div 2^32); its words give the 53-bit uniforms
  u1 = (w0 >> 5) 2^-27 + (w1 >> 6) 2^-53 and u2 likewise from w2, w3, and the
  Box-Muller transform gives sqrt(-2 ln(1 - u1)) (cos 2 pi u2, sin 2 pi u2).
* Streams: 1 the rotation's Gaussian matrix, 2 the QJL draws, 3 the Hadamard
  signs (the sign of each draw: negative -> -1, else +1).
"""

import math

import numpy as np

STREAM_ROTATION = 1
STREAM_QJL = 2
STREAM_HADAMARD = 3

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """The block function on arrays of counters: ctr uint64 [..., 4] holding
    32-bit words, key (k0, k1).  Returns the four output words."""
    c = [np.asarray(ctr[..., i], dtype=np.uint64) for i in range(4)]
    k0, k1 = np.uint64(key[0] & _MASK), np.uint64(key[1] & _MASK)
    m = np.uint64(_MASK)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_W0)) & m
            k1 = (k1 + np.uint64(_W1)) & m
        p0 = np.uint64(_M0) * c[0]
        p1 = np.uint64(_M1) * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & m, p1 & m, ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & m, p0 & m]
    return np.stack(c, axis=-1)


def normals(seed, stream, n):
    """n N(0,1) draws (float64) of one stream."""
    nb = (n + 1) // 2
    j = np.arange(nb, dtype=np.uint64)
    ctr = np.stack([j & np.uint64(_MASK), j >> np.uint64(32), np.full(nb, stream, np.uint64),
                    np.zeros(nb, np.uint64)], axis=-1)
    w = philox4x32_10(ctr, (int(seed) & _MASK, (int(seed) >> 32) & _MASK))
    u1 = ((w[:, 0] >> np.uint64(5)).astype(np.float64) * 67108864.0 + (w[:, 1] >> np.uint64(6)).astype(np.float64)) \
        * 2.0 ** -53
    u2 = ((w[:, 2] >> np.uint64(5)).astype(np.float64) * 67108864.0 + (w[:, 3] >> np.uint64(6)).astype(np.float64)) \
        * 2.0 ** -53
    out = np.empty(2 * nb)
    for i in range(nb):  # the C library's log / cos / sin, one pair at a time
        rad = math.sqrt(-2.0 * math.log(1.0 - u1[i]))
        ang = 6.283185307179586 * u2[i]
        out[2 * i] = rad * math.cos(ang)
        out[2 * i + 1] = rad * math.sin(ang)
    return out[:n]


def rotation_draws(seed, d):
    return normals(seed, STREAM_ROTATION, d * d).reshape(d, d)


def qjl_draws(seed, d):
    return normals(seed, STREAM_QJL, d * d).reshape(d, d)


def hadamard_draws(seed, d):
    """d Rademacher values: the signs of stream 3's draws."""
    return np.where(normals(seed, STREAM_HADAMARD, d) < 0.0, -1.0, 1.0)

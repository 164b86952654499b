"""Philox4x32-10 counter-based generator (oracle side): TEST INFRASTRUCTURE ONLY.

Written from the published definition (Salmon, Moraes, Dror, Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11, the Philox-4x32 bijection with
10 rounds).  The pages leave the sampler open: stage 1 of §3 of "Prof-K:
Probabilistic One-Pass Filtering for Efficient Top-k Selection" only asks
for S indices drawn uniformly without replacement, and App. C says they came
from standard library calls.  The GPU library implements the same
generator independently; the two share no code.

One round maps a 4x32-bit counter (c0, c1, c2, c3) under a 2x32-bit key
(k0, k1) to

    (hi(B*c2) ^ c1 ^ k0,  lo(B*c2),  hi(A*c0) ^ c3 ^ k1,  lo(A*c0))

with A = 0xD2511F53, B = 0xCD9E8D57 (hi/lo = upper/lower 32 bits of the
64-bit product).  Between rounds the key is advanced by the Weyl constants
(0x9E3779B9, 0xBB67AE85) modulo 2^32.
"""
from __future__ import annotations

import numpy as np

_A = np.uint64(0xD2511F53)
_B = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32(c0, c1, c2, c3, k0: int, k1: int, rounds: int = 10):
    """Vectorised Philox4x32-R.  Counters are array-likes of uint32 values;
    returns four uint64 arrays holding the 32-bit output words."""
    c0 = np.asarray(c0, dtype=np.uint64) & _M32
    c1 = np.asarray(c1, dtype=np.uint64) & _M32
    c2 = np.asarray(c2, dtype=np.uint64) & _M32
    c3 = np.asarray(c3, dtype=np.uint64) & _M32
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _A * c0  # both factors < 2^32, product fits in 64 bits
        p1 = _B * c2
        n0 = (p1 >> _S32) ^ c1 ^ np.uint64(k0)
        n1 = p1 & _M32
        n2 = (p0 >> _S32) ^ c3 ^ np.uint64(k1)
        n3 = p0 & _M32
        c0, c1, c2, c3 = n0, n1, n2, n3
    return c0, c1, c2, c3

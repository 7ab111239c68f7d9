"""Philox4x32-10 counter-based generator and the random-sign test matrix drawn
from it — oracle only (test infrastructure, never part of the product path).

Philox4x32-10 is the generator of Salmon, Moraes, Dror & Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11): a 4 x 32-bit counter and a 2 x 32-bit key,
ten rounds of two 32 x 32 -> 64-bit multiplications (multipliers 0xD2511F53 and
0xCD9E8D57) whose high halves are xored with the other counter words and the
round key, the key advancing by the Weyl constants 0x9E3779B9 and 0xBB67AE85
after each round.  Written here from that description in plain Python integers.

Test matrix (the library's choice when the caller passes none): entries are
independent random signs, +1 or -1 (a sub-Gaussian test matrix, Halko, Martinsson
& Tropp 2011, §4.6 and §11).  For matrix `mat` (2*b for K, 2*b+1 for V) element
(w, j) of the W x ell matrix has linear index i = j*W + w; Philox is called with
counter (i // 128, mat, 0, 0) and key (seed mod 2^32, seed >> 32); bit i % 32 of
output word (i // 32) % 4 set means -1.

Pins: the published known-answer vectors of Philox4x32-10
(tests/golden/philox_kat.json, tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """One Philox4x32-10 block: four 32-bit words from counter[4] and key[2]."""
    c0, c1, c2, c3 = (int(x) & MASK for x in counter)
    k0, k1 = (int(x) & MASK for x in key)
    for _ in range(10):
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK
        hi1, lo1 = p1 >> 32, p1 & MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + W0) & MASK
        k1 = (k1 + W1) & MASK
    return c0, c1, c2, c3


def sign_omega(seed: int, mat: int, W: int, ell: int) -> np.ndarray:
    """The W x ell random-sign test matrix of matrix `mat`, float64 of +-1."""
    key = (seed & MASK, (seed >> 32) & MASK)
    n = W * ell
    flat = np.empty(n, dtype=np.float64)
    for blk in range((n + 127) // 128):
        words = philox4x32_10((blk, mat, 0, 0), key)
        for t in range(min(128, n - 128 * blk)):
            bit = (words[t >> 5] >> (t & 31)) & 1
            flat[128 * blk + t] = -1.0 if bit else 1.0
    # flat is laid out [j][w]
    return flat.reshape(ell, W).T.copy()

"""One-dimensional Sobol points at p bits (test infrastructure; see package
docstring).

Source: "Precision As You Need" paper notes, Key design 1: the stream
generator is a Sobol-8 sequence whose cumulative indicator table is built once
and sliced by prefix.  The notes name the generator but not its ordering or
scrambling; the reading taken here is the plain, unscrambled 1-D Sobol
sequence in Gray-code order with first point 0 (direction numbers
v_k = 2^(p-k)), the textbook construction.
"""

import numpy as np


def sobol_points(p: int, n: int) -> np.ndarray:
    """First ``n`` points r_0 .. r_{n-1} of the 1-D Sobol sequence as integers
    in [0, 2^p).

    Gray-code recurrence: r_0 = 0 and r_l = r_{l-1} XOR v_c, where c is one
    plus the number of trailing one-bits of l-1 and v_c = 2^(p-c).

    Pinned by: the bit-reversed Gray-code closed form, torch's unscrambled
    SobolEngine, and the permutation property over a full period.
    """
    if not (1 <= p <= 16):
        raise ValueError("p out of range")
    if not (0 <= n <= (1 << p)):
        raise ValueError("n must be in [0, 2^p]")
    r = np.zeros(n, dtype=np.int64)
    for l in range(1, n):
        prev = l - 1
        c = 1
        while prev & 1:
            prev >>= 1
            c += 1
        r[l] = r[l - 1] ^ (1 << (p - c))
    return r

"""Rows whose quantisation hits exact .5 ties, for tests with no tie window.

For a Hadamard matrix H of order b (+-1 entries) pick an output column i0 of
a block, a subset S of the block's input positions and positive integers
c_j (j in S) summing to M = 4 * qmax, and set u_j = c_j * H[j, i0] (zero
elsewhere).  Then y = u.H has y_i0 = sum c_j = M, |y_i| <= M everywhere, and
every y_i = sum c_j H[j, i0] H[j, i] has the parity of M: all y_i are even.
Built block by block, every block's maximum is M, so the row's (and any
group of whole blocks') maximum is M and x'/scale = qmax * y / M = y / 4,
which lies exactly on a .5 boundary wherever y = 2 (mod 4).  The input is
x = u * s for the sign vector s (s = +-1, so (x * s) = u).

All values are small integers: exact in bf16 (|c_j| <= 256 here), f16 and
fp32, and every partial sum of a transform is an integer below 2^24, so a
GPU computing in fp32 from these inputs makes no rounding error before the
quantiser.  The Hadamard matrices come from the oracle (whose Sylvester and
Paley constructions are pinned on their own).
"""
from __future__ import annotations

import numpy as np


def tie_rows(H: np.ndarray, rows: int, n: int, s: np.ndarray, bits: int,
             rng: np.random.Generator) -> np.ndarray:
    """float32 [rows, n] of small integers; H is the b x b matrix of the
    block rotation (b divides n)."""
    b = H.shape[0]
    qmax = (1 << (bits - 1)) - 1
    M = 4 * qmax
    x = np.zeros((rows, n), dtype=np.int64)
    for r in range(rows):
        for k in range(n // b):
            i0 = int(rng.integers(b))
            cap = min(b, M)
            cnt = int(rng.integers(max(1, cap // 2), cap + 1))
            S = rng.choice(b, size=cnt, replace=False)
            c = 1 + rng.multinomial(M - cnt, np.full(cnt, 1.0 / cnt))
            u = np.zeros(b, dtype=np.int64)
            u[S] = c * H[S, i0].astype(np.int64)
            x[r, k * b:(k + 1) * b] = u
    assert np.abs(x).max() <= 256
    return (x * s.astype(np.int64)[None, :]).astype(np.float32)


def to_dtype(x: np.ndarray, dtype: int) -> np.ndarray:
    """The same (exactly representable) values as raw fp32, bf16 or f16
    storage (element types numbered as in the library: 0 f32, 1 bf16,
    2 f16)."""
    if dtype == 0:
        return x
    if dtype == 2:
        h = x.astype(np.float16)
        assert np.array_equal(h.astype(np.float32), x)
        return h.view(np.uint16)
    bits = x.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    return (bits >> 16).astype(np.uint16)


def exact_ties(preround: np.ndarray) -> int:
    """How many pre-rounding values lie exactly on a .5 boundary."""
    return int(np.sum(np.abs(preround - np.floor(preround)) == 0.5))

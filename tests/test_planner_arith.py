"""Integer identity the rank-per-lane planner relies on for the water-fill's
division S / m* (m* <= 64 instances, S < 2^32): with R = floor((2^32 - 1) / m),
the high word of S * R is floor(S / m) or one less, so one correction step
gives the exact quotient.  Checked here on the host, exhaustively over m and
over the dividends where an off-by-one would show (multiples of m and their
neighbours, the top of the range) plus random ones."""
import numpy as np


def _quotient(S, m):
    R = np.uint64(0xFFFFFFFF // m)
    q = (S.astype(np.uint64) * R) >> np.uint64(32)
    rem = S.astype(np.uint64) - q * np.uint64(m)
    fix = rem >= np.uint64(m)
    return q + fix.astype(np.uint64), rem - np.where(fix, np.uint64(m), np.uint64(0))


def test_reciprocal_division_exact():
    rng = np.random.default_rng(7)
    top = np.uint64(0xFFFFFFFF)
    for m in range(1, 65):
        mult = np.arange(0, 2**32, m * 1009, dtype=np.uint64)
        cand = np.concatenate([
            mult, mult + 1, np.clip(mult.astype(np.int64) - 1, 0, None).astype(np.uint64),
            np.arange(2**32 - 4 * m, 2**32, dtype=np.uint64),
            (np.arange(1, 2**32 // m, 997, dtype=np.uint64) * np.uint64(m)) - np.uint64(1),
            rng.integers(0, 2**32, 20000, dtype=np.uint64),
        ])
        cand = cand[cand <= top]
        q, rem = _quotient(cand, m)
        assert np.array_equal(q, cand // np.uint64(m)), m
        assert np.array_equal(rem, cand % np.uint64(m)), m

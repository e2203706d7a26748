"""Numerical model of the sliced Gram matrix (CPU).

The int8 Gram kernel writes each float32 column q_j as 2^e_j times five
signed base-128 digits (d_t in [-64, 64], weight 2^-(7 t + 6)) and keeps the
digit products of level a + b <= 4.  This model restates that arithmetic in
numpy integers, independently of the kernel source, and checks the claims
the library makes about it: the digits fit int8, the remainder is below
2^-35, every product q_ik q_jk is formed within 2^-30 max|q_i| max|q_j| even
for digits at their largest, the int32 level sums of 65,536 rows cannot
overflow, and on random columns the Gram matrix agrees with the exact one
far inside the bound.
"""
from fractions import Fraction

import numpy as np

DIGITS = 5


def column_exponent(q):
    """The e with max|q| < 2^e (0 for a zero column)."""
    m = float(np.max(np.abs(q)))
    return 0 if m == 0.0 else int(np.frexp(m)[1])


def digits(q, e):
    """Base-128 digits of q / 2^e (float64 arithmetic is exact here)."""
    y = np.ldexp(q.astype(np.float64), -e)
    out = np.zeros((DIGITS,) + q.shape, dtype=np.int64)
    for t in range(DIGITS):
        x = np.rint(np.ldexp(y, 7 * t + 6))
        y = y - np.ldexp(x, -(7 * t + 6))
        out[t] = x.astype(np.int64)
    return out, y


def sliced_gram(Q):
    """S from the digit products of level <= DIGITS - 1, as the kernel sums them."""
    r = Q.shape[1]
    e = [column_exponent(Q[:, j]) for j in range(r)]
    D = [digits(Q[:, j], e[j])[0] for j in range(r)]
    S = np.zeros((r, r))
    for i in range(r):
        for j in range(r):
            lev = [sum(int(D[i][a] @ D[j][l - a]) for a in range(l + 1)) for l in range(DIGITS)]
            x = sum(lev[l] << (7 * (DIGITS - 1 - l)) for l in range(DIGITS))
            S[i, j] = np.ldexp(float(x), e[i] + e[j] - (7 * (DIGITS - 1) + 12))
    return S


def exact_gram(Q):
    r = Q.shape[1]
    F = [[Fraction(float(v)) for v in Q[:, j]] for j in range(r)]
    return np.array([[float(sum(a * b for a, b in zip(F[i], F[j]))) for j in range(r)] for i in range(r)])


def test_digits_fit_int8_and_reconstruct():
    rng = np.random.default_rng(0)
    q = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    e = column_exponent(q)
    D, rem = digits(q, e)
    assert np.abs(D).max() <= 64
    assert np.abs(rem).max() <= 2.0 ** -35
    recon = sum(np.ldexp(D[t].astype(np.float64), e - (7 * t + 6)) for t in range(DIGITS))
    assert np.all(np.abs(recon - q.astype(np.float64)) <= np.ldexp(1.0, e - 35))


def test_product_bound_at_largest_digits():
    # entries whose digits are all +-64 or close (the largest dropped
    # products), and spikes next to tiny entries
    vals = []
    for s in (1.0, -1.0):
        x = 0.0
        for t in range(DIGITS + 2):
            x += s * 64 * 2.0 ** -(7 * t + 6) * (1 - 2 ** -20)
        vals.append(np.float32(x))
    vals += [np.float32(0.9999999), np.float32(-0.5000001), np.float32(2.0 ** -30), np.float32(3e-12)]
    vals = np.array(vals, dtype=np.float32)
    for qi in vals:
        for qj in vals:
            col_i = np.array([qi, np.float32(0.99)], dtype=np.float32)
            col_j = np.array([qj, np.float32(0.99)], dtype=np.float32)
            ei, ej = column_exponent(col_i), column_exponent(col_j)
            Di, _ = digits(col_i[:1], ei)
            Dj, _ = digits(col_j[:1], ej)
            lev = sum(int(Di[a][0] * Dj[l - a][0]) * 2 ** (7 * (DIGITS - 1 - l))
                      for l in range(DIGITS) for a in range(l + 1))
            got = Fraction(lev) * Fraction(2) ** (ei + ej - (7 * (DIGITS - 1) + 12))
            want = Fraction(float(qi)) * Fraction(float(qj))
            bound = Fraction(2) ** -30 * Fraction(float(np.max(np.abs(col_i)))) * Fraction(float(np.max(np.abs(col_j))))
            assert abs(got - want) <= bound, (qi, qj)


def test_int32_level_sums_do_not_overflow():
    # one flush interval (65,536 rows): a level has at most 5 digit pairs
    # of magnitude <= 64 each per row
    assert 65536 * DIGITS * 64 * 64 < 2 ** 31


def test_sliced_gram_close_to_exact():
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((300, 6)).astype(np.float32)
    Q[:, 1] *= np.float32(1e-20)
    Q[:, 2] *= np.float32(1e20)
    Q[:, 4] = 0.0
    S = sliced_gram(Q)
    E = exact_gram(Q)
    d = np.sqrt(np.diag(E))
    norm = np.outer(d, d)
    norm[norm == 0] = 1.0
    assert np.max(np.abs(S - E) / norm) < 1e-9
    assert np.all(S[4, :] == 0) and np.all(S[:, 4] == 0)


def test_model_detects_a_missing_level():
    # the same comparison fails when the last level (5 digit products) is
    # left out, so the check above is sensitive to the kept terms
    global DIGITS
    rng = np.random.default_rng(2)
    Q = rng.standard_normal((200, 4)).astype(np.float32)
    E = exact_gram(Q)
    d = np.sqrt(np.diag(E))
    saved = DIGITS
    try:
        DIGITS = 4
        S = sliced_gram(Q)
    finally:
        DIGITS = saved
    assert np.max(np.abs(S - E) / np.outer(d, d)) > 1e-9


def test_float32_digit_steps_are_exact():
    # the digit steps in float32 (scale by 2^-e, then per digit: multiply by
    # a power of two, round to nearest, subtract) give the float64 digits,
    # including entries far below the column's largest and subnormal ones
    rng = np.random.default_rng(3)
    q = (rng.standard_normal(20000) * np.exp(rng.uniform(-60, 0, 20000))).astype(np.float32)
    q[:4] = np.array([1.0, -0.999999, 1e-40, -3e-42], dtype=np.float32)
    e = column_exponent(q)
    d64, _ = digits(q, e)
    y = np.ldexp(q, -e).astype(np.float32)
    for t in range(DIGITS):
        up = np.float32(2.0 ** (7 * t + 6))
        x = np.rint(y * up).astype(np.float32)
        y = (y - x / up).astype(np.float32)
        assert np.array_equal(x.astype(np.int64), d64[t]), t

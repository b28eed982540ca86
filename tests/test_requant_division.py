"""The int8-output epilogue divides by the output scale with Markstein's
correction step instead of a full IEEE division: with r = RN(1/s),
q0 = RN(y r), e = y - q0 s (exact, one FMA) and RN(q0 + e r), which equals
RN(y / s) for quotients in the normal range (P. Markstein, "Computation of
elementary functions on the IBM RISC System/6000 processor", IBM J. Res. Dev.
34(1), 1990).  The codes must equal those of the graph-entry quantiser, which
divides with a correctly rounded division, so the claim is checked here in
exact rational arithmetic on random and near-tie operands (CPU only), together
with the host's reciprocal rule r = float(1 / double(s)).
"""
from fractions import Fraction

import numpy as np


def rn32(x: Fraction) -> Fraction:
    """Round a rational to the nearest fp32 value, ties to even (normal range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # 2^e <= a < 2^(e+1): scale the 24-bit significand to an integer
    scale = Fraction(2) ** (e - 23)
    m = a / scale
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * scale


def f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def markstein(y: Fraction, s: Fraction, r: Fraction) -> Fraction:
    q0 = rn32(y * r)
    e = rn32(y - q0 * s)          # the FMA's single rounding; exact in practice
    return rn32(q0 + e * r)


def host_reciprocal(s: np.float32) -> Fraction:
    return Fraction(float(np.float32(1.0 / float(s))))


def test_host_reciprocal_is_correctly_rounded():
    rng = np.random.default_rng(0)
    for s in np.concatenate([rng.uniform(1e-4, 10, 3000), 2.0 ** rng.integers(-20, 10, 200),
                             rng.uniform(0.01, 0.1, 3000)]).astype(np.float32):
        assert host_reciprocal(s) == rn32(1 / Fraction(float(s))), s


def test_markstein_quotient_is_correctly_rounded():
    rng = np.random.default_rng(1)
    cases = []
    for _ in range(6000):
        s = np.float32(rng.uniform(1e-3, 1.0))
        y = np.float32(rng.uniform(-128, 128) * s)
        cases.append((y, s))
    # operands whose quotient sits next to a rounding boundary (k + 1/2) of the quantiser
    for _ in range(6000):
        s = np.float32(np.exp(rng.uniform(np.log(1e-3), np.log(10))))
        k = int(rng.integers(-128, 128))
        y0 = np.float32((k + 0.5) * float(s))
        d = int(rng.integers(-3, 4))
        y = np.float32(np.nextafter(y0, np.float32(np.inf if d > 0 else -np.inf))) if d else y0
        for _ in range(abs(d) - 1):
            y = np.float32(np.nextafter(y, np.float32(np.inf if d > 0 else -np.inf)))
        cases.append((y, s))
    # exact multiples, zero and tiny values
    for s in (np.float32(0.03), np.float32(0.5), np.float32(1.0 / 3.0)):
        for k in range(-128, 129, 7):
            cases.append((np.float32(k * float(s)), s))
        cases += [(np.float32(0.0), s), (np.float32(1e-30), s), (np.float32(-1e-30), s)]
    bad = 0
    for y, s in cases:
        yf, sf = Fraction(float(y)), Fraction(float(s))
        got = markstein(yf, sf, host_reciprocal(s))
        if got != rn32(yf / sf):
            bad += 1
    assert bad == 0, "%d of %d quotients differ from the correctly rounded one" % (bad, len(cases))


def test_rn32_matches_numpy_on_doubles():
    """The rational rounding helper itself agrees with IEEE fp64 -> fp32 conversion."""
    rng = np.random.default_rng(2)
    for v in rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000):
        assert rn32(Fraction(float(v))) == Fraction(float(np.float32(v))), v

"""The kernels divide pixel and workgroup indices by run-time constants (OW,
OH, tile counts, split-K) with a multiply-high, an add and a shift
(Granlund and Montgomery, "Division by invariant integers using
multiplication", PLDI 1994, Figure 4.1).  This checks the rule the host uses
to derive the multiplier, for every numerator form the kernels can produce
(below 2^31), on the CPU: divisors 1..4096 and random ones up to 2^31 - 1,
numerators at and around multiples of the divisor up to the top of the range.
"""
import numpy as np


def magic(d):
    l = 0
    while (1 << l) < d:
        l += 1
    return ((1 << 32) * ((1 << l) - d)) // d + 1, l


def fdiv(n, d):
    m, l = magic(d)
    assert 0 <= m < (1 << 32)
    t = (n * m) >> 32                      # mulhi
    s = t + n
    assert s < (1 << 32), "sum must stay within 32 bits"
    return s >> l


def test_fastdiv_exact_below_2_31():
    rng = np.random.default_rng(0)
    divisors = list(range(1, 4097)) + [int(v) for v in rng.integers(4097, 2**31 - 1, 300)] + [2**31 - 1, 2**30, 6400,
                                                                                              102400, 409600]
    top = 2**31 - 1
    for d in divisors:
        ks = {0, 1, 2, 3, top // d - 1, top // d, top // (2 * d), int(rng.integers(0, top // d + 1))}
        ns = set()
        for k in ks:
            for delta in (-1, 0, 1):
                n = k * d + delta
                if 0 <= n <= top:
                    ns.add(n)
        ns.update(int(v) for v in rng.integers(0, top + 1, 8))
        ns.add(top)
        for n in ns:
            assert fdiv(n, d) == n // d, (n, d)

"""Host-side pins of the activation digits that the single-token kernels feed
to the matrix unit (built on the GPU; restated here in exact arithmetic to
check the claims the kernels rest on):

- the E4M3 code of a digit d in 0..15 is d itself and means d * 2^-9, from
  the format's definition (1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits, exponent field 0 subnormal); sign in bit 7;
- six base-16 digits of |v| rounded at 2^(Emax - 23) carry every bf16 value
  within 2^-16 of its group's largest exactly, and any fp32 value to within
  2^(Emax - 24) (half an ulp of the group's largest);
- a block's products (E2M1 magnitude times digit) span less than 2^8.
"""
from fractions import Fraction

import numpy as np

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def e4m3_value(code):
    """Value of an E4M3 byte (finite codes), from the format's fields."""
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def digits(group):
    """(Emax, [(sign, d_0..d_5)] per value): the scheme's digits of a group of
    32 float32 values (all finite, not all zero)."""
    bits = np.asarray(group, np.float32).view(np.uint32)
    emax = int(((bits >> 23) & 255).max())
    E = emax - 127
    out = []
    for v in np.asarray(group, np.float32):
        F = int(np.rint(abs(float(v)) * 2.0 ** (150 - emax)))  # exact product, < 2^24
        assert 0 <= F < 2 ** 24
        out.append((-1 if np.signbit(v) else 1, [(F >> (20 - 4 * p)) & 15 for p in range(6)]))
    return E, out


def rebuild(E, digs, code_value=lambda d: Fraction(d, 512)):
    """Each value from its digits: slice p's code d (meaning d 2^-9) times its
    block scale 2^(E - 3 - 4p + 9)."""
    vals = []
    for sign, ds in digs:
        vals.append(sign * sum(code_value(d) * Fraction(2) ** (E - 3 - 4 * p + 9)
                               for p, d in enumerate(ds)))
    return vals


def to_bf16(a):
    u = np.asarray(a, np.float32).view(np.uint32)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def test_digit_codes_are_linear():
    for d in range(16):
        assert e4m3_value(d) == Fraction(d, 512)
        assert e4m3_value(0x80 | d) == -Fraction(d, 512)
    # 16 (1.0 * 2^-5) is still 16 * 2^-9; 17 is the first code that is not
    assert e4m3_value(16) == Fraction(16, 512)
    assert e4m3_value(17) != Fraction(17, 512)


def test_rebuild_uses_the_decoded_codes():
    rng = np.random.default_rng(7)
    g = rng.standard_normal(32).astype(np.float32)
    E, digs = digits(g)
    assert rebuild(E, digs, e4m3_value) == rebuild(E, digs)


def test_bf16_within_2_16_of_the_largest_is_exact():
    rng = np.random.default_rng(11)
    for trial in range(300):
        top = rng.integers(-40, 40)
        mags = 2.0 ** (top - rng.uniform(0, 16, 32))  # within 2^-16 of 2^top
        g = to_bf16(mags * rng.choice([-1.0, 1.0], 32))
        E, digs = digits(g)
        got = rebuild(E, digs)
        assert all(gv == Fraction(float(v)) for gv, v in zip(got, g)), trial


def test_fp32_within_half_an_ulp_of_the_group_largest():
    rng = np.random.default_rng(13)
    for trial in range(300):
        g = (rng.standard_normal(32) * 2.0 ** rng.uniform(-30, 0, 32)).astype(np.float32)
        E, digs = digits(g)
        got = rebuild(E, digs)
        bound = Fraction(2) ** (E - 24)
        assert all(abs(gv - Fraction(float(v))) <= bound for gv, v in zip(got, g)), trial


def test_block_products_span_less_than_2_8():
    prods = [c * d for c in E2M1[1:] for d in range(1, 16)]
    assert max(prods) / min(prods) < 2 ** 8

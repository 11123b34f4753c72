"""Definitions used to pin the oracle, written independently of it.

Each function restates a fact from the format or from mathematics through a
different route than the oracle's code: E2M1 from its bit fields instead of a
table, exact rational arithmetic instead of fp64 loops, numpy expansion plus a
library matrix product instead of the packed group-then-scale loop.
"""
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_from_bits(code):
    """OCP E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exact."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def e2m1_signbit(code):
    return (code >> 3) & 1


def pack_codes(codes):
    """codes int[rows][cols] -> canonical nibble bytes (even element in the
    low nibble, as the pages state)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    rows, half = nib.shape
    codes = np.empty((rows, half * 2), np.uint8)
    codes[:, 0::2] = nib & 15
    codes[:, 1::2] = nib >> 4
    return codes


_E2M1_F = np.array([float(e2m1_from_bits(c)) for c in range(16)])
_E2M1_F[8] = -0.0


def dequant_numpy(nib, sc):
    """Expand to float64 through the bit definition (vectorised)."""
    codes = unpack_codes(nib)
    rows, cols = codes.shape
    vals = _E2M1_F[codes]
    scale = np.array([math.ldexp(1.0, int(e) - 127) if e != 255 else 0.0
                      for e in np.asarray(sc).ravel()]).reshape(sc.shape)
    return vals * np.repeat(scale, 32, axis=1)


def exact_gemv(nib, sc, x):
    """Exact rational y = W x (255 groups skipped) and sum |terms| per row."""
    codes = unpack_codes(nib)
    rows, cols = codes.shape
    xf = [Fraction(float(v)) for v in x]
    ys, mags = [], []
    for r in range(rows):
        acc, mag = Fraction(0), Fraction(0)
        for g in range(cols // 32):
            e = int(sc[r, g])
            if e == 255:
                continue
            s = Fraction(2) ** (e - 127)
            for i in range(32):
                t = e2m1_from_bits(int(codes[r, 32 * g + i])) * xf[32 * g + i] * s
                acc += t
                mag += abs(t)
        ys.append(acc)
        mags.append(mag)
    return ys, mags


def bf16_to_float_bits(a):
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sigmoid(v):
    return 1.0 / (1.0 + math.exp(-v))


def silu_tanh_form(v):
    """SiLU through identities other than v/(1+e^-v): v/2 * (1 + tanh(v/2))
    for v >= 0 and v e^v / (1 + e^v) for v < 0 (both free of cancellation)."""
    if v >= 0:
        return 0.5 * v * (1.0 + math.tanh(0.5 * v))
    ev = math.exp(v)
    return v * ev / (1.0 + ev)


def read_golden_rows(name):
    rows, data_bytes = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "bytes":
                data_bytes = [int(t, 16) for t in tok[1:]]
            elif tok[0] == "row":
                vals = [(-0.0 if t == "-0" else float(Fraction(t))) for t in tok[2:]]
                rows.append((int(tok[1]), vals))
    return data_bytes, rows


def read_census():
    out = {}
    with open(os.path.join(GOLDEN, "census.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tok = line.split()
            out[tok[0]] = float(tok[1])
    return out


def bf16_nearest_even_bits(u32):
    """bf16 bits nearest to the float32 with bits u32, ties to the even
    pattern, by exact rational comparison of the two bf16 neighbours.
    Overflow follows IEEE 754 round-to-nearest: the value past the largest
    finite bf16 is taken as 2^128, so ties there go to the infinity (whose
    mantissa is even). NaN inputs are not handled here."""
    u32 = int(u32) & 0xFFFFFFFF
    sign = u32 >> 31
    mag_bits = u32 & 0x7FFFFFFF
    if mag_bits == 0x7F800000:
        return (sign << 15) | 0x7F80
    v = abs(Fraction(float(np.array([mag_bits], np.uint32).view(np.float32)[0])))
    lo = mag_bits >> 16                   # toward zero

    def val(b):
        if b >= 0x7F80:
            return Fraction(2) ** 128
        return abs(Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0])))

    d_lo, d_hi = v - val(lo), val(lo + 1) - v
    if d_lo < d_hi or (d_lo == d_hi and lo % 2 == 0):
        out = lo
    else:
        out = lo + 1
    return (sign << 15) | min(out, 0x7F80)

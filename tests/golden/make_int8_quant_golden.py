"""Write int8_quant_cases.txt: per-(token, head) INT8 codes derived with exact
rational arithmetic, for vectors on which plausible implementations of the
quantiser's division disagree.

The quantiser (the library's INT8 KV scheme; the paper, "LongLive: Real-time
Interactive Long Video Generation", Abstract and §5, reports INT8 inference
without a scheme) is, per vector x of bf16 values:

    a = max |x|                          exact
    s = fl32(a / 127)                    the binary32 value nearest a/127
    code = clamp(rne(fl32(x / s)), -127, 127)

Here every step is done on Python Fractions: a/127 and x/s are exact
rationals, fl32 rounds an exact rational to the nearest binary32 value by hand
(ties to an even significand; subnormals included), and rne rounds a rational
to the nearest integer (ties to even).  No floating-point division is used to
derive a stored value.

Vectors come from a seeded N(0,1) draw rounded to bf16.  A vector is kept when
the exact codes differ from those of one of two near-miss variants, so that a
quantiser implementing either variant fails the table:

    recip: rne(fl32(x * fl32(1/s)))      (multiply by a rounded reciprocal)
    f64:   rne(fl64(x / s))              (division in binary64)

(both variants are also evaluated with Fractions and explicit rounding).  The
table also keeps a few vectors on which all variants agree, a zero vector, and
a vector whose max is 127 (s = 1 exactly).

Run:  python tests/golden/make_int8_quant_golden.py
"""

import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "int8_quant_cases.txt")
D = 16


def nearest_binary(r, mant_bits, emin):
    """Nearest binary floating-point value to the rational r with a
    significand of mant_bits bits (implicit bit included) and minimum normal
    exponent emin, ties to even; no overflow handling (not needed here)."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    m = abs(r)
    # exponent e with 2^e <= m < 2^(e+1)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    e = max(e, emin)                       # subnormal range: fixed quantum
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    n = m / quantum
    f = n.numerator // n.denominator
    rem = n - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return sign * f * quantum


def fl32(r):
    return nearest_binary(r, 24, -126)


def fl64(r):
    return nearest_binary(r, 53, -1022)


def rne(r):
    f = r.numerator // r.denominator
    rem = r - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def clamp127(c):
    return max(-127, min(127, c))


def quantise_exact(xs):
    """xs: list of Fractions (bf16 values).  Returns (scale, codes, recip codes,
    f64 codes)."""
    a = max(abs(x) for x in xs)
    if a == 0:
        z = [0] * len(xs)
        return Fraction(0), z, z, z
    s = fl32(a / 127)
    inv = fl32(1 / s)
    exact = [clamp127(rne(fl32(x / s))) for x in xs]
    recip = [clamp127(rne(fl32(x * inv))) for x in xs]
    f64 = [clamp127(rne(fl64(x / s))) for x in xs]
    return s, exact, recip, f64


def bf16_values(bits):
    """uint16 bf16 bit patterns -> exact Fractions."""
    f32 = (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return [Fraction(float(v)) for v in f32]


def f32_hex(fr):
    return "%08x" % np.array([float(fr)], np.float32).view(np.uint32)[0]


def draw_bits(rng, n):
    x = rng.standard_normal((n, D)).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)


def main():
    rng = np.random.default_rng(20260314)
    rows = []
    want_recip, want_f64, want_plain = 6, 6, 3
    n_recip = n_f64 = n_plain = 0
    while n_recip < want_recip or n_f64 < want_f64 or n_plain < want_plain:
        for bits in draw_bits(rng, 512):
            xs = bf16_values(bits)
            s, exact, recip, f64 = quantise_exact(xs)
            tag = []
            if exact != recip and n_recip < want_recip:
                tag.append("recip")
            if exact != f64 and n_f64 < want_f64:
                tag.append("f64")
            if not tag and exact == recip == f64 and n_plain < want_plain:
                tag.append("plain")
            if not tag:
                continue
            n_recip += "recip" in tag
            n_f64 += "f64" in tag
            n_plain += "plain" in tag
            diff = sorted({i for i in range(D) if exact[i] != recip[i] or exact[i] != f64[i]})
            rows.append((bits, s, exact, ",".join(tag), diff))
    # a zero vector and a vector with max exactly 127 (s = 1, x/s = x)
    zero = np.zeros(D, np.uint16)
    rows.append((zero,) + quantise_exact(bf16_values(zero))[:2] + ("zero", []))
    t = np.zeros(D, np.float32)
    t[:6] = [127.0, 2.5, 3.5, -2.5, 0.5, -126.5]
    tb = (t.view(np.uint32) >> 16).astype(np.uint16)
    rows.append((tb,) + quantise_exact(bf16_values(tb))[:2] + ("ties", []))
    with open(OUT, "w") as f:
        f.write("# INT8 quantiser cases: per-(token, head) vectors of %d bf16 values, their fp32\n" % D)
        f.write("# scale s = fl32(max|x| / 127) and codes clamp(rne(fl32(x / s)), -127, 127).\n")
        f.write("# Written by make_int8_quant_golden.py from exact rational arithmetic (Fractions,\n")
        f.write("# rounding to binary32 and to integers done by hand, ties to even); no value\n")
        f.write("# comes from a floating-point division or from the library.\n")
        f.write("# tag: recip = the exact codes differ from rne(fl32(x * fl32(1/s)));\n")
        f.write("#      f64 = they differ from rne(fl64(x / s)); plain = all three agree.\n")
        f.write("# diff lists the element indices where a variant differs.\n")
        f.write("# format: tag | diff | x as bf16 hex bits | s as fp32 hex bits | codes\n")
        for bits, s, codes, tag, diff in rows:
            f.write("%s | %s | %s | %s | %s\n" % (
                tag, ",".join(map(str, diff)) or "-", ",".join("%04x" % b for b in bits),
                f32_hex(s), ",".join(map(str, codes))))
    print("wrote", OUT, len(rows), "rows")


if __name__ == "__main__":
    main()

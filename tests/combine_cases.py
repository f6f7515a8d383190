"""Exact model of the combine arithmetic and inputs that separate it from
its near neighbours, shared by the oracle pins and the GPU combine test.

The combine reading fixes fp32 accumulation with one fused multiply-add per
routed row, in column order j = 0..K-1, and one final rounding to bf16.  The
model rebuilds that chain from its mathematical definition: exact rationals,
each fma rounded once to the nearest binary32 (ties to even)."""
from fractions import Fraction

import numpy as np
import torch

from synth.gen import bf16_bits


def _torch_bf16_bits(v: np.ndarray) -> np.ndarray:
    return bf16_bits(torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16))


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round_rational(q: Fraction, prec: int, emin: int = -126) -> Fraction:
    """Nearest number with `prec` significant bits (binary32: 24, bf16: 8) and
    the binary32 exponent range (subnormals below 2^emin), ties to an even
    last significand bit.  Overflow is not modelled: inputs stay finite."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    quantum = Fraction(2) ** (max(e, emin) - (prec - 1))
    n = a / quantum
    lo = n.numerator // n.denominator
    rest = n - lo
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def _bf16_of(q: Fraction) -> int:
    """bf16 bit pattern of a rational that is exactly a bf16 value."""
    f = np.float32(float(q))
    assert Fraction(float(f)) == q
    return int(np.array([f], np.float32).view(np.uint32)[0]) >> 16


def _chain(w_row, y_rows, h, fused=True, reverse=False):
    """bf16 bits of one output element: acc = 0; acc = fma(w_j, y_j[h], acc)
    over j (fused: one rounding per step; unfused: the product is rounded
    first), then one rounding to bf16."""
    acc = Fraction(0)
    order = range(len(w_row) - 1, -1, -1) if reverse else range(len(w_row))
    for j in order:
        prod = Fraction(float(w_row[j])) * Fraction(float(_f32(y_rows[j][h:h + 1])[0]))
        if not fused:
            prod = _round_rational(prod, 24)
        acc = _round_rational(prod + acc, 24)
    return _bf16_of(_round_rational(acc, 8))


def _adversarial_combine_case(seed: int, nt: int, K: int, H: int):
    """Rows and weights whose fp32 chains end on a binary32 rounding tie.

    Column 0 puts the accumulator on a bf16 midpoint m (w0 = m, y0 = a power
    of two per element).  One later column c adds the product w_c * y_c =
    (1 + eps) * ulp32(m) / 2 with 0 < eps < 2^-24: a fused step keeps eps and
    rounds m + ulp32/2 up, while a product rounded first loses it and the tie
    goes to even (m, whose last binary32 bit is 0).  The final bf16 rounding
    of m is itself a tie, so half of the elements end one bf16 ulp apart.
    The other columns have zero weights, which leave a fused chain exact.
    Reversed, the chain adds the rounded product to m last: the unfused
    result again."""
    rng = np.random.default_rng(seed)
    y = np.zeros((nt, K, H), np.uint16)
    w = np.zeros((nt, K), np.float32)
    for q in range(nt):
        while True:
            ex = int(rng.integers(-20, 20))
            mant = int(rng.integers(0x80, 0x100))
            m = (mant + 0.5) * 2.0 ** (ex - 7)  # a bf16 midpoint, 9 significant bits
            sgn = 1.0 if rng.random() < 0.5 else -1.0
            ulp32 = 2.0 ** (np.floor(np.log2(m)) - 23)
            yc = 1.0 + int(rng.integers(1, 128)) / 128.0  # bf16 with low bits
            half = ulp32 / 2
            wc = np.float32(half / yc)
            if Fraction(float(wc)) * Fraction(yc) <= Fraction(half):
                wc = np.nextafter(wc, np.float32(np.inf))
            eps = Fraction(float(wc)) * Fraction(yc) / Fraction(half) - 1
            if 0 < eps < Fraction(1, 2 ** 24):
                break
        c = int(rng.integers(1, K)) if K > 1 else 0
        assert K > 1
        w[q, 0] = np.float32(sgn * m)
        w[q, c] = np.float32(sgn * float(wc))
        for h in range(H):
            k2 = int(rng.integers(-3, 4))
            y[q, 0, h] = _torch_bf16_bits(np.array([2.0 ** k2], np.float32))[0]
            y[q, c, h] = _torch_bf16_bits(np.array([yc * 2.0 ** k2], np.float32))[0]
            for j in range(1, K):
                if j != c:
                    y[q, j, h] = _torch_bf16_bits(rng.standard_normal(1).astype(np.float32))[0]
    return y, w

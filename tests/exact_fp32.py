"""Exact-rational binary32 emulator of the contract's operation order (tiny inputs only).

Every value is a binary32 number held exactly in a Python float. Every operation is done
exactly with ``fractions.Fraction`` and then rounded once to binary32 with round to nearest,
ties to even, including the subnormal range; the sign of an exact zero follows IEEE 754.
It shares nothing with the C oracle or the HIP kernels: it pins that they really perform
the stated sequence of correctly rounded operations (no hidden contraction, a fused fma,
the stated tree).
"""

from fractions import Fraction
import math

_EMIN = -126
_PREC = 24


def _round(r: Fraction) -> float:
    if r == 0:
        return 0.0
    neg = r < 0
    a = -r if neg else r
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, _EMIN) - (_PREC - 1))
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = float(n * quantum)
    if val >= 2.0 ** 128:
        val = math.inf
    return -val if neg else val


def _neg0(x: float) -> bool:
    return math.copysign(1.0, x) < 0


def mul(x: float, y: float) -> float:
    if x == 0 or y == 0:
        return -0.0 if _neg0(x) != _neg0(y) else 0.0
    return _round(Fraction(x) * Fraction(y))


def add(x: float, y: float) -> float:
    r = Fraction(x) + Fraction(y)
    if r == 0:
        return -0.0 if (x == 0 and y == 0 and _neg0(x) and _neg0(y)) else 0.0
    return _round(r)


def sub(x: float, y: float) -> float:
    return add(x, -y)


def fma(x: float, y: float, z: float) -> float:
    p = Fraction(x) * Fraction(y)
    r = p + Fraction(z)
    if r == 0:
        p_neg = _neg0(x) != _neg0(y)
        both_zero = p == 0 and z == 0
        return -0.0 if (both_zero and p_neg and _neg0(z)) else 0.0
    return _round(r)


def to_f32(x) -> float:
    return _round(Fraction(float(x)))


def dot(x, y):
    """16 contiguous leaves (product, then fma ascending); pairwise sum of leaves."""
    d = len(x)
    m = d // 16
    leaves = []
    for l in range(16):
        acc = mul(x[l * m], y[l * m])
        for e in range(l * m + 1, l * m + m):
            acc = fma(x[e], y[e], acc)
        leaves.append(acc)
    width = 1
    while width < 16:
        for l in range(0, 16, 2 * width):
            leaves[l] = add(leaves[l], leaves[l + width])
        width *= 2
    return leaves[0]


def token(s, a, b, v_i, k, q):
    """One token on one state row; returns (new row, o_i)."""
    x = [mul(a, se) for se in s]
    u = dot(x, k)
    delta = mul(b, sub(v_i, u))
    s_new = [fma(delta, ke, xe) for ke, xe in zip(k, x)]
    return s_new, dot(s_new, q)

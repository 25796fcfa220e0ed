"""Exact-arithmetic brute force for tiny routing inputs.

Every fp32 operation is recomputed from its exact rational value
(fractions.Fraction) and rounded to nearest-even by hand, including signed
zeros, subnormals and overflow.  Nothing here calls the oracle or any float
library routine for the arithmetic being checked, so it pins the oracle from
outside.  Only finite inputs are supported.
"""
from __future__ import annotations

import itertools
import struct
from fractions import Fraction

F32_EMIN, F32_P = -126, 24      # fp32: min normal exponent, significand bits
BF16_EMIN, BF16_P = -126, 8


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def is_neg(v: float) -> bool:
    return bool(f32_bits(v) >> 31)


def _round_to(q: Fraction, emin: int, p: int, max_exp: int) -> float:
    """RNE of a nonzero rational to a binary format with p significand bits,
    min normal exponent emin, and values < 2^(max_exp+1)."""
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, emin) - (p - 1)
    scaled = a / (Fraction(2) ** quantum_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = Fraction(n) * Fraction(2) ** quantum_exp
    if r >= Fraction(2) ** (max_exp + 1):
        val = float("inf")
    else:
        val = float(r)
    if val == 0.0:
        val = 0.0
    return -val if neg else val


def rne_f32(q: Fraction) -> float:
    """fp32 RNE of a nonzero rational (a zero result keeps the sign of q)."""
    return _round_to(q, F32_EMIN, F32_P, 127)


def fma(a: float, b: float, c: float) -> float:
    """IEEE fp32 fused multiply-add, a*b+c with one rounding."""
    exact = Fraction(a) * Fraction(b) + Fraction(c)
    if exact != 0:
        return rne_f32(exact)
    prod_zero = a == 0.0 or b == 0.0
    if prod_zero and c == 0.0:
        prod_neg = is_neg(a) != is_neg(b)
        return -0.0 if (prod_neg and is_neg(c)) else 0.0
    return 0.0  # exact cancellation of nonzero terms rounds to +0


def add(a: float, b: float) -> float:
    """IEEE fp32 addition with RNE."""
    exact = Fraction(a) + Fraction(b)
    if exact != 0:
        return rne_f32(exact)
    if a == 0.0 and b == 0.0:
        return -0.0 if (is_neg(a) and is_neg(b)) else 0.0
    return 0.0


def tree(vals):
    """Level-by-level pairwise combination, odd last element carried up."""
    v = list(vals)
    while len(v) > 1:
        nxt = [add(v[2 * i], v[2 * i + 1]) for i in range(len(v) // 2)]
        if len(v) % 2:
            nxt.append(v[-1])
        v = nxt
    return v[0]


def canonical_dot(xrow, wcol, kblock: int) -> float:
    """fmaf chain from +0 per K-block, then the tree over block partials."""
    K = len(xrow)
    parts = []
    for k0 in range(0, K, kblock):
        p = 0.0
        for k in range(k0, min(k0 + kblock, K)):
            p = fma(float(xrow[k]), float(wcol[k]), p)
        parts.append(p)
    return tree(parts)


def sequential_dot(xrow, wcol) -> float:
    p = 0.0
    for a, b in zip(xrow, wcol):
        p = fma(float(a), float(b), p)
    return p


def bf16_bits(v: float) -> int:
    """bf16 RNE bit pattern of a finite fp32 value (or of +-inf)."""
    if v != v:
        return 0x7FC0
    if v in (float("inf"), float("-inf")):
        return 0xFF80 if v < 0 else 0x7F80
    if v == 0.0:
        return 0x8000 if is_neg(v) else 0x0000
    r = _round_to(Fraction(v), BF16_EMIN, BF16_P, 127)
    if r == 0.0:
        return 0x8000 if v < 0 else 0x0000
    return f32_bits(r) >> 16


def _all_finite_bf16_sorted():
    """Every finite bf16 value in increasing order, +0 and -0 merged."""
    vals = set()
    for b in range(0x10000):
        exp = (b >> 7) & 0xFF
        if exp == 0xFF:
            continue
        v = struct.unpack("<f", struct.pack("<I", b << 16))[0]
        vals.add(v)  # -0.0 == 0.0 collapse in the set
    return sorted(vals)


_BF16_SORTED = None
_BF16_INDEX = None


def bf16_steps(a_bits: int, b_bits: int) -> int:
    """Signed number of representable bf16 steps from b up to a, counted on the
    sorted list of all finite bf16 values (the sign-magnitude order's meaning,
    derived without its formula)."""
    global _BF16_SORTED, _BF16_INDEX
    if _BF16_SORTED is None:
        _BF16_SORTED = _all_finite_bf16_sorted()
        _BF16_INDEX = {v: i for i, v in enumerate(_BF16_SORTED)}
    va = struct.unpack("<f", struct.pack("<I", a_bits << 16))[0]
    vb = struct.unpack("<f", struct.pack("<I", b_bits << 16))[0]
    return _BF16_INDEX[va] - _BF16_INDEX[vb]


def select_topk_bruteforce(vals, k: int):
    """The unique k-subset S with: every selected i beats every rejected j
    (l_i > l_j, or l_i == l_j and i < j); then ranked by the same relation."""
    E = len(vals)

    def beats(i, j):
        return vals[i] > vals[j] or (vals[i] == vals[j] and i < j)

    found = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(beats(i, j) for i in S for j in rest):
            found.append(S)
    assert len(found) == 1, found
    S = list(found[0])
    ranked = []
    while S:
        top = [i for i in S if all(i == j or beats(i, j) for j in S)]
        assert len(top) == 1
        ranked.append(top[0])
        S.remove(top[0])
    return ranked

"""Exact-rational brute force for tiny shapes (test infrastructure only).

A second, independent statement of the quantiser and of the GEMM, written with
Python's fractions.Fraction so that no floating-point rounding happens except
where the format itself rounds (FP16 scale, integer codes).  Used to pin the C
oracle on tiny inputs.  Follows the same passages as oracle.c: per-group
asymmetric quantisation with scale = range / (2^b - 1) ("β-Informed Deployment
Features" page, CTX-TIER kernel details), codes packed b bits at a time along
K, dequant (q - z) * s, Y = X @ w^.
"""
from __future__ import annotations

from fractions import Fraction

FP16_MAX = Fraction(65504)


def floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); fix up
    if a >= Fraction(2) ** e:
        return e
    return e - 1


def round_half_even(a: Fraction) -> int:
    return round(a)  # Fraction.__round__ rounds half to even


def fp16_round(x: Fraction) -> Fraction | None:
    """Nearest FP16 value (ties to even); None when it overflows."""
    if x == 0:
        return Fraction(0)
    a = abs(x)
    E = max(floor_log2(a), -14)
    quantum = Fraction(2) ** (E - 10)
    r = round_half_even(a / quantum) * quantum
    if r > FP16_MAX:
        return None
    return r if x > 0 else -r


def quantise_group(ws: list[Fraction], bits: int):
    """(s, z, codes) of one group of exact weight values."""
    qmax = (1 << bits) - 1
    lo = min([Fraction(0)] + ws)
    hi = max([Fraction(0)] + ws)
    s = fp16_round((hi - lo) / qmax)
    if s is None:
        raise OverflowError("scale overflows FP16")
    if s == 0:
        s = Fraction(1)
    z = min(max(round_half_even(-lo / s), 0), qmax)
    q = [min(max(round_half_even(w / s) + z, 0), qmax) for w in ws]
    return s, z, q


def pack(W, bits: int, group: int = 128):
    """W: list of K rows of N floats.  Returns (s[n][g], z[n][g], q[n][k]) exact."""
    K, N = len(W), len(W[0])
    S = [[None] * (K // group) for _ in range(N)]
    Z = [[None] * (K // group) for _ in range(N)]
    Q = [[None] * K for _ in range(N)]
    for n in range(N):
        for g in range(K // group):
            ws = [Fraction(float(W[k][n])) for k in range(g * group, (g + 1) * group)]
            s, z, q = quantise_group(ws, bits)
            S[n][g], Z[n][g] = s, z
            Q[n][g * group:(g + 1) * group] = q
    return S, Z, Q


def words(Q_row: list[int], bits: int) -> list[int]:
    """Pack one row of codes into uint32 words: code j of a word (j = k mod 32/b)
    at bit 16*(j mod 2) + b*(j // 2), i.e. even codes in the low half-word and
    odd codes in the high half-word."""
    per = 32 // bits
    out = []
    for i in range(0, len(Q_row), per):
        w = 0
        for j, q in enumerate(Q_row[i:i + per]):
            w |= int(q) << (16 * (j % 2) + bits * (j // 2))
        out.append(w)
    return out


def gemm(X, S, Z, Q, group: int = 128):
    """Exact Y[m][n] = sum_k X[m][k] * (Q[n][k] - Z[n][g]) * S[n][g]."""
    M, K, N = len(X), len(X[0]), len(Q)
    Y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // group
                acc += Fraction(float(X[m][k])) * (Q[n][k] - Z[n][g]) * S[n][g]
            Y[m][n] = acc
    return Y

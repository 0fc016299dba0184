"""Exact-rational brute force of the FedAvg definition -- TEST INFRASTRUCTURE.

For tiny inputs only: every client value is turned into an exact Fraction, the
weighted mean over the senders of each parameter is formed exactly, and the
result is rounded once to the nearest binary32 value with ties to even.  This
is an independent second statement of the definition the C oracle follows (the
plain or contribution-weighted average of the Clara federated-learning page,
averaged per parameter over the clients that sent it as in the FLARE page's
client update contract), used to pin the C oracle.
"""

from fractions import Fraction
import math


def _exponent(a):
    """floor(log2(a)) for a positive Fraction."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); settle which side
    if e >= 0:
        if a < Fraction(2) ** e:
            e -= 1
    else:
        if a < Fraction(1, 2 ** (-e)):
            e -= 1
    return e


def round_fp32(q):
    """Nearest binary32 value to the exact rational q (ties to even), returned
    as a Python float (which holds it exactly).  Overflow gives +-inf."""
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    e = _exponent(a)
    e = max(e, -126)              # subnormal range has a fixed spacing 2^-149
    if e > 127:
        return -math.inf if neg else math.inf
    scale = Fraction(2) ** (e - 23)
    scaled = a / scale
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    r = Fraction(m) * scale
    if r >= Fraction(2) ** 128:
        return -math.inf if neg else math.inf
    f = float(r)
    return -f if neg else f


def weighted_average_exact(xs, n, mode="weights", base=None, sent=None):
    """xs: K lists of N finite floats (each exactly an fp32 or bf16 value);
    n: K non-negative ints; base: N floats or None; sent: None or K lists of
    N bools.  mode "deltas_zero_fill": a client that did not send a
    parameter counts as sending a zero delta, so the mean divides by the
    total weight of all clients.  Returns the N correctly rounded fp32
    results as floats."""
    K = len(xs)
    N = len(xs[0])
    S_all = sum(v for v in n if v > 0)
    out = []
    for i in range(N):
        s = Fraction(0)
        W = 0
        for k in range(K):
            if n[k] == 0 or (sent is not None and not sent[k][i]):
                continue
            s += n[k] * Fraction(xs[k][i])
            W += n[k]
        b = Fraction(base[i]) if base is not None else Fraction(0)
        if W == 0:
            if base is None:
                raise ValueError("parameter without sender and no base")
            out.append(round_fp32(b))
            continue
        v = s / (S_all if mode == "deltas_zero_fill" else W)
        out.append(round_fp32(v if mode == "weights" else b + v))
    return out

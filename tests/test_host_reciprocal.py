"""The kernels' reciprocal of a stored fp16 scale: the hardware reciprocal (within one
ulp) refined by one Newton step with fused multiply-adds, y + y*(1 - s*y).  Checked
here with exact rational arithmetic: for every significand an fp16 value can have
(at most 11 significant bits) and every start within two ulps of 1/s, the refined
value is the correctly rounded binary32 reciprocal, which is what the codec's
1/scale step asks for.  The exponent plays no part: 1/s is a normal binary32 for
every non-zero fp16 s, and so are the residual and the step."""
from fractions import Fraction as Fr


def _binade(x):
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fr(2) ** e > x:
        e -= 1
    while Fr(2) ** (e + 1) <= x:
        e += 1
    return e


def _rn32(x):
    """Round a rational to the nearest binary32 value, ties to even (normal range)."""
    if x == 0:
        return Fr(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    ulp = Fr(2) ** (_binade(x) - 23)
    q = x / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def _succ(y):
    return y + Fr(2) ** (_binade(y) - 23)


def _pred(y):
    e = _binade(y)
    return y - Fr(2) ** (e - 24 if y == Fr(2) ** e else e - 23)


def _refine(s, y):
    e = _rn32(1 - s * y)            # fma(-s, y, 1): one rounding
    return _rn32(y * e + y)         # fma(y, e, y): one rounding


def test_one_newton_step_gives_the_correctly_rounded_reciprocal():
    failures = []
    for m in range(1024, 2048):      # significands 1.f with 10 fraction bits
        s = Fr(m, 1024)
        exact = 1 / s
        r = _rn32(exact)
        lo = r if r <= exact else _pred(r)
        hi = r if r >= exact else _succ(r)
        for y in {lo, hi, _pred(lo), _succ(hi)}:
            if _refine(s, y) != r:
                failures.append((m, y))
    assert not failures, f"{len(failures)} cases, first {failures[:3]}"


def test_the_check_rejects_an_unfused_residual():
    """A plausible mistake, the residual 1 - s*y formed with a rounded product (no
    fused multiply-add), leaves starts that are one ulp off where they are: the same
    check finds them."""
    failures = 0
    for m in range(1024, 2048):
        s = Fr(m, 1024)
        exact = 1 / s
        r = _rn32(exact)
        y = _succ(r) if r >= exact else _pred(r)     # a faithful start on the far side
        e = _rn32(1 - _rn32(s * y))
        if _rn32(y * e + y) != r:
            failures += 1
    assert failures > 100

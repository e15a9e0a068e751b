"""The scalar map that one Newton-Schulz iteration applies to a singular value.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

An odd matrix polynomial acts on each singular value independently: if
X = P diag(sigma) Q^T, then a X + (b A + c A^2) X with A = X X^T equals
P diag(p(sigma)) Q^T with p(s) = a s + b s^3 + c s^5 [textbook: functions of
matrices via the SVD].  Composing k iterations gives p applied k times.  This
is the closed form that pins the matrix iteration in ``muon_ref``; it is
computed here on scalars only, with exact rational arithmetic, so it shares no
arithmetic path with the matrix products.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Sequence


def _q(x) -> Fraction:
    # Decimal literals such as 3.4445 are meant as the exact decimals, not as
    # their nearest binary64 values.
    return Fraction(str(x)) if isinstance(x, float) else Fraction(x)


def quintic_scalar_exact(sigma, steps: int, abc: Sequence) -> Fraction:
    """p composed `steps` times at sigma, p(s) = a s + b s^3 + c s^5, exactly."""
    a, b, c = (_q(t) for t in abc)
    s = _q(sigma)
    for _ in range(steps):
        s2 = s * s
        s = a * s + b * s2 * s + c * s2 * s2 * s
    return s


def quintic_scalar_float(sigma: float, steps: int, abc: Sequence[float]) -> float:
    """Same map in binary64 (for vectors of singular values)."""
    a, b, c = abc
    s = float(sigma)
    for _ in range(steps):
        s2 = s * s
        s = a * s + b * s2 * s + c * s2 * s2 * s
    return s

"""Clebsch-Gordan coefficients, the real basis and real coupling tensors (fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

* Complex CG: Racah's closed form (Condon-Shortley phase), evaluated with
  exact integer arithmetic and one final square root.
* Real basis: the unitary U^l that maps complex-basis components (index mu)
  to real components (index m, ordered m = -l..l).
* Real coupling of path (l1, l2, l3):
      z[m1, m2, m3] = sum U1[m1,mu1] U2[m2,mu2] conj(U3[m3,mu3]) <l1 mu1 l2 mu2|l3 mu3>
  and C = Re z when l1+l2+l3 is even, C = Im z when it is odd (the other part
  vanishes).  These are the equivariant bilinear maps that FlashCart
  (arXiv 2610.06409, section on spherical vs Cartesian products) notes are
  unique per admissible path up to normalisation; orthonormal normalisation is
  used: sum_{m1,m2} C[m1,m2,m3] C[m1,m2,m3'] = delta(m3, m3').
* Paths: every (l1, l2, l3) with l_k <= L_k and |l1-l2| <= l3 <= l1+l2, in
  lexicographic order (l1 outer, then l2, then l3), no parity filter.
"""
from __future__ import annotations

import math
from fractions import Fraction
from functools import lru_cache

import numpy as np


def paths(l_in: int, l_sh: int, l_out: int, natural: bool = False):
    """All triangle-allowed (l1, l2, l3), lexicographic; with natural=True only
    the natural-parity ones (l1 + l2 + l3 even: FlashCart, arXiv 2610.06409,
    background section, restricts its products to these)."""
    return [(l1, l2, l3)
            for l1 in range(l_in + 1)
            for l2 in range(l_sh + 1)
            for l3 in range(l_out + 1)
            if abs(l1 - l2) <= l3 <= l1 + l2 and (not natural or (l1 + l2 + l3) % 2 == 0)]


def _f(n: int) -> int:
    return math.factorial(n)


@lru_cache(maxsize=None)
def cg_complex(j1: int, m1: int, j2: int, m2: int, J: int, M: int) -> float:
    """<j1 m1 j2 m2 | J M> by Racah's closed form (Condon-Shortley)."""
    if M != m1 + m2:
        return 0.0
    if not (abs(j1 - j2) <= J <= j1 + j2):
        return 0.0
    if abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    pre = Fraction((2 * J + 1) * _f(J + j1 - j2) * _f(J - j1 + j2) * _f(j1 + j2 - J),
                   _f(j1 + j2 + J + 1))
    pre *= (_f(J + M) * _f(J - M) * _f(j1 - m1) * _f(j1 + m1)
            * _f(j2 - m2) * _f(j2 + m2))
    s = Fraction(0)
    for k in range(0, j1 + j2 + J + 2):
        args = (k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k,
                J - j2 + m1 + k, J - j1 - m2 + k)
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= _f(a)
        s += Fraction((-1) ** k, den)
    if s == 0:
        return 0.0
    # value = sign(s) * sqrt(pre * s^2), with pre * s^2 an exact rational
    r = pre * s * s
    return math.copysign(math.sqrt(r.numerator) / math.sqrt(r.denominator), float(s))


def real_basis(l: int) -> np.ndarray:
    """U^l[m, mu]: row m (real, -l..l), column mu (complex, -l..l)."""
    n = 2 * l + 1
    U = np.zeros((n, n), dtype=np.complex128)
    s = 1.0 / math.sqrt(2.0)
    for m in range(-l, l + 1):
        r = m + l
        if m > 0:
            U[r, m + l] = (-1) ** m * s
            U[r, -m + l] = s
        elif m == 0:
            U[r, l] = 1.0
        else:
            a = -m
            U[r, a + l] = -1j * (-1) ** a * s
            U[r, -a + l] = 1j * s
    return U


@lru_cache(maxsize=None)
def _real_cg_cached(l1: int, l2: int, l3: int) -> np.ndarray:
    cgc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for mu1 in range(-l1, l1 + 1):
        for mu2 in range(-l2, l2 + 1):
            mu3 = mu1 + mu2
            if abs(mu3) <= l3:
                cgc[mu1 + l1, mu2 + l2, mu3 + l3] = cg_complex(l1, mu1, l2, mu2, l3, mu3)
    U1, U2, U3 = real_basis(l1), real_basis(l2), real_basis(l3)
    z = np.einsum("ai,bj,ck,ijk->abc", U1, U2, U3.conj(), cgc)
    c = z.real if (l1 + l2 + l3) % 2 == 0 else z.imag
    # Entries that cancel exactly in the transform leave round-off of order
    # 1e-17; make them exact zeros so the sparsity pattern is exact.
    c = np.where(np.abs(c) < 1e-13, 0.0, c)
    c.setflags(write=False)
    return c


def real_cg(l1: int, l2: int, l3: int) -> np.ndarray:
    """Real coupling tensor C[m1, m2, m3] of path (l1, l2, l3), orthonormal."""
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        raise ValueError(f"path ({l1},{l2},{l3}) violates the triangle rule")
    return np.array(_real_cg_cached(l1, l2, l3))


def complex_part_residual(l1: int, l2: int, l3: int) -> float:
    """Largest |part| of z that the parity rule discards (must vanish)."""
    cgc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for mu1 in range(-l1, l1 + 1):
        for mu2 in range(-l2, l2 + 1):
            mu3 = mu1 + mu2
            if abs(mu3) <= l3:
                cgc[mu1 + l1, mu2 + l2, mu3 + l3] = cg_complex(l1, mu1, l2, mu2, l3, mu3)
    U1, U2, U3 = real_basis(l1), real_basis(l2), real_basis(l3)
    z = np.einsum("ai,bj,ck,ijk->abc", U1, U2, U3.conj(), cgc)
    other = z.imag if (l1 + l2 + l3) % 2 == 0 else z.real
    return float(np.abs(other).max())


def comp_index(l: int, m: int) -> int:
    """Flat component index d(l, m) = l^2 + l + m."""
    return l * l + l + m


def dim(L: int) -> int:
    return (L + 1) ** 2

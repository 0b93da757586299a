"""Real spherical harmonics and their gradient (fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Legendre closed form, orthonormal on the sphere, no Condon-Shortley phase:

    Y_lm(r) = N_lm * A_m(x, y) * P_l^(|m|)(z),   r = v / |v|
    N_lm = sqrt((2l+1)/(4 pi) * (l-|m|)!/(l+|m|)!) * (sqrt 2 if m != 0)
    A_m  = Re (x+iy)^m (m > 0),  1 (m = 0),  Im (x+iy)^|m| (m < 0)

where P_l^(k) is the k-th derivative of the Legendre polynomial P_l.  This is
the real form U^l applied to the complex Condon-Shortley harmonics, with
components ordered m = -l..l (so l = 1 is sqrt(3/4pi) * (y, z, x)).  It is a
polynomial in (x, y, z), so the gradient below is exact.

A zero vector has no direction; by convention r := 0 gives Y_00 = 1/sqrt(4 pi),
every Y_{l>=1} = 0, and a zero gradient.
"""
from __future__ import annotations

import math

import numpy as np
from numpy.polynomial import legendre as npleg


def _norm(l: int, m: int) -> float:
    a = abs(m)
    n = math.sqrt((2 * l + 1) / (4 * math.pi) * math.factorial(l - a) / math.factorial(l + a))
    return n * (math.sqrt(2.0) if m != 0 else 1.0)


def _legendre_deriv(l: int, k: int):
    """Coefficients (power basis, ascending) of d^k/dz^k P_l(z)."""
    c = np.zeros(l + 1)
    c[l] = 1.0
    p = npleg.leg2poly(c)
    return np.polynomial.polynomial.polyder(p, k) if k > 0 else p


def _A(m: int, x, y):
    w = (x + 1j * y) ** abs(m)
    if m > 0:
        return w.real
    if m < 0:
        return w.imag
    return np.ones_like(x)


def _dA(m: int, x, y):
    """(dA/dx, dA/dy)."""
    a = abs(m)
    if a == 0:
        z = np.zeros_like(x)
        return z, z
    w = a * (x + 1j * y) ** (a - 1)   # d/dx (x+iy)^a;  d/dy = i * that
    if m > 0:
        return w.real, (1j * w).real
    return w.imag, (1j * w).imag


def real_sh(L: int, vec) -> np.ndarray:
    """Y[..., (L+1)^2] of the directions of `vec` (any length, fp64)."""
    v = np.asarray(vec, dtype=np.float64)
    n = np.linalg.norm(v, axis=-1)
    zero = n == 0
    r = v / np.where(zero, 1.0, n)[..., None]
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    out = np.zeros(v.shape[:-1] + ((L + 1) ** 2,))
    for l in range(L + 1):
        for m in range(-l, l + 1):
            P = np.polynomial.polynomial.polyval(z, _legendre_deriv(l, abs(m)))
            out[..., l * l + l + m] = _norm(l, m) * _A(m, x, y) * P
    out[zero] = 0.0
    out[zero, 0] = 1.0 / math.sqrt(4 * math.pi)
    return out


def real_sh_grad(L: int, vec) -> np.ndarray:
    """dY/dvec [..., (L+1)^2, 3] for Y(vec/|vec|) (zero rows at vec = 0)."""
    v = np.asarray(vec, dtype=np.float64)
    n = np.linalg.norm(v, axis=-1)
    zero = n == 0
    ns = np.where(zero, 1.0, n)
    r = v / ns[..., None]
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    grad_r = np.zeros(v.shape[:-1] + ((L + 1) ** 2, 3))
    for l in range(L + 1):
        for m in range(-l, l + 1):
            cP = _legendre_deriv(l, abs(m))
            P = np.polynomial.polynomial.polyval(z, cP)
            dP = np.polynomial.polynomial.polyval(z, np.polynomial.polynomial.polyder(cP))
            A = _A(m, x, y)
            dAx, dAy = _dA(m, x, y)
            k = l * l + l + m
            N = _norm(l, m)
            grad_r[..., k, 0] = N * dAx * P
            grad_r[..., k, 1] = N * dAy * P
            grad_r[..., k, 2] = N * A * dP
    # chain rule through r = v/|v|:  dr/dv = (I - r r^T) / |v|
    proj = np.eye(3) - r[..., :, None] * r[..., None, :]
    g = np.einsum("...kj,...ji->...ki", grad_r, proj) / ns[..., None, None]
    g[zero] = 0.0
    return g


def vec_grad_from_sh_grad(L: int, vec, dY) -> np.ndarray:
    """dvec[e] = J(vec_e)^T dY[e], with J = dY/dvec."""
    J = real_sh_grad(L, vec)
    return np.einsum("...k,...ki->...i", np.asarray(dY, dtype=np.float64), J)


def _d2A(m: int, x, y):
    """(d2A/dx2, d2A/dxdy, d2A/dy2)."""
    a = abs(m)
    if a < 2:
        z = np.zeros_like(x)
        return z, z, z
    w = a * (a - 1) * (x + 1j * y) ** (a - 2)   # d2/dx2 (x+iy)^a; d2/dxdy = i w; d2/dy2 = -w
    part = (lambda c: c.real) if m > 0 else (lambda c: c.imag)
    return part(w), part(1j * w), part(-w)


def _poly_derivs(L: int, r):
    """Gradient [..., K, 3] and Hessian [..., K, 3, 3] in r of the polynomial
    form of every Y_k (r a free vector, not constrained to the sphere)."""
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    K = (L + 1) ** 2
    g = np.zeros(r.shape[:-1] + (K, 3))
    h = np.zeros(r.shape[:-1] + (K, 3, 3))
    pp = np.polynomial.polynomial
    for l in range(L + 1):
        for m in range(-l, l + 1):
            k = l * l + l + m
            N = _norm(l, m)
            cP = _legendre_deriv(l, abs(m))
            P, dP, d2P = (pp.polyval(z, c) for c in (cP, pp.polyder(cP), pp.polyder(cP, 2)))
            A = _A(m, x, y)
            Ax, Ay = _dA(m, x, y)
            Axx, Axy, Ayy = _d2A(m, x, y)
            g[..., k, 0], g[..., k, 1], g[..., k, 2] = N * Ax * P, N * Ay * P, N * A * dP
            h[..., k, 0, 0] = N * Axx * P
            h[..., k, 1, 1] = N * Ayy * P
            h[..., k, 2, 2] = N * A * d2P
            h[..., k, 0, 1] = h[..., k, 1, 0] = N * Axy * P
            h[..., k, 0, 2] = h[..., k, 2, 0] = N * Ax * dP
            h[..., k, 1, 2] = h[..., k, 2, 1] = N * Ay * dP
    return g, h


def real_sh_hess(L: int, vec) -> np.ndarray:
    """d2Y/dvec2 [..., (L+1)^2, 3, 3] for Y(vec/|vec|) (zero at vec = 0), by the
    chain rule through r = v/|v|: with R = dr/dv = (I - r r^T)/|v|,
    d2Y/dv_i dv_j = sum_ab P_ab R_ai R_bj + sum_a P_a dR_aj/dv_i, and
    dR_aj/dv_i = -(R_ai r_j + r_a R_ji)/|v| - (delta_aj - r_a r_j) r_i/|v|^2."""
    v = np.asarray(vec, dtype=np.float64)
    n = np.linalg.norm(v, axis=-1)
    zero = n == 0
    ns = np.where(zero, 1.0, n)
    r = v / ns[..., None]
    g, h = _poly_derivs(L, r)
    eye = np.eye(3)
    R = (eye - r[..., :, None] * r[..., None, :]) / ns[..., None, None]
    # dR[..., a, j, i] = d R_aj / d v_i
    dR = (-(np.einsum("...ai,...j->...aji", R, r) + np.einsum("...a,...ji->...aji", r, R)) / ns[..., None, None, None]
          - np.einsum("...aj,...i->...aji", eye - r[..., :, None] * r[..., None, :], r) / (ns ** 2)[..., None, None, None])
    H = np.einsum("...kab,...ai,...bj->...kij", h, R, R) + np.einsum("...ka,...aji->...kij", g, dR)
    H[zero] = 0.0
    return H


def real_sh_jvp(L: int, vec, a) -> np.ndarray:
    """aY[e] = J(vec_e) a[e]: the change of Y along a change a of the vector."""
    return np.einsum("...ki,...i->...k", real_sh_grad(L, vec), np.asarray(a, dtype=np.float64))


def vec_hess_term(L: int, vec, dY, a) -> np.ndarray:
    """d/dvec of sum_k dY_k (J(vec) a)_k with dY and a held fixed:
    sum_k dY_k H_k a, H_k the Hessian of Y_k(vec/|vec|)."""
    H = real_sh_hess(L, vec)
    return np.einsum("...k,...kij,...j->...i", np.asarray(dY, dtype=np.float64), H, np.asarray(a, dtype=np.float64))

"""Real Wigner-D matrices for equivariance checks (fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Rotation R = Rz(alpha) Ry(beta) Rz(gamma) (active, ZYZ Euler angles).  The
complex matrix is D^l_{m'm} = exp(-i m' alpha) d^l_{m'm}(beta) exp(-i m gamma)
with Wigner's closed form for the small-d matrix.  Since
(R Y_lm)(r) = Y_lm(R^-1 r) = sum_m' D_{m'm} Y_lm'(r), the component vector
obeys Y(R r) = conj(D(R)) Y(r); in the real basis Y_real = U Y_complex this
becomes Y_real(R r) = D_real(R) Y_real(r) with D_real = U conj(D) U^dagger.
"""
from __future__ import annotations

import math

import numpy as np

from .cg import real_basis


def small_d(j: int, beta: float) -> np.ndarray:
    """Wigner small-d matrix d^j_{m'm}(beta), rows m', columns m."""
    n = 2 * j + 1
    d = np.zeros((n, n))
    c, s = math.cos(beta / 2), math.sin(beta / 2)
    f = math.factorial
    for mp in range(-j, j + 1):
        for m in range(-j, j + 1):
            pre = math.sqrt(f(j + m) * f(j - m) * f(j + mp) * f(j - mp))
            tot = 0.0
            for k in range(0, 2 * j + 1):
                a = (j + m - k, k, j - k - mp, k - m + mp)
                if min(a) < 0:
                    continue
                tot += ((-1) ** (k - m + mp) / (f(a[0]) * f(a[1]) * f(a[2]) * f(a[3]))
                        * c ** (2 * j - 2 * k + m - mp) * s ** (2 * k - m + mp))
            d[mp + j, m + j] = pre * tot
    return d


def complex_D(j: int, alpha: float, beta: float, gamma: float) -> np.ndarray:
    ms = np.arange(-j, j + 1)
    return (np.exp(-1j * ms * alpha)[:, None] * small_d(j, beta)
            * np.exp(-1j * ms * gamma)[None, :])


def real_D(l: int, alpha: float, beta: float, gamma: float) -> np.ndarray:
    """Real representation matrix with Y_real(R r) = D Y_real(r)."""
    U = real_basis(l)
    D = U @ complex_D(l, alpha, beta, gamma).conj() @ U.conj().T
    if np.abs(D.imag).max() > 1e-12:
        raise AssertionError("real Wigner-D has an imaginary part")
    return D.real


def rotation_matrix(alpha: float, beta: float, gamma: float) -> np.ndarray:
    def rz(t):
        return np.array([[math.cos(t), -math.sin(t), 0.0],
                         [math.sin(t), math.cos(t), 0.0],
                         [0.0, 0.0, 1.0]])

    def ry(t):
        return np.array([[math.cos(t), 0.0, math.sin(t)],
                         [0.0, 1.0, 0.0],
                         [-math.sin(t), 0.0, math.cos(t)]])
    return rz(alpha) @ ry(beta) @ rz(gamma)


def block_D(L: int, alpha: float, beta: float, gamma: float) -> np.ndarray:
    """Block-diagonal D over l = 0..L, acting on [(L+1)^2] component vectors."""
    n = (L + 1) ** 2
    D = np.zeros((n, n))
    for l in range(L + 1):
        D[l * l:(l + 1) ** 2, l * l:(l + 1) ** 2] = real_D(l, alpha, beta, gamma)
    return D


def random_angles(rng: np.random.Generator):
    """Euler angles of a rotation drawn uniformly (Haar) from SO(3)."""
    alpha = rng.uniform(0, 2 * math.pi)
    gamma = rng.uniform(0, 2 * math.pi)
    beta = math.acos(rng.uniform(-1.0, 1.0))
    return alpha, beta, gamma

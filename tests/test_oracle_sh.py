"""Pins of the oracle's real spherical harmonics, their gradient and the
Wigner-D matrices used by the equivariance tests."""
import math

import numpy as np
import pytest
import scipy.special as sps

from oracle import cg, sh, wigner


def _dirs(n, seed):
    v = np.random.default_rng(seed).standard_normal((n, 3))
    return v


def test_matches_scipy_complex_harmonics():
    v = _dirs(64, 0)
    r = v / np.linalg.norm(v, axis=1, keepdims=True)
    th, ph = np.arccos(r[:, 2]), np.arctan2(r[:, 1], r[:, 0])
    Y = sh.real_sh(3, v)
    for l in range(4):
        Yc = np.stack([sps.sph_harm_y(l, mu, th, ph) for mu in range(-l, l + 1)], -1)
        Yr = (cg.real_basis(l) @ Yc.T).T
        assert np.abs(Yr.imag).max() < 1e-14
        np.testing.assert_allclose(Yr.real, Y[:, l * l:(l + 1) ** 2], atol=1e-14)


def test_explicit_low_degree_forms():
    v = _dirs(32, 1)
    r = v / np.linalg.norm(v, axis=1, keepdims=True)
    x, y, z = r.T
    Y = sh.real_sh(2, v)
    pi = math.pi
    np.testing.assert_allclose(Y[:, 0], 1 / math.sqrt(4 * pi), atol=1e-15)
    np.testing.assert_allclose(Y[:, 1:4], math.sqrt(3 / (4 * pi)) * np.stack([y, z, x], 1), atol=1e-15)
    np.testing.assert_allclose(Y[:, 4], math.sqrt(15 / (4 * pi)) * x * y, atol=1e-15)
    np.testing.assert_allclose(Y[:, 5], math.sqrt(15 / (4 * pi)) * y * z, atol=1e-15)
    np.testing.assert_allclose(Y[:, 6], math.sqrt(5 / (16 * pi)) * (3 * z * z - 1), atol=1e-15)
    np.testing.assert_allclose(Y[:, 7], math.sqrt(15 / (4 * pi)) * x * z, atol=1e-15)
    np.testing.assert_allclose(Y[:, 8], math.sqrt(15 / (16 * pi)) * (x * x - y * y), atol=1e-15)


def test_quadrature_orthonormality():
    """Gauss-Legendre in z times a uniform grid in phi integrates degree <= 2L exactly."""
    L = 3
    zq, wz = np.polynomial.legendre.leggauss(L + 2)
    nphi = 2 * L + 3
    phi = 2 * math.pi * np.arange(nphi) / nphi
    Z, PH = np.meshgrid(zq, phi, indexing="ij")
    W = np.outer(wz, np.full(nphi, 2 * math.pi / nphi)).ravel()
    s = np.sqrt(1 - Z ** 2)
    v = np.stack([s * np.cos(PH), s * np.sin(PH), Z], -1).reshape(-1, 3)
    Y = sh.real_sh(L, v)
    gram = np.einsum("q,qa,qb->ab", W, Y, Y)
    np.testing.assert_allclose(gram, np.eye((L + 1) ** 2), atol=1e-13)


def test_addition_theorem():
    Y = sh.real_sh(3, _dirs(40, 2))
    for l in range(4):
        np.testing.assert_allclose((Y[:, l * l:(l + 1) ** 2] ** 2).sum(1),
                                   (2 * l + 1) / (4 * math.pi), atol=1e-14)


def test_scale_invariance_and_zero_vector():
    v = _dirs(10, 3)
    np.testing.assert_allclose(sh.real_sh(3, 3.7 * v), sh.real_sh(3, v), atol=1e-15)
    Y0 = sh.real_sh(3, np.zeros((2, 3)))
    ref = np.zeros((2, 16))
    ref[:, 0] = 1 / math.sqrt(4 * math.pi)
    np.testing.assert_array_equal(Y0, ref)
    assert not sh.real_sh_grad(3, np.zeros((1, 3))).any()


def test_gradient_finite_differences():
    v = _dirs(12, 4) * 1.3
    J = sh.real_sh_grad(3, v)
    h = 1e-5
    for i in range(3):
        e = np.zeros(3)
        e[i] = h
        fd = (sh.real_sh(3, v + e) - sh.real_sh(3, v - e)) / (2 * h)
        np.testing.assert_allclose(J[..., i], fd, atol=1e-9)


def test_gradient_is_tangent():
    """Y depends only on the direction, so J(v) v = 0."""
    v = _dirs(12, 5)
    J = sh.real_sh_grad(3, v)
    np.testing.assert_allclose(np.einsum("eki,ei->ek", J, v), 0.0, atol=1e-13)


def test_wigner_D_properties():
    rng = np.random.default_rng(9)
    a1, a2 = wigner.random_angles(rng), wigner.random_angles(rng)
    R1, R2 = wigner.rotation_matrix(*a1), wigner.rotation_matrix(*a2)
    np.testing.assert_allclose(R1 @ R1.T, np.eye(3), atol=1e-14)
    # l = 1 block is the rotation matrix in (y, z, x) order
    perm = [1, 2, 0]
    np.testing.assert_allclose(wigner.real_D(1, *a1), R1[np.ix_(perm, perm)], atol=1e-13)
    v = rng.standard_normal((50, 3))
    for l in range(4):
        D1, D2 = wigner.real_D(l, *a1), wigner.real_D(l, *a2)
        np.testing.assert_allclose(D1 @ D1.T, np.eye(2 * l + 1), atol=1e-13)
        # Y(R v) = D Y(v), and D agrees with a least-squares fit from samples
        Yv = sh.real_sh(l, v)[:, l * l:]
        YRv = sh.real_sh(l, v @ R1.T)[:, l * l:]
        np.testing.assert_allclose(YRv, Yv @ D1.T, atol=1e-13)
        Dfit, *_ = np.linalg.lstsq(Yv, YRv, rcond=None)
        np.testing.assert_allclose(Dfit.T, D1, atol=1e-11)
        # homomorphism: D(R1 R2) = D(R1) D(R2)
        Y12 = sh.real_sh(l, v @ (R1 @ R2).T)[:, l * l:]
        np.testing.assert_allclose(Y12, Yv @ (D1 @ D2).T, atol=1e-12)

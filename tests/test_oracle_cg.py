"""Pins of the oracle's Clebsch-Gordan and real coupling tensors.

Each check is fixed by something other than the oracle's own formula: sympy's
exact CG, orthonormality, textbook special cases, the Gaunt integral identity,
the Cartesian forms of the l=1 couplings, Wigner-D equivariance, and a real
basis fitted from scipy's complex harmonics instead of the typed U.
"""
import math

import numpy as np
import pytest
import scipy.special as sps
from sympy.physics.wigner import clebsch_gordan

from oracle import cg, sh, wigner

L3_PATHS = cg.paths(3, 3, 3)


def test_path_counts_and_order():
    assert cg.paths(1, 1, 1) == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 1, 1)]
    assert [len(cg.paths(L, L, L)) for L in (0, 1, 2, 3)] == [1, 5, 15, 34]
    assert L3_PATHS == sorted(L3_PATHS)
    # mixed degrees: scalar input features, l<=3 harmonics and outputs
    assert cg.paths(0, 3, 3) == [(0, l, l) for l in range(4)]


def test_nonzero_counts():
    nnz = [sum(int((cg.real_cg(*p) != 0).sum()) for p in cg.paths(L, L, L)) for L in (1, 2, 3)]
    assert nnz == [16, 137, 611]


@pytest.mark.parametrize("j1,j2", [(a, b) for a in range(4) for b in range(4)])
def test_complex_cg_matches_sympy(j1, j2):
    for J in range(abs(j1 - j2), j1 + j2 + 1):
        for m1 in range(-j1, j1 + 1):
            for m2 in range(-j2, j2 + 1):
                M = m1 + m2
                if abs(M) > J:
                    continue
                ref = float(clebsch_gordan(j1, j2, J, m1, m2, M))
                assert abs(cg.cg_complex(j1, m1, j2, m2, J, M) - ref) < 1e-14


def test_complex_cg_orthonormal():
    for j1 in range(4):
        for j2 in range(4):
            rows = []
            for J in range(abs(j1 - j2), j1 + j2 + 1):
                for M in range(-J, J + 1):
                    rows.append([cg.cg_complex(j1, m1, j2, m2, J, M)
                                 for m1 in range(-j1, j1 + 1) for m2 in range(-j2, j2 + 1)])
            A = np.array(rows)
            n = (2 * j1 + 1) * (2 * j2 + 1)
            assert A.shape == (n, n)
            np.testing.assert_allclose(A @ A.T, np.eye(n), atol=1e-14)


@pytest.mark.parametrize("p", L3_PATHS)
def test_real_cg_orthonormal_and_real(p):
    C = cg.real_cg(*p)
    n3 = C.shape[2]
    G = np.einsum("abk,abq->kq", C, C)
    np.testing.assert_allclose(G, np.eye(n3), atol=1e-14)
    assert cg.complex_part_residual(*p) < 1e-12


def test_special_cases():
    for l in range(4):
        n = 2 * l + 1
        np.testing.assert_allclose(cg.real_cg(l, 0, l)[:, 0, :], np.eye(n), atol=1e-15)
        np.testing.assert_allclose(cg.real_cg(0, l, l)[0, :, :], np.eye(n), atol=1e-15)
    np.testing.assert_allclose(cg.real_cg(1, 1, 0)[:, :, 0], -np.eye(3) / math.sqrt(3), atol=1e-15)


def test_l1_cartesian_forms():
    """(1,1->1) is -(a x b)/sqrt(2) and (1,1->0) is -(a.b)/sqrt(3); l=1 <-> (y,z,x)."""
    rng = np.random.default_rng(7)
    perm = [1, 2, 0]
    for _ in range(5):
        a, b = rng.standard_normal(3), rng.standard_normal(3)
        out1 = np.einsum("ijk,i,j->k", cg.real_cg(1, 1, 1), a[perm], b[perm])
        np.testing.assert_allclose(out1, -np.cross(a, b)[perm] / math.sqrt(2), atol=1e-14)
        out0 = np.einsum("ijk,i,j->k", cg.real_cg(1, 1, 0), a[perm], b[perm])
        np.testing.assert_allclose(out0, [-(a @ b) / math.sqrt(3)], atol=1e-14)


@pytest.mark.parametrize("p", L3_PATHS)
def test_gaunt_identity(p):
    """Even paths: C(Y_l1(r), Y_l2(r)) = sqrt((2l1+1)(2l2+1)/(4pi(2l3+1))) <l1 0 l2 0|l3 0> Y_l3(r).
    Odd paths: the same contraction vanishes identically."""
    l1, l2, l3 = p
    rng = np.random.default_rng(11)
    v = rng.standard_normal((16, 3))
    Y = sh.real_sh(3, v)
    y1, y2, y3 = (Y[:, l * l:(l + 1) ** 2] for l in (l1, l2, l3))
    lhs = np.einsum("abk,ea,eb->ek", cg.real_cg(*p), y1, y2)
    if (l1 + l2 + l3) % 2:
        np.testing.assert_allclose(lhs, 0.0, atol=1e-14)
    else:
        k = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (4 * math.pi * (2 * l3 + 1)))
        k *= float(clebsch_gordan(l1, l2, l3, 0, 0, 0))
        np.testing.assert_allclose(lhs, k * y3, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_equivariance_all_paths(seed):
    rng = np.random.default_rng(seed)
    ang = wigner.random_angles(rng)
    Ds = [wigner.real_D(l, *ang) for l in range(4)]
    for (l1, l2, l3) in L3_PATHS:
        C = cg.real_cg(l1, l2, l3)
        a = rng.standard_normal(2 * l1 + 1)
        b = rng.standard_normal(2 * l2 + 1)
        lhs = np.einsum("abk,a,b->k", C, Ds[l1] @ a, Ds[l2] @ b)
        rhs = Ds[l3] @ np.einsum("abk,a,b->k", C, a, b)
        np.testing.assert_allclose(lhs, rhs, atol=1e-13)


def _fitted_real_basis(l, rng):
    """U fitted by least squares from scipy's complex harmonics to the real Y."""
    v = rng.standard_normal((200, 3))
    r = v / np.linalg.norm(v, axis=1, keepdims=True)
    th, ph = np.arccos(r[:, 2]), np.arctan2(r[:, 1], r[:, 0])
    Yc = np.stack([sps.sph_harm_y(l, mu, th, ph) for mu in range(-l, l + 1)], -1)
    Yr = sh.real_sh(l, v)[:, l * l:(l + 1) ** 2]
    U, *_ = np.linalg.lstsq(Yc, Yr.astype(np.complex128), rcond=None)
    return U.T  # Yr = Yc @ U  ->  Yr^T = U^T Yc^T


def test_real_cg_from_fitted_basis_and_sympy():
    """Rebuild every real coupling from sympy's exact CG and a basis fitted to the
    real harmonics; agrees with the oracle's tensors, odd-path signs included."""
    rng = np.random.default_rng(5)
    Us = [_fitted_real_basis(l, rng) for l in range(4)]
    for l in range(4):
        np.testing.assert_allclose(Us[l], cg.real_basis(l), atol=1e-12)
    for (l1, l2, l3) in L3_PATHS:
        cgc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                if abs(m1 + m2) <= l3:
                    cgc[m1 + l1, m2 + l2, m1 + m2 + l3] = float(
                        clebsch_gordan(l1, l2, l3, m1, m2, m1 + m2))
        z = np.einsum("ai,bj,ck,ijk->abc", Us[l1], Us[l2], Us[l3].conj(), cgc)
        ref = z.real if (l1 + l2 + l3) % 2 == 0 else z.imag
        np.testing.assert_allclose(cg.real_cg(l1, l2, l3), ref, atol=1e-12)


def test_triangle_rule_enforced():
    with pytest.raises(ValueError):
        cg.real_cg(0, 1, 2)

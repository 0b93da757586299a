"""Planted mistakes in the oracle must be caught by its pins.

Each test plants one plausible error (a flipped sign, a dropped factor, a
transposed operand, a wrong gather index, a dropped term) into the oracle on
the CPU and checks that the corresponding pin check fails.
"""
import math

import numpy as np
import pytest
import scipy.special as sps
from sympy.physics.wigner import clebsch_gordan

from oracle import cg, convtp as ct, graph, sh


def _fitted_basis_residual(real_cg_fn):
    """Largest deviation of real_cg_fn from sympy CG + a fitted real basis."""
    rng = np.random.default_rng(5)
    worst = 0.0
    Us = []
    for l in range(4):
        v = rng.standard_normal((200, 3))
        r = v / np.linalg.norm(v, axis=1, keepdims=True)
        th, ph = np.arccos(r[:, 2]), np.arctan2(r[:, 1], r[:, 0])
        Yc = np.stack([sps.sph_harm_y(l, mu, th, ph) for mu in range(-l, l + 1)], -1)
        U, *_ = np.linalg.lstsq(Yc, sh.real_sh(l, v)[:, l * l:].astype(complex), rcond=None)
        Us.append(U.T)
    for (l1, l2, l3) in cg.paths(3, 3, 3):
        cgc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                if abs(m1 + m2) <= l3:
                    cgc[m1 + l1, m2 + l2, m1 + m2 + l3] = float(
                        clebsch_gordan(l1, l2, l3, m1, m2, m1 + m2))
        z = np.einsum("ai,bj,ck,ijk->abc", Us[l1], Us[l2], Us[l3].conj(), cgc)
        ref = z.real if (l1 + l2 + l3) % 2 == 0 else z.imag
        worst = max(worst, float(np.abs(real_cg_fn(l1, l2, l3) - ref).max()))
    return worst


def test_flipped_odd_path_sign_is_caught():
    assert _fitted_basis_residual(cg.real_cg) < 1e-12

    def planted(l1, l2, l3):
        c = cg.real_cg(l1, l2, l3)
        return -c if (l1, l2, l3) == (2, 1, 2) else c
    assert _fitted_basis_residual(planted) > 0.1


def test_transposed_coupling_is_caught_by_cross_product_pin():
    a, b = np.array([0.3, -1.2, 0.7]), np.array([1.1, 0.4, -0.5])
    perm = [1, 2, 0]
    C = cg.real_cg(1, 1, 1)
    good = np.einsum("ijk,i,j->k", C, a[perm], b[perm])
    bad = np.einsum("ijk,i,j->k", C.transpose(2, 1, 0), a[perm], b[perm])
    ref = -np.cross(a, b)[perm] / math.sqrt(2)
    assert np.abs(good - ref).max() < 1e-14
    assert np.abs(bad - ref).max() > 0.1


def test_dropped_sqrt2_in_harmonics_is_caught_by_quadrature(monkeypatch):
    def gram():
        zq, wz = np.polynomial.legendre.leggauss(5)
        phi = 2 * math.pi * np.arange(9) / 9
        Z, PH = np.meshgrid(zq, phi, indexing="ij")
        W = np.outer(wz, np.full(9, 2 * math.pi / 9)).ravel()
        s = np.sqrt(1 - Z ** 2)
        v = np.stack([s * np.cos(PH), s * np.sin(PH), Z], -1).reshape(-1, 3)
        Y = sh.real_sh(3, v)
        return np.abs(np.einsum("q,qa,qb->ab", W, Y, Y) - np.eye(16)).max()
    assert gram() < 1e-13
    orig = sh._norm
    monkeypatch.setattr(sh, "_norm", lambda l, m: orig(l, m) / (math.sqrt(2) if m else 1.0))
    assert gram() > 0.1


def _small(L=2, seed=0):
    rng = np.random.default_rng(seed)
    prob = ct.Problem(L, L, L)
    n, e, c = 8, 30, 3
    recv = np.sort(rng.integers(0, n, size=e))
    row_ptr = graph.row_ptr_from_receivers(recv, n)
    senders = rng.integers(0, n, size=e).astype(np.int32)
    x = rng.standard_normal((n, prob.D1, c)).astype(np.float32)
    w = rng.standard_normal((e, prob.P, c)).astype(np.float32)
    G = rng.standard_normal((n, prob.D3, c)).astype(np.float32)
    Y = sh.real_sh(L, rng.standard_normal((e, 3)))
    return prob, row_ptr, senders, x, w, G, Y


def test_wrong_gather_index_is_caught_by_brute_force(oracle_lib):
    prob, row_ptr, senders, x, w, G, Y = _small()
    c_loop = ct.fwd(prob, x, Y, w, row_ptr, senders)
    assert np.abs(c_loop - ct.materialised_fwd(prob, x, Y, w, row_ptr, senders)).max() < 1e-12
    recv = graph.receivers_of(row_ptr)       # planted: gather x at the receiver
    bad = ct.materialised_fwd(prob, x, Y, w, row_ptr, recv)
    assert np.abs(c_loop - bad).max() > 1e-3


def test_dropped_dw_path_is_caught_by_adjoint_identity():
    prob, row_ptr, senders, x, w, G, Y = _small(L=3, seed=1)
    out = ct.materialised_fwd(prob, x, Y, w, row_ptr, senders)
    dx, dw, dY = ct.materialised_bwd(prob, x, Y, w, G, row_ptr, senders)
    ref = (G.astype(np.float64) * out).sum()
    assert abs((dw * w).sum() - ref) < 1e-10
    dw_bad = dw.copy()
    dw_bad[:, 17, :] = 0.0                   # planted: one path's weight gradient lost
    assert abs((dw_bad * w).sum() - ref) > 1e-6


def test_off_by_one_transpose_is_caught():
    rng = np.random.default_rng(2)
    n = 12
    recv = np.sort(rng.integers(0, n, size=50))
    row_ptr = graph.row_ptr_from_receivers(recv, n)
    senders = rng.integers(0, n, size=50).astype(np.int32)
    sp, pe, sr = graph.transpose(n, row_ptr, senders)
    ref = np.argsort(senders, kind="stable")
    assert np.array_equal(pe, ref)
    bad = np.argsort(senders, kind="stable")
    bad[1:] = bad[:-1].copy()
    assert not np.array_equal(bad, ref)
    # an unstable sort is caught too whenever a sender has repeated edges
    unstable = np.lexsort((-np.arange(50), senders))
    assert not np.array_equal(unstable, ref)

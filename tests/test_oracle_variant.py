"""Pins of the oracle's MACE variant: natural-parity paths, one output slot
per path (oracle.convtp.Problem(..., variant=1)).

Fixed by: the path counts; summing the slots of paths that share l3 gives the
(pinned) summed convolution with the odd-parity paths' weights set to zero;
inversion parity (x_l -> (-1)^l x_l and vec -> -vec send every slot to
(-1)^l3 times itself, which an odd-parity path would violate); rotation
equivariance slot by slot; the adjoint identities; the C edge loop against
the materialised definition; finite differences of the backward.
"""
import numpy as np
import pytest

from oracle import convtp as ct
from oracle import graph, sh, wigner


def _case(L, n=8, e=30, c=3, seed=0):
    rng = np.random.default_rng(seed)
    recv = np.sort(rng.integers(0, n, size=e))
    row_ptr = graph.row_ptr_from_receivers(recv, n)
    senders = rng.integers(0, n, size=e).astype(np.int32)
    vec = rng.standard_normal((e, 3))
    return rng, row_ptr, senders, vec


def _parity(L):
    return np.concatenate([np.full(2 * l + 1, (-1.0) ** l) for l in range(L + 1)])


def test_path_counts():
    assert [ct.Problem(L, L, L, variant=1).P for L in range(4)] == [1, 4, 11, 23]
    for L in range(4):
        pr = ct.Problem(L, L, L, variant=1)
        assert all((a + b + c) % 2 == 0 for a, b, c in pr.paths)
        assert pr.D3 == sum(2 * c + 1 for _, _, c in pr.paths)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_slots_sum_to_summed_variant_without_odd_paths(L):
    rng, rp, s, vec = _case(L, seed=L)
    p1, p0 = ct.Problem(L, L, L, variant=1), ct.Problem(L, L, L)
    Y = sh.real_sh(L, vec)
    x = rng.standard_normal((8, p1.D1, 3))
    w1 = rng.standard_normal((30, p1.P, 3))
    w0 = np.zeros((30, p0.P, 3))
    for k, path in enumerate(p1.paths):
        w0[:, p0.paths.index(path), :] = w1[:, k, :]
    out1 = ct.materialised_fwd(p1, x, Y, w1, rp, s)
    out0 = ct.materialised_fwd(p0, x, Y, w0, rp, s)
    summed = np.zeros_like(out0)
    for k, (_, _, l3) in enumerate(p1.paths):
        summed[:, l3 * l3:(l3 + 1) ** 2, :] += out1[:, p1.oslice(k), :]
    np.testing.assert_allclose(summed, out0, atol=1e-12)


@pytest.mark.parametrize("L", [2, 3])
def test_inversion_parity_and_rotation(L):
    rng, rp, s, vec = _case(L, seed=10 + L)
    pr = ct.Problem(L, L, L, variant=1)
    x = rng.standard_normal((8, pr.D1, 3))
    w = rng.standard_normal((30, pr.P, 3))
    out = ct.materialised_fwd(pr, x, sh.real_sh(L, vec), w, rp, s)
    par = _parity(L)
    outP = ct.materialised_fwd(pr, par[None, :, None] * x, sh.real_sh(L, -vec), w, rp, s)
    sign = np.concatenate([np.full(2 * l3 + 1, (-1.0) ** l3) for _, _, l3 in pr.paths])
    np.testing.assert_allclose(outP, sign[None, :, None] * out, atol=1e-12)
    # the summed variant keeps odd paths, which break the same identity
    p0 = ct.Problem(L, L, L)
    w0 = rng.standard_normal((30, p0.P, 3))
    o0 = ct.materialised_fwd(p0, x, sh.real_sh(L, vec), w0, rp, s)
    o0P = ct.materialised_fwd(p0, par[None, :, None] * x, sh.real_sh(L, -vec), w0, rp, s)
    assert not np.allclose(o0P, par[None, :, None] * o0, atol=1e-6)
    # rotations act on each slot with its own D^l3
    ang = wigner.random_angles(rng)
    R = wigner.rotation_matrix(*ang)
    D = wigner.block_D(L, *ang)
    outR = ct.materialised_fwd(pr, np.einsum("ab,nbc->nac", D, x), sh.real_sh(L, vec @ R.T), w, rp, s)
    for k, (_, _, l3) in enumerate(pr.paths):
        Dl = wigner.real_D(l3, *ang)
        np.testing.assert_allclose(outR[:, pr.oslice(k), :], np.einsum("ab,nbc->nac", Dl, out[:, pr.oslice(k), :]),
                                   atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_adjoint_and_c_loop(L, oracle_lib):
    rng, rp, s, vec = _case(L, n=10, e=45, c=4, seed=20 + L)
    pr = ct.Problem(L, L, L, variant=1)
    Y = sh.real_sh(L, vec)
    x = rng.standard_normal((10, pr.D1, 4)).astype(np.float32)
    w = rng.standard_normal((45, pr.P, 4)).astype(np.float32)
    G = rng.standard_normal((10, pr.D3, 4)).astype(np.float32)
    out = ct.materialised_fwd(pr, x, Y, w, rp, s)
    dx, dw, dY = ct.materialised_bwd(pr, x, Y, w, G, rp, s)
    ref = (G * out).sum()
    for a, b in ((dx, x), (dw, w), (dY, Y)):
        assert abs((a * b).sum() - ref) <= 1e-11 * max(1.0, abs(ref))
    sp, pe, sr = graph.transpose(10, rp, s)
    np.testing.assert_allclose(ct.fwd(pr, x, Y, w, rp, s), out, atol=1e-11)
    np.testing.assert_allclose(ct.bwd_dx(pr, Y, w, G, sp, pe, sr), dx, atol=1e-11)
    cdw, cdY = ct.bwd_edges(pr, x, Y, w, G, rp, s)
    np.testing.assert_allclose(cdw, dw, atol=1e-11)
    np.testing.assert_allclose(cdY, dY, atol=1e-11)


def test_finite_differences():
    L = 2
    rng, rp, s, vec = _case(L, n=5, e=9, c=2, seed=31)
    pr = ct.Problem(L, L, L, variant=1)
    Y = sh.real_sh(L, vec)
    x = rng.standard_normal((5, pr.D1, 2))
    w = rng.standard_normal((9, pr.P, 2))
    G = rng.standard_normal((5, pr.D3, 2))
    dx, dw, dY = ct.materialised_bwd(pr, x, Y, w, G, rp, s)
    loss = lambda x_, Y_, w_: (G * ct.materialised_fwd(pr, x_, Y_, w_, rp, s)).sum()  # noqa: E731
    h = 1e-5
    for arr, grad, f in ((x, dx, lambda a: loss(a, Y, w)), (w, dw, lambda a: loss(x, Y, a)),
                         (Y, dY, lambda a: loss(x, a, w))):
        for k in rng.choice(arr.size, size=min(arr.size, 30), replace=False):
            idx = np.unravel_index(k, arr.shape)
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            assert abs((f(a1) - f(a2)) / (2 * h) - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx]))

"""Pins of the oracle's second derivatives of the harmonics (used by the
edge-vector VJP-of-VJP): the Hessian against central differences of the
(pinned) gradient, its symmetry, the radial identity H v = -J (Y has degree 0
in |v|), and the full edge-vector VJP-of-VJP of a small convolution against
central differences of L2 = <ax, dx> + <aw, dw> + <avec, dvec> in vec."""
import numpy as np
import pytest

from oracle import convtp as ct
from oracle import graph, sh


@pytest.mark.parametrize("L", [1, 2, 3])
def test_hessian_matches_gradient_differences(L):
    rng = np.random.default_rng(L)
    v = rng.standard_normal((20, 3)) * rng.uniform(0.5, 2.0, (20, 1))
    H = sh.real_sh_hess(L, v)
    h = 1e-6
    for i in range(3):
        vp, vm = v.copy(), v.copy()
        vp[:, i] += h
        vm[:, i] -= h
        num = (sh.real_sh_grad(L, vp) - sh.real_sh_grad(L, vm)) / (2 * h)   # [e, k, j] = d(dY_k/dv_j)/dv_i
        np.testing.assert_allclose(H[:, :, i, :], num, atol=2e-7 * np.abs(H).max())
    np.testing.assert_allclose(H, np.swapaxes(H, -1, -2), atol=1e-12)
    # Y(t v) = Y(v) for t > 0:  J v = 0, and differentiating again  H v = -J
    np.testing.assert_allclose(np.einsum("ekij,ej->eki", H, v), -sh.real_sh_grad(L, v), atol=1e-12)
    assert np.all(sh.real_sh_hess(L, np.zeros((1, 3))) == 0.0)


@pytest.mark.parametrize("L", [2, 3])
def test_edge_vector_double_backward(L):
    rng = np.random.default_rng(40 + L)
    n, e, c = 6, 12, 3
    prob = ct.Problem(L, L, L)
    recv = np.sort(rng.integers(0, n, size=e))
    rp = graph.row_ptr_from_receivers(recv, n)
    s = rng.integers(0, n, size=e).astype(np.int32)
    vec = rng.standard_normal((e, 3))
    x, w, G = (rng.standard_normal(sh_) for sh_ in ((n, prob.D1, c), (e, prob.P, c), (n, prob.D3, c)))
    ax, aw, av = (rng.standard_normal(sh_) for sh_ in ((n, prob.D1, c), (e, prob.P, c), (e, 3)))

    def L2(vec_):
        Y = sh.real_sh(L, vec_)
        dx, dw, dY = ct.materialised_bwd(prob, x, Y, w, G, rp, s)
        dvec = sh.vec_grad_from_sh_grad(L, vec_, dY)
        return (ax * dx).sum() + (aw * dw).sum() + (av * dvec).sum()

    # the composition the library offers: aY = J av; Y-given double backward;
    # gvec = J^T gY + d/dvec <J av, dY>
    Y = sh.real_sh(L, vec)
    aY = sh.real_sh_jvp(L, vec, av)
    gx, gw, gY, gG = ct.materialised_double_bwd(prob, x, Y, w, G, ax, aw, aY, rp, s)
    _, _, dY = ct.materialised_bwd(prob, x, Y, w, G, rp, s)
    gvec = sh.vec_grad_from_sh_grad(L, vec, gY) + sh.vec_hess_term(L, vec, dY, av)
    h = 1e-5
    for k in range(e):
        for i in range(3):
            vp, vm = vec.copy(), vec.copy()
            vp[k, i] += h
            vm[k, i] -= h
            num = (L2(vp) - L2(vm)) / (2 * h)
            assert abs(num - gvec[k, i]) <= 2e-7 * max(1.0, abs(gvec[k, i])), (k, i, num, gvec[k, i])

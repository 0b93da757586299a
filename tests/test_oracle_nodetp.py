"""Pins of the oracle's node-local channelwise tensor product and its VJP.

Fixed by: the convolution oracle (itself pinned) on a graph of self-edges
when y carries the same harmonics in every channel; rotation equivariance in
both inputs; the adjoint identities of the trilinear map; central finite
differences; a planted mistake (inputs swapped inside one path) caught by the
reduction to the convolution.
"""
import numpy as np
import pytest

from oracle import convtp as ct
from oracle import nodetp as nt
from oracle import sh, wigner


def _case(L, n=7, c=3, seed=0):
    rng = np.random.default_rng(seed)
    prob = nt.NodeProblem(L, L, L)
    x = rng.standard_normal((n, prob.D1, c))
    y = rng.standard_normal((n, prob.D2, c))
    w = rng.standard_normal((n, prob.P, c))
    G = rng.standard_normal((n, prob.D3, c))
    return prob, x, y, w, G


@pytest.mark.parametrize("L", [1, 2, 3])
def test_reduces_to_convolution_over_self_edges(L):
    # y[i, :, c] = Y(v_i) for every channel: out_i is the convolution of x over
    # the single edge i -> i with harmonic Y(v_i) and weights w_i.
    rng = np.random.default_rng(40 + L)
    n, c = 9, 4
    prob = nt.NodeProblem(L, L, L)
    cprob = ct.Problem(L, L, L)
    vec = rng.standard_normal((n, 3))
    Y = sh.real_sh(L, vec)
    x = rng.standard_normal((n, prob.D1, c))
    w = rng.standard_normal((n, prob.P, c))
    G = rng.standard_normal((n, prob.D3, c))
    y = np.repeat(Y[:, :, None], c, axis=2)
    row_ptr = np.arange(n + 1, dtype=np.int32)
    senders = np.arange(n, dtype=np.int32)
    np.testing.assert_allclose(nt.fwd(prob, x, y, w),
                               ct.materialised_fwd(cprob, x, Y, w, row_ptr, senders), atol=1e-12)
    dx, dy, dw = nt.bwd(prob, x, y, w, G)
    cdx, cdw, cdY = ct.materialised_bwd(cprob, x, Y, w, G, row_ptr, senders)
    np.testing.assert_allclose(dx, cdx, atol=1e-12)
    np.testing.assert_allclose(dw, cdw, atol=1e-12)
    np.testing.assert_allclose(dy.sum(axis=2), cdY, atol=1e-12)


@pytest.mark.parametrize("L", [2, 3])
def test_rotation_equivariance(L):
    rng = np.random.default_rng(50 + L)
    prob, x, y, w, G = _case(L, n=8, c=3, seed=L)
    D = wigner.block_D(L, *wigner.random_angles(rng))
    rot = lambda a: np.einsum("ab,nbc->nac", D, a)  # noqa: E731
    out = nt.fwd(prob, x, y, w)
    np.testing.assert_allclose(nt.fwd(prob, rot(x), rot(y), w), rot(out), atol=1e-12)
    dx, dy, dw = nt.bwd(prob, x, y, w, G)
    dxR, dyR, dwR = nt.bwd(prob, rot(x), rot(y), w, rot(G))
    np.testing.assert_allclose(dxR, rot(dx), atol=1e-12)
    np.testing.assert_allclose(dyR, rot(dy), atol=1e-12)
    np.testing.assert_allclose(dwR, dw, atol=1e-12)


@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_adjoint_identities(L):
    prob, x, y, w, G = _case(L, n=11, c=5, seed=60 + L)
    ref = (G * nt.fwd(prob, x, y, w)).sum()
    dx, dy, dw = nt.bwd(prob, x, y, w, G)
    for a, b in ((dx, x), (dy, y), (dw, w)):
        assert abs((a * b).sum() - ref) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("L", [2, 3])
def test_finite_differences(L):
    prob, x, y, w, G = _case(L, n=4, c=3, seed=70 + L)
    dx, dy, dw = nt.bwd(prob, x, y, w, G)
    loss = lambda x_, y_, w_: (G * nt.fwd(prob, x_, y_, w_)).sum()  # noqa: E731
    h = 1e-5
    rng = np.random.default_rng(1)
    for arr, grad, f in ((x, dx, lambda a: loss(a, y, w)), (y, dy, lambda a: loss(x, a, w)),
                         (w, dw, lambda a: loss(x, y, a))):
        for k in rng.choice(arr.size, size=min(arr.size, 50), replace=False):
            idx = np.unravel_index(k, arr.shape)
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            num = (f(a1) - f(a2)) / (2 * h)
            assert abs(num - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx])), (idx, num, grad[idx])


def test_swapped_inputs_in_one_path_are_caught(monkeypatch):
    # plant: path (1, 2, 2) contracts y's l=1 block with x's l=2 block
    L = 2
    prob = nt.NodeProblem(L, L, L)
    bad = prob.paths.index((1, 2, 2))
    good = nt.fwd

    def planted(prob_, x, y, w):
        out = good(prob_, x, y, w)
        Cp = prob_.blocks[bad]
        s1, s2 = slice(1, 4), slice(4, 9)
        right = np.einsum("abk,nac,nbc->nkc", Cp, x[:, s1], y[:, s2])
        wrong = np.einsum("abk,nac,nbc->nkc", Cp, y[:, s1], x[:, s2])
        out[:, s2] += w[:, bad, None, :] * (wrong - right)
        return out

    monkeypatch.setattr(nt, "fwd", planted)
    with pytest.raises(AssertionError):
        test_reduces_to_convolution_over_self_edges(L)

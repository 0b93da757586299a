"""Pins of the oracle's VJP of the VJP (materialised_double_bwd).

Fixed by: central finite differences of L2 = <ax, dx> + <aw, dw> + <aY, dY>,
with (dx, dw, dY) from the pinned first backward, in every input (x, w, Y, G);
the linearity of L2 in G (<gG, G> = L2); its joint degree 2 in (x, w, Y)
(<gx, x> + <gw, w> + <gY, Y> = 2 L2); a planted dropped term caught by the
finite differences.
"""
import numpy as np
import pytest

from oracle import convtp as ct
from oracle import graph, sh


def _case(L, n=6, e=11, c=3, seed=0):
    rng = np.random.default_rng(seed)
    prob = ct.Problem(L, L, L)
    recv = np.sort(rng.integers(0, n, size=e))
    row_ptr = graph.row_ptr_from_receivers(recv, n)
    senders = rng.integers(0, n, size=e).astype(np.int32)
    Y = sh.real_sh(L, rng.standard_normal((e, 3)))
    x = rng.standard_normal((n, prob.D1, c))
    w = rng.standard_normal((e, prob.P, c))
    G = rng.standard_normal((n, prob.D3, c))
    ax = rng.standard_normal((n, prob.D1, c))
    aw = rng.standard_normal((e, prob.P, c))
    aY = rng.standard_normal((e, prob.D2))
    return prob, row_ptr, senders, x, Y, w, G, ax, aw, aY


def _L2(prob, row_ptr, senders, x, Y, w, G, ax, aw, aY):
    dx, dw, dY = ct.materialised_bwd(prob, x, Y, w, G, row_ptr, senders)
    return (ax * dx).sum() + (aw * dw).sum() + (aY * dY).sum()


@pytest.mark.parametrize("L", [1, 2, 3])
def test_invariants(L):
    prob, rp, s, x, Y, w, G, ax, aw, aY = _case(L, n=9, e=40, c=4, seed=L)
    l2 = _L2(prob, rp, s, x, Y, w, G, ax, aw, aY)
    gx, gw, gY, gG = ct.materialised_double_bwd(prob, x, Y, w, G, ax, aw, aY, rp, s)
    tol = 1e-12 * max(1.0, abs(l2))
    assert abs((gG * G).sum() - l2) <= tol
    assert abs((gx * x).sum() + (gw * w).sum() + (gY * Y).sum() - 2 * l2) <= 2 * tol


@pytest.mark.parametrize("L", [2, 3])
def test_finite_differences(L):
    prob, rp, s, x, Y, w, G, ax, aw, aY = _case(L, seed=10 + L)
    grads = ct.materialised_double_bwd(prob, x, Y, w, G, ax, aw, aY, rp, s)
    args = [x, w, Y, G]
    h = 1e-5
    rng = np.random.default_rng(2)

    def f(k, a):
        v = list(args)
        v[k] = a
        return _L2(prob, rp, s, v[0], v[2], v[1], v[3], ax, aw, aY)

    for k, (arr, grad) in enumerate(zip(args, grads)):
        for flat in rng.choice(arr.size, size=min(arr.size, 40), replace=False):
            idx = np.unravel_index(flat, arr.shape)
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            num = (f(k, a1) - f(k, a2)) / (2 * h)
            assert abs(num - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx])), (k, idx, num, grad[idx])


def test_dropped_term_is_caught(monkeypatch):
    good = ct.materialised_double_bwd

    def planted(prob, x, Y, w, G, ax, aw, aY, row_ptr, senders):
        gx, gw, gY, gG = good(prob, x, Y, w, G, ax, aw, aY, row_ptr, senders)
        # drop the <aY, dY> part of gw
        _, gw_only_ax, _, _ = good(prob, x, Y, w, G, ax, aw, np.zeros_like(aY), row_ptr, senders)
        return gx, gw_only_ax, gY, gG

    monkeypatch.setattr(ct, "materialised_double_bwd", planted)
    with pytest.raises(AssertionError):
        test_finite_differences(2)


def test_c_oracle_composition_matches(oracle_lib):
    # The sampled full-size GPU checks build the double backward from the C
    # edge loop's forward and backward with swapped operands; on a small graph
    # that composition equals the finite-difference-pinned numpy function.
    L = 3
    prob, rp, s, x, Y, w, G, ax, aw, aY = _case(L, n=12, e=60, c=5, seed=33)
    x, w, G, ax, aw = (a.astype(np.float32) for a in (x, w, G, ax, aw))
    sp, pe, sr = graph.transpose(12, rp, s)
    gx, gw, gY, gG = ct.materialised_double_bwd(prob, x, Y, w, G, ax, aw, aY, rp, s)
    cG = ct.fwd(prob, ax, Y, w, rp, s) + ct.fwd(prob, x, Y, aw, rp, s) + ct.fwd(prob, x, aY, w, rp, s)
    cx = ct.bwd_dx(prob, Y, aw, G, sp, pe, sr) + ct.bwd_dx(prob, aY, w, G, sp, pe, sr)
    dw1, dY1 = ct.bwd_edges(prob, ax, Y, w, G, rp, s)
    dw2, _ = ct.bwd_edges(prob, x, aY, w, G, rp, s)
    _, dY3 = ct.bwd_edges(prob, x, Y, aw, G, rp, s)
    for a, b in ((cG, gG), (cx, gx), (dw1 + dw2, gw), (dY1 + dY3, gY)):
        np.testing.assert_allclose(a, b, atol=1e-11, rtol=0)

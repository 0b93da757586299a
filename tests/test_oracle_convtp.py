"""Pins of the oracle's convolution, its VJP and the graph bookkeeping.

Fixed by: the l=0 special case against a numpy segment sum, brute-force
materialisation against the C edge loop, invariance under permutations of a
receiver's edges, rotation equivariance of outputs and gradients, adjoint
identities of the trilinear map, and central finite differences of
<G, out> in every input (x, w, Y and the edge vectors).
"""
import math

import numpy as np
import pytest

from oracle import convtp as ct
from oracle import graph, sh, wigner
from workloads import gen


def _random_graph(n, e, rng):
    recv = np.sort(rng.integers(0, n, size=e))
    send = rng.integers(0, n, size=e)
    return graph.row_ptr_from_receivers(recv, n), send.astype(np.int32)


def _case(L, n=6, e=10, c=3, seed=0, lin=None, lsh=None, lout=None):
    rng = np.random.default_rng(seed)
    lin = L if lin is None else lin
    lsh = L if lsh is None else lsh
    lout = L if lout is None else lout
    prob = ct.Problem(lin, lsh, lout)
    row_ptr, senders = _random_graph(n, e, rng)
    vec = rng.standard_normal((e, 3))
    x = rng.standard_normal((n, prob.D1, c))
    w = rng.standard_normal((e, prob.P, c))
    G = rng.standard_normal((n, prob.D3, c))
    return prob, row_ptr, senders, vec, x, w, G


@pytest.fixture(scope="module", autouse=True)
def _lib(oracle_lib):
    return oracle_lib


def test_l0_special_case_is_a_segment_sum():
    rng = np.random.default_rng(1)
    n, e, c = 20, 90, 5
    row_ptr, senders = _random_graph(n, e, rng)
    x = rng.standard_normal((n, 1, c)).astype(np.float32)
    w = rng.standard_normal((e, 1, c)).astype(np.float32)
    Y = np.full((e, 1), 1 / math.sqrt(4 * math.pi))
    prob = ct.Problem(0, 0, 0)
    out = ct.fwd(prob, x, Y, w, row_ptr, senders)
    ref = np.zeros((n, c))
    np.add.at(ref, graph.receivers_of(row_ptr),
              w[:, 0, :].astype(np.float64) * x[senders, 0, :] / math.sqrt(4 * math.pi))
    np.testing.assert_allclose(out[:, 0, :], ref, atol=1e-13)


@pytest.mark.parametrize("dims", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (0, 3, 3), (3, 2, 1), (1, 3, 2)])
def test_c_edge_loop_matches_materialised_definition(dims):
    rng = np.random.default_rng(2)
    prob = ct.Problem(*dims)
    n, e, c = 12, 60, 7
    row_ptr, senders = _random_graph(n, e, rng)
    x = rng.standard_normal((n, prob.D1, c)).astype(np.float32)
    w = rng.standard_normal((e, prob.P, c)).astype(np.float32)
    G = rng.standard_normal((n, prob.D3, c)).astype(np.float32)
    Y = sh.real_sh(prob.l_sh, rng.standard_normal((e, 3)))
    out = ct.fwd(prob, x, Y, w, row_ptr, senders)
    np.testing.assert_allclose(out, ct.materialised_fwd(prob, x, Y, w, row_ptr, senders), atol=1e-12)
    dx, dw, dY = ct.materialised_bwd(prob, x, Y, w, G, row_ptr, senders)
    sp, pe, sr = graph.transpose(n, row_ptr, senders)
    np.testing.assert_allclose(ct.bwd_dx(prob, Y, w, G, sp, pe, sr), dx, atol=1e-12)
    dw2, dY2 = ct.bwd_edges(prob, x, Y, w, G, row_ptr, senders)
    np.testing.assert_allclose(dw2, dw, atol=1e-12)
    np.testing.assert_allclose(dY2, dY, atol=1e-12)
    # subsets evaluate the same rows
    rows = np.array([5, 0, 11, 5])
    np.testing.assert_allclose(ct.fwd(prob, x, Y, w, row_ptr, senders, rows=rows), out[rows], atol=0)
    erows = np.array([59, 3, 17])
    dws, dYs = ct.bwd_edges(prob, x, Y, w, G, row_ptr, senders, rows=erows)
    np.testing.assert_allclose(dws, dw2[erows], atol=0)
    np.testing.assert_allclose(dYs, dY2[erows], atol=0)


def test_permuting_edges_within_receivers():
    rng = np.random.default_rng(3)
    prob, row_ptr, senders, vec, x, w, G = _case(3, n=10, e=80, c=4, seed=3)
    Y = sh.real_sh(3, vec)
    perm = np.concatenate([rng.permutation(np.arange(row_ptr[i], row_ptr[i + 1]))
                           for i in range(len(row_ptr) - 1)]).astype(np.int64)
    a = ct.materialised_fwd(prob, x, Y, w, row_ptr, senders)
    b = ct.materialised_fwd(prob, x, Y[perm], w[perm], row_ptr, senders[perm])
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_zero_in_degree_and_empty_graph():
    prob, row_ptr, senders, vec, x, w, G = _case(2, n=8, e=6, c=2, seed=4)
    Y = sh.real_sh(2, vec)
    out = ct.fwd(prob, x, Y, w, row_ptr, senders)
    empty = np.diff(row_ptr) == 0
    assert empty.any()
    assert not out[empty].any()
    rp0 = np.zeros(9, dtype=np.int32)
    s0 = np.zeros(0, dtype=np.int32)
    out0 = ct.fwd(prob, x, np.zeros((0, 9)), np.zeros((0, prob.P, 2)), rp0, s0)
    assert out0.shape == (8, 9, 2) and not out0.any()


@pytest.mark.parametrize("L", [2, 3])
def test_rotation_equivariance(L):
    rng = np.random.default_rng(10 + L)
    prob, row_ptr, senders, vec, x, w, G = _case(L, n=9, e=40, c=3, seed=L)
    ang = wigner.random_angles(rng)
    R = wigner.rotation_matrix(*ang)
    D = wigner.block_D(L, *ang)
    Y, YR = sh.real_sh(L, vec), sh.real_sh(L, vec @ R.T)
    xR = np.einsum("ab,nbc->nac", D, x)
    GR = np.einsum("ab,nbc->nac", D, G)
    out = ct.materialised_fwd(prob, x, Y, w, row_ptr, senders)
    outR = ct.materialised_fwd(prob, xR, YR, w, row_ptr, senders)
    np.testing.assert_allclose(outR, np.einsum("ab,nbc->nac", D, out), atol=1e-12)
    dx, dw, dY = ct.materialised_bwd(prob, x, Y, w, G, row_ptr, senders)
    dxR, dwR, dYR = ct.materialised_bwd(prob, xR, YR, w, GR, row_ptr, senders)
    np.testing.assert_allclose(dxR, np.einsum("ab,nbc->nac", D, dx), atol=1e-12)
    np.testing.assert_allclose(dwR, dw, atol=1e-12)          # invariant
    np.testing.assert_allclose(dYR, dY @ D.T, atol=1e-12)
    dv = sh.vec_grad_from_sh_grad(L, vec, dY)
    dvR = sh.vec_grad_from_sh_grad(L, vec @ R.T, dYR)
    np.testing.assert_allclose(dvR, dv @ R.T, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_adjoint_identities(L):
    prob, row_ptr, senders, vec, x, w, G = _case(L, n=10, e=50, c=4, seed=20 + L)
    Y = sh.real_sh(L, vec)
    out = ct.materialised_fwd(prob, x, Y, w, row_ptr, senders)
    dx, dw, dY = ct.materialised_bwd(prob, x, Y, w, G, row_ptr, senders)
    ref = (G * out).sum()
    for a, b in ((dx, x), (dw, w), (dY, Y)):
        assert abs((a * b).sum() - ref) <= 1e-12 * max(1.0, abs(ref))
    dv = sh.vec_grad_from_sh_grad(L, vec, dY)
    np.testing.assert_allclose((dv * vec).sum(1), 0.0, atol=1e-12)


@pytest.mark.parametrize("L", [2, 3])
def test_finite_differences(L):
    """Central differences (h = 1e-5, fp64) of <G, out> on N=6, E=10, C=3."""
    prob, row_ptr, senders, vec, x, w, G = _case(L, n=6, e=10, c=3, seed=30 + L)
    Y = sh.real_sh(L, vec)

    def loss(x_, Y_, w_):
        return (G * ct.materialised_fwd(prob, x_, Y_, w_, row_ptr, senders)).sum()

    dx, dw, dY = ct.materialised_bwd(prob, x, Y, w, G, row_ptr, senders)
    h = 1e-5

    def fd(arr, idx, f):
        a1, a2 = arr.copy(), arr.copy()
        a1[idx] += h
        a2[idx] -= h
        return (f(a1) - f(a2)) / (2 * h)

    rng = np.random.default_rng(0)
    for arr, grad, f in ((x, dx, lambda a: loss(a, Y, w)),
                         (w, dw, lambda a: loss(x, Y, a)),
                         (Y, dY, lambda a: loss(x, a, w))):
        flat = rng.choice(arr.size, size=min(arr.size, 60), replace=False)
        for k in flat:
            idx = np.unravel_index(k, arr.shape)
            num = fd(arr, idx, f)
            assert abs(num - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx])), (idx, num, grad[idx])
    dv = sh.vec_grad_from_sh_grad(L, vec, dY)
    for e in range(vec.shape[0]):
        for i in range(3):
            num = fd(vec, (e, i), lambda v: loss(x, sh.real_sh(L, v), w))
            assert abs(num - dv[e, i]) <= 1e-7 * max(1.0, abs(dv[e, i]))


def test_graph_transpose_and_check():
    rng = np.random.default_rng(6)
    n = 30
    row_ptr, senders = gen.poisson_graph(n, 5.0, rng)
    sp, pe, sr = graph.transpose(n, row_ptr, senders)
    assert np.array_equal(np.sort(pe), np.arange(senders.size))
    recv = graph.receivers_of(row_ptr)
    for j in range(n):
        seg = pe[sp[j]:sp[j + 1]]
        assert (senders[seg] == j).all()
        assert (np.diff(seg) > 0).all()          # stable: CSR edge order kept
        assert np.array_equal(sr[sp[j]:sp[j + 1]], recv[seg])
    assert graph.check_graph(n, row_ptr, senders) == 0
    bad_s = senders.copy()
    bad_s[[0, 3]] = [n, -1]
    assert graph.check_graph(n, row_ptr, bad_s) == 2
    bad_rp = row_ptr.copy()
    bad_rp[5] = bad_rp[6] + 1
    assert graph.check_graph(n, bad_rp, senders) == 1


def test_generators_shape_and_law():
    t = gen.tiny()
    assert t["n_edges"] == 1024 and t["w"].shape == (1024, 5, 16)
    rp, s = t["row_ptr"], t["senders"]
    recv = graph.receivers_of(rp)
    assert not (s == recv).any()
    for i in range(64):
        assert len(set(s[rp[i]:rp[i + 1]].tolist())) == 16
    np.testing.assert_allclose(np.linalg.norm(t["vec"], axis=1), 1.0, atol=1e-6)
    rng = np.random.default_rng(0)
    rp, s = gen.poisson_graph(4096, 45.0, rng)
    deg = np.diff(rp)
    assert abs(deg.mean() - 45) < 0.5 and abs(deg.var() - 45) < 4
    assert not (s == graph.receivers_of(rp)).any()
    wb = gen.water_box_graph()
    assert wb["n_edges"] == 83325 and abs(wb["n_real"] - 75650) < 5 * 382
    assert graph.check_graph(1503, wb["row_ptr"], wb["senders"]) == 0

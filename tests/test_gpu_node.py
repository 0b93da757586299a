"""GPU parity of the node-local channelwise tensor product (forward and VJP)
against the fp64 oracle, through the C ABI.

Bar as for the convolution: per output tensor, max |gpu - oracle| <=
1e-4 * max |oracle|; bitwise reproducible run to run.  Small cases element by
element (ragged channel tails, every degree); the full-size workload on a
seeded sample of nodes, which the oracle evaluates on their rows alone (every
node is independent).
"""
import numpy as np
import pytest
import torch

from oracle import nodetp as ont
from workloads import gen

pytestmark = pytest.mark.gpu
RTOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_product_message_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ctp(dev):
    import tensor_product_message_amd as t
    return t


def close(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    scale = float(np.abs(ref).max())
    assert scale > 0.0, f"{name}: reference is identically zero"
    assert np.isfinite(got).all(), name
    err = float(np.abs(got - ref).max())
    assert err <= RTOL * scale, f"{name}: max err {err:.3e} vs scale {scale:.3e}"


def T(a, dev):
    return torch.as_tensor(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("n,c,L", [(50, 16, 0), (60, 48, 1), (70, 128, 2), (40, 100, 3), (30, 256, 3),
                                   (9, 1024, 3), (33, 64, 3), (17, 1, 2)])
def test_small(ctp, dev, n, c, L):
    d = gen.node_small(n, c, L, seed=n + c + L)
    prob = ont.NodeProblem(L, L, L)
    x, y, w, G = (T(d[k], dev) for k in ("x", "y", "w", "grad_out"))
    out = ctp.node_tp_fwd(x, y, w, L)
    dx, dy, dw = ctp.node_tp_bwd(G, x, y, w, L)
    torch.cuda.synchronize()
    close("out", out.cpu().numpy(), ont.fwd(prob, d["x"], d["y"], d["w"]))
    rdx, rdy, rdw = ont.bwd(prob, d["x"], d["y"], d["w"], d["grad_out"])
    close("dx", dx.cpu().numpy(), rdx)
    close("dy", dy.cpu().numpy(), rdy)
    close("dw", dw.cpu().numpy(), rdw)


def test_full_size_sampled_and_deterministic(ctp, dev):
    s = gen.NODE
    L = s["lmax"]
    d = gen.node_full(s["n_nodes"], s["channels"], L, dev, seed=0)
    x, y, w, G = d["x"], d["y"], d["w"], d["grad_out"]
    out = ctp.node_tp_fwd(x, y, w, L)
    dx, dy, dw = ctp.node_tp_bwd(G, x, y, w, L)
    out2 = ctp.node_tp_fwd(x, y, w, L)
    dx2, dy2, dw2 = ctp.node_tp_bwd(G, x, y, w, L)
    torch.cuda.synchronize()
    for a, b in ((out, out2), (dx, dx2), (dy, dy2), (dw, dw2)):
        assert torch.equal(a, b)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(s["n_nodes"], size=64, replace=False))
    rows = np.concatenate([[0], rows, [s["n_nodes"] - 1]])
    idx = torch.as_tensor(rows, device=dev)
    host = lambda t: t.index_select(0, idx).cpu().numpy()  # noqa: E731
    prob = ont.NodeProblem(L, L, L)
    hx, hy, hw, hG = host(x), host(y), host(w), host(G)
    close("out", host(out), ont.fwd(prob, hx, hy, hw))
    rdx, rdy, rdw = ont.bwd(prob, hx, hy, hw, hG)
    close("dx", host(dx), rdx)
    close("dy", host(dy), rdy)
    close("dw", host(dw), rdw)


def test_empty(ctp, dev):
    z = torch.zeros((0, 16, 8), device=dev)
    out = ctp.node_tp_fwd(z, z, torch.zeros((0, 34, 8), device=dev), 3)
    assert out.shape == (0, 16, 8)

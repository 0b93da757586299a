"""Second-order autograd through the library (force training): a loss on the
gradient of an energy, differentiated again with create_graph=True, must give
the oracle's VJP of the VJP (FlashCart, arXiv 2610.06409, section 3: the
VJP-of-VJP that force training needs).

The energy is E = <H, conv(x, Y or vec, w)> with a fixed H, so its gradients
are the backward with G = H.  The force-style loss pairs them with fixed
cotangents; its gradients in x, w and Y (or vec) are the oracle's
materialised_double_bwd, plus, for edge vectors, the harmonics' second-order
term vec_hess_term.  Bar: max |gpu - oracle| <= 1e-4 * max |oracle|.
"""
import numpy as np
import pytest
import torch

from oracle import convtp as oc
from oracle import sh as osh
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
    err = float(np.abs(got - ref).max())
    assert err <= RTOL * scale, f"{name}: max err {err:.3e} vs scale {scale:.3e}"


def T(a, dev):
    return torch.as_tensor(np.ascontiguousarray(a)).to(dev)


def host(t):
    return t.detach().cpu().numpy()


def setup(deg, variant, seed):
    prob = oc.Problem(*deg, variant=variant)
    d = gen.poisson_degrees(60, 48, deg[0], deg[1], prob.P, prob.D3, mean_deg=8.0, seed=seed)
    return prob, d


@pytest.mark.parametrize("deg", [(2, 2, 2), (3, 3, 3), (0, 3, 3)])
@pytest.mark.parametrize("variant", [0, 1])
def test_force_loss_edge_vectors(ctp, dev, deg, variant):
    prob, d = setup(deg, variant, seed=13 + variant)
    n, l_sh = d["n_nodes"], deg[1]
    rng = np.random.default_rng(5)
    a_vec = rng.standard_normal(d["vec"].shape).astype(np.float32)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x = T(d["x"], dev).requires_grad_(True)
    w = T(d["w"], dev).requires_grad_(True)
    vec = T(d["vec"], dev).requires_grad_(True)
    H = T(d["grad_out"], dev)
    print(f"[autograd] force loss deg={deg} variant={variant}", flush=True)
    energy = (ctp.conv_tp(x, vec, w, g, deg, ctp.VEC_GIVEN, variant=variant) * H).sum()
    forces = torch.autograd.grad(energy, vec, create_graph=True)[0]
    loss = (forces * T(a_vec, dev)).sum()
    gx, gw, gvec = torch.autograd.grad(loss, (x, w, vec))

    v64 = d["vec"].astype(np.float64)
    Y = osh.real_sh(l_sh, v64)
    _, _, dY = oc.materialised_bwd(prob, d["x"], Y, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    close("forces", host(forces), osh.vec_grad_from_sh_grad(l_sh, v64, dY))
    aY = osh.real_sh_jvp(l_sh, v64, a_vec)
    zx, zw = np.zeros_like(d["x"]), np.zeros_like(d["w"])
    rx, rw, rY, _ = oc.materialised_double_bwd(prob, d["x"], Y, d["w"], d["grad_out"], zx, zw, aY,
                                               d["row_ptr"], d["senders"])
    close("dL/dx", host(gx), rx)
    close("dL/dw", host(gw), rw)
    close("dL/dvec", host(gvec), osh.vec_grad_from_sh_grad(l_sh, v64, rY) + osh.vec_hess_term(l_sh, v64, dY, a_vec))


@pytest.mark.parametrize("variant", [0, 1])
def test_second_order_y_given(ctp, dev, variant):
    deg = (2, 2, 2)
    prob, d = setup(deg, variant, seed=29 + variant)
    n = d["n_nodes"]
    Y32 = osh.real_sh(2, d["vec"].astype(np.float64)).astype(np.float32)
    rng = np.random.default_rng(8)
    ax = rng.standard_normal(d["x"].shape).astype(np.float32)
    aY = rng.standard_normal(Y32.shape).astype(np.float32)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x = T(d["x"], dev).requires_grad_(True)
    w = T(d["w"], dev).requires_grad_(True)
    Y = T(Y32, dev).requires_grad_(True)
    H = T(d["grad_out"], dev).requires_grad_(True)
    energy = (ctp.conv_tp(x, Y, w, g, deg, ctp.Y_GIVEN, variant=variant) * H).sum()
    dEdx, dEdY = torch.autograd.grad(energy, (x, Y), create_graph=True)
    loss = (dEdx * T(ax, dev)).sum() + (dEdY * T(aY, dev)).sum()
    gx, gw, gY, gH = torch.autograd.grad(loss, (x, w, Y, H))
    rx, rw, rY, rG = oc.materialised_double_bwd(prob, d["x"], Y32, d["w"], d["grad_out"], ax,
                                                np.zeros_like(d["w"]), aY, d["row_ptr"], d["senders"])
    close("dL/dx", host(gx), rx)
    close("dL/dw", host(gw), rw)
    close("dL/dY", host(gY), rY)
    close("dL/dH", host(gH), rG)


def test_third_order_is_refused(ctp, dev):
    prob, d = setup((1, 1, 1), 0, seed=3)
    g = ctp.Graph(d["n_nodes"], T(d["row_ptr"], dev), T(d["senders"], dev))
    x = T(d["x"], dev).requires_grad_(True)
    w = T(d["w"], dev).requires_grad_(True)
    vec = T(d["vec"], dev).requires_grad_(True)
    energy = (ctp.conv_tp(x, vec, w, g, 1, ctp.VEC_GIVEN) * T(d["grad_out"], dev)).sum()
    forces = torch.autograd.grad(energy, vec, create_graph=True)[0]
    gw = torch.autograd.grad(forces.sum(), w, create_graph=True)[0]
    with pytest.raises(RuntimeError):
        torch.autograd.grad(gw.sum(), x)

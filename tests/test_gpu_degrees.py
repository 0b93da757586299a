"""GPU parity for independent degrees (l_in, l_sh, l_out) and for up to 1024
channels in every backward entry point, through the C ABI, against the fp64
oracle.

Bar as in test_gpu_parity: max |gpu - oracle| <= 1e-4 * max |oracle| per
output tensor; the deterministic kernels bitwise reproducible run to run
(with two channel tiles the channel sums meet as two fp32 addends onto zero,
which is order-free).  Small graphs are compared element by element.
"""
import numpy as np
import pytest
import torch

from oracle import convtp as oc
from oracle import graph as og
from oracle import sh as osh
from workloads import gen

pytestmark = pytest.mark.gpu
RTOL = 1e-4

TRIPLES = [(0, 3, 3), (1, 3, 2), (3, 2, 1), (2, 2, 2), (0, 1, 1), (2, 0, 2), (3, 3, 0), (1, 0, 3), (0, 0, 0),
           (3, 1, 3), (2, 3, 1)]


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


def close(name, got, ref, nonzero=True):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if nonzero:
        assert scale > 0.0, f"{name}: reference is identically zero"
    assert np.isfinite(got).all(), name
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= RTOL * scale or err == 0.0, f"{name}: max err {err:.3e} vs scale {scale:.3e}"


def T(a, dev):
    return torch.as_tensor(np.ascontiguousarray(a)).to(dev)


def host(t):
    return t.detach().cpu().numpy()


def workload(deg, n, c, variant, seed, mean_deg=10.0):
    a, b, _ = deg
    prob = oc.Problem(*deg, variant=variant)
    d = gen.poisson_degrees(n, c, a, b, prob.P, prob.D3, mean_deg=mean_deg, seed=seed)
    return prob, d


def check_all(ctp, dev, deg, n, c, variant, y_mode, seed, msg=True):
    prob, d = workload(deg, n, c, variant, seed)
    l_sh = deg[1]
    vec = d["vec"]
    Y32 = osh.real_sh(l_sh, vec.astype(np.float64)).astype(np.float32)
    yin = Y32 if y_mode == 0 else vec
    Yref = Y32.astype(np.float64) if y_mode == 0 else osh.real_sh(l_sh, vec.astype(np.float64))
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, yv, G = T(d["x"], dev), T(d["w"], dev), T(yin, dev), T(d["grad_out"], dev)
    print(f"[degrees] deg={deg} n={n} c={c} variant={variant} y_mode={y_mode}", flush=True)
    ref = oc.fwd(prob, d["x"], Yref, d["w"], d["row_ptr"], d["senders"])
    for algo in (0, 1):
        out = ctp.conv_tp_fwd(x, yv, w, g, deg, y_mode, algo, variant=variant)
        close(f"out(algo {algo})", host(out), ref)
    sp, pe, sr = og.transpose(n, d["row_ptr"], d["senders"])
    ref_dx = oc.bwd_dx(prob, Yref, d["w"], d["grad_out"], sp, pe, sr)
    ref_dw, ref_dY = oc.bwd_edges(prob, d["x"], Yref, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    ref_dy = ref_dY if y_mode == 0 else osh.vec_grad_from_sh_grad(l_sh, vec.astype(np.float64), ref_dY)
    dy_nonzero = y_mode == 0 or any(p[1] > 0 for p in prob.paths)   # dvec is exactly 0 without l2 > 0
    runs = [ctp.conv_tp_bwd(G, x, yv, w, g, deg, y_mode, variant=variant)]
    if msg:
        runs.append(ctp.conv_tp_bwd_msg(G, x, yv, w, g, deg, y_mode, variant=variant))
        # algo 1: receiver-major with dx added by atomics; dw and dY the same bits as the message pass
        runs.append(ctp.conv_tp_bwd(G, x, yv, w, g, deg, y_mode, variant=variant, algo=ctp.ALGO_ATOMIC))
        assert torch.equal(runs[2][1], runs[1][1]) and torch.equal(runs[2][2], runs[1][2])
    for k, (dx, dw, dy) in enumerate(runs):
        close(f"dx[{k}]", host(dx), ref_dx)
        close(f"dw[{k}]", host(dw), ref_dw)
        close(f"dy[{k}]", host(dy), ref_dy, nonzero=dy_nonzero)
    dx2, dw2, dy2 = ctp.conv_tp_bwd(G, x, yv, w, g, deg, y_mode, variant=variant)
    assert torch.equal(dx2, runs[0][0]) and torch.equal(dw2, runs[0][1]) and torch.equal(dy2, runs[0][2])
    if y_mode == 0:
        dy_only = ctp.conv_tp_bwd_dy(G, x, w, g, deg, variant=variant)
        assert torch.equal(dy_only, runs[0][2])
    return prob, d


@pytest.mark.parametrize("deg", TRIPLES)
@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("y_mode", [0, 1])
def test_degree_triples_small(ctp, dev, deg, variant, y_mode):
    check_all(ctp, dev, deg, 70, 96, variant, y_mode, seed=sum(deg) * 7 + variant)


@pytest.mark.parametrize("deg", [(0, 3, 3), (1, 3, 2), (3, 2, 1), (2, 2, 2)])
def test_degree_triples_many_receivers(ctp, dev, deg):
    # 4096 receivers at C = 128: the unsplit grids, every output element by element
    for y_mode in (0, 1):
        check_all(ctp, dev, deg, 4096, 128, 0, y_mode, seed=11, msg=False)


@pytest.mark.parametrize("deg", [(0, 3, 3), (1, 3, 2), (3, 2, 1), (2, 2, 2)])
@pytest.mark.parametrize("variant", [0, 1])
def test_degree_triples_double_bwd(ctp, dev, deg, variant):
    prob, d = workload(deg, 60, 64, variant, seed=5 + variant)
    n, l_sh = d["n_nodes"], deg[1]
    Y = osh.real_sh(l_sh, d["vec"].astype(np.float64)).astype(np.float32)
    rng = np.random.default_rng(99)
    ax = rng.standard_normal(d["x"].shape, dtype=np.float32)
    aw = rng.standard_normal(d["w"].shape, dtype=np.float32)
    aY = rng.standard_normal(Y.shape, dtype=np.float32)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    res = ctp.conv_tp_bwd_bwd(T(d["grad_out"], dev), T(d["x"], dev), T(Y, dev), T(d["w"], dev), T(ax, dev),
                              T(aw, dev), T(aY, dev), g, deg, variant=variant)
    ref = oc.materialised_double_bwd(prob, d["x"], Y, d["w"], d["grad_out"], ax, aw, aY, d["row_ptr"],
                                     d["senders"])
    for name, got, want in zip(("g_x", "g_w", "g_y", "g_grad"), res, ref):
        close(name, host(got), want)


@pytest.mark.parametrize("deg", [(0, 3, 3), (3, 2, 1), (1, 1, 2)])
@pytest.mark.parametrize("variant", [0, 1])
def test_degree_triples_double_bwd_edge_vectors(ctp, dev, deg, variant):
    """conv_tp_bwd_bwd_vec against the oracle, with dY recomputed and with the
    first backward's dY passed in (the same bits)."""
    prob, d = workload(deg, 50, 64, variant, seed=17 + variant)
    n, l_sh = d["n_nodes"], deg[1]
    rng = np.random.default_rng(7)
    ax = rng.standard_normal(d["x"].shape, dtype=np.float32)
    aw = rng.standard_normal(d["w"].shape, dtype=np.float32)
    av = rng.standard_normal((d["n_edges"], 3), dtype=np.float32)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    G, x, w, vt = T(d["grad_out"], dev), T(d["x"], dev), T(d["w"], dev), T(d["vec"], dev)
    args = (G, x, vt, w, T(ax, dev), T(aw, dev), T(av, dev), g, deg)
    res = ctp.conv_tp_bwd_bwd_vec(*args, variant=variant)
    v64 = d["vec"].astype(np.float64)
    Y = osh.real_sh(l_sh, v64)
    aY = osh.real_sh_jvp(l_sh, v64, av)
    rx, rw, rY, rG = oc.materialised_double_bwd(prob, d["x"], Y, d["w"], d["grad_out"], ax, aw, aY,
                                                d["row_ptr"], d["senders"])
    _, _, dY = oc.materialised_bwd(prob, d["x"], Y, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    rvec = osh.vec_grad_from_sh_grad(l_sh, v64, rY) + osh.vec_hess_term(l_sh, v64, dY, av)
    for name, got, want in zip(("g_x", "g_w", "g_vec", "g_grad"), res, (rx, rw, rvec, rG)):
        close(name, host(got), want)
    dYt = ctp.conv_tp_bwd(G, x, ctp.spherical_harmonics(vt, l_sh), w, g, deg, ctp.Y_GIVEN, variant=variant)[2]
    for u, v in zip(res, ctp.conv_tp_bwd_bwd_vec(*args, variant=variant, dY=dYt)):
        assert torch.equal(u, v)


def test_double_bwd_edge_vectors_nodes_without_edges(ctp, dev):
    """Nodes but no edges: g_x and g_grad come out zero, the per-edge outputs
    are empty, with and without dY."""
    n, c, deg = 12, 64, (2, 2, 2)
    prob = oc.Problem(*deg)
    g = ctp.Graph(n, torch.zeros(n + 1, dtype=torch.int32, device=dev), torch.zeros(0, dtype=torch.int32, device=dev))
    x = torch.randn(n, prob.D1, c, device=dev)
    G = torch.randn(n, prob.D3, c, device=dev)
    w = torch.zeros(0, prob.P, c, device=dev)
    v = torch.zeros(0, 3, device=dev)
    for dY in (None, torch.zeros(0, 9, device=dev)):
        gx, gw, gv, gG = ctp.conv_tp_bwd_bwd_vec(G, x, v, w, torch.randn_like(x), w.clone(), v.clone(), g, deg,
                                                 dY=dY)
        assert gw.numel() == 0 and gv.numel() == 0
        assert torch.count_nonzero(gx) == 0 and torch.count_nonzero(gG) == 0


@pytest.mark.parametrize("deg", [(0, 3, 3), (2, 1, 3), (3, 3, 3)])
def test_degree_triples_frame_forward(ctp, dev, deg):
    prob, d = workload(deg, 80, 64, 0, seed=3)
    n = d["n_nodes"]
    vec = d["vec"].copy()
    vec[::29] = 0.0                     # zero vectors: D = identity, l2 >= 1 paths dropped
    vec[1::31] = (0.0, 0.0, -1.0)       # south pole
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    out = ctp.conv_tp_fwd(T(d["x"], dev), T(vec, dev), T(d["w"], dev), g, deg, ctp.VEC_GIVEN, ctp.ALGO_FRAME)
    ref = oc.fwd(prob, d["x"], osh.real_sh(deg[1], vec.astype(np.float64)), d["w"], d["row_ptr"], d["senders"])
    close("out(frame)", host(out), ref)


# ------------------------------------------------------------ up to 1024 channels in every backward


@pytest.mark.parametrize("c", [1024, 640, 513])
@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("y_mode", [0, 1])
def test_backward_up_to_1024_channels(ctp, dev, c, variant, y_mode):
    check_all(ctp, dev, (2, 2, 2), 30, c, variant, y_mode, seed=c + variant)


def test_backward_1024_channels_l3_unsplit_and_deterministic(ctp, dev):
    # 300 senders x 2 tiles x 8 waves is above the split threshold (4096
    # waves): the unsplit backward grid at C = 1024, lmax 3
    deg, n, c = (3, 3, 3), 300, 1024
    for y_mode in (0, 1):
        prob, d = check_all(ctp, dev, deg, n, c, 0, y_mode, seed=2, msg=False)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G, vec = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev), T(d["vec"], dev)
    first = ctp.conv_tp_bwd(G, x, vec, w, g, deg, ctp.VEC_GIVEN)
    for _ in range(2):
        again = ctp.conv_tp_bwd(G, x, vec, w, g, deg, ctp.VEC_GIVEN)
        for u, v in zip(first, again):
            assert torch.equal(u, v)


@pytest.mark.parametrize("variant", [0, 1])
def test_double_bwd_1024_channels(ctp, dev, variant):
    deg = (2, 2, 2)
    prob, d = workload(deg, 24, 1024, variant, seed=41 + variant)
    Y = osh.real_sh(2, d["vec"].astype(np.float64)).astype(np.float32)
    rng = np.random.default_rng(7)
    ax = rng.standard_normal(d["x"].shape, dtype=np.float32)
    aw = rng.standard_normal(d["w"].shape, dtype=np.float32)
    aY = rng.standard_normal(Y.shape, dtype=np.float32)
    g = ctp.Graph(24, T(d["row_ptr"], dev), T(d["senders"], dev))
    args = (T(d["grad_out"], dev), T(d["x"], dev), T(Y, dev), T(d["w"], dev), T(ax, dev), T(aw, dev), T(aY, dev))
    res = ctp.conv_tp_bwd_bwd(*args, g, deg, variant=variant)
    ref = oc.materialised_double_bwd(prob, d["x"], Y, d["w"], d["grad_out"], ax, aw, aY, d["row_ptr"],
                                     d["senders"])
    for name, got, want in zip(("g_x", "g_w", "g_y", "g_grad"), res, ref):
        close(name, host(got), want)
    again = ctp.conv_tp_bwd_bwd(*args, g, deg, variant=variant)
    for u, v in zip(res, again):
        assert torch.equal(u, v)


# ------------------------------------------------------------ backward in each edge's frame (algo 2)


def check_frame_bwd(ctp, dev, deg, n, c, seed, vec_edit=None, mean_deg=10.0):
    prob, d = workload(deg, n, c, 0, seed, mean_deg=mean_deg)
    vec = d["vec"].copy()
    if vec_edit is not None:
        vec_edit(vec)
    l_sh = deg[1]
    v64 = vec.astype(np.float64)
    Y = osh.real_sh(l_sh, v64)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G, vt = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev), T(vec, dev)
    print(f"[frame bwd] deg={deg} n={n} c={c}", flush=True)
    dx, dw, dvec = ctp.conv_tp_bwd(G, x, vt, w, g, deg, ctp.VEC_GIVEN, algo=ctp.ALGO_FRAME)
    sp, pe, sr = og.transpose(n, d["row_ptr"], d["senders"])
    close("dx", host(dx), oc.bwd_dx(prob, Y, d["w"], d["grad_out"], sp, pe, sr))
    ref_dw, ref_dY = oc.bwd_edges(prob, d["x"], Y, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    close("dw", host(dw), ref_dw)
    close("dvec", host(dvec), osh.vec_grad_from_sh_grad(l_sh, v64, ref_dY),
          nonzero=any(p[1] > 0 for p in prob.paths))
    again = ctp.conv_tp_bwd(G, x, vt, w, g, deg, ctp.VEC_GIVEN, algo=ctp.ALGO_FRAME)
    for u, v in zip((dx, dw, dvec), again):
        assert torch.equal(u, v)


@pytest.mark.parametrize("deg", TRIPLES + [(3, 3, 3), (1, 1, 1)])
def test_frame_backward_small(ctp, dev, deg):
    check_frame_bwd(ctp, dev, deg, 70, 96, seed=sum(deg) + 40)


def test_frame_backward_poles_and_zero_vectors(ctp, dev):
    def edit(v):
        v[::17] = 0.0                        # zero vectors: only the l2 = 0 paths, dvec = 0
        v[1::19] = (0.0, 0.0, 1.0)           # north pole
        v[2::23] = (0.0, 0.0, -1.0)          # south pole
        v[3::29] = (1e-4, -2e-4, -0.7)       # near the south pole
        v[4::31] *= 7.5                      # lengths other than one
    check_frame_bwd(ctp, dev, (3, 3, 3), 60, 64, seed=77, vec_edit=edit)
    check_frame_bwd(ctp, dev, (2, 3, 1), 60, 64, seed=78, vec_edit=edit)


@pytest.mark.parametrize("c", [1024, 640, 128])
def test_frame_backward_channel_tiles_and_unsplit_grid(ctp, dev, c):
    # N = 4096 at C >= 128 is above the small-grid split threshold
    n = 4096 if c == 128 else 30
    check_frame_bwd(ctp, dev, (3, 3, 3), n, c, seed=c, mean_deg=3.0 if n > 100 else 10.0)


def test_frame_backward_rejections(ctp, dev):
    prob, d = workload((2, 2, 2), 10, 16, 0, seed=1)
    g = ctp.Graph(10, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev)
    Y = T(osh.real_sh(2, d["vec"].astype(np.float64)).astype(np.float32), dev)
    with pytest.raises(ctp.ConvTPError):
        ctp.conv_tp_bwd(G, x, Y, w, g, 2, ctp.Y_GIVEN, algo=ctp.ALGO_FRAME)


# ------------------------------------------------------------ small grids: edge lists split between workgroups


def skewed_graph(n, c, l_in, l_sh, n_paths, out_dim, seed):
    """In-degrees 0, 1, 2, ... 13, 25 and a hub of 300, and the same out-degrees
    in another node order (edges paired at random), so that both the receiver
    lists (the forward) and the sender lists (the backward) run shorter than,
    equal to and longer than every chunk count; a few zero and polar edge
    vectors."""
    rng = np.random.default_rng(seed)
    indeg = np.array([(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 13, 25)[k % 13] for k in range(n)])
    indeg[n // 2] = 300
    recv = np.repeat(np.arange(n), indeg)
    e = recv.size
    send = rng.permutation(np.repeat(rng.permutation(n), indeg)).astype(np.int32)
    vec = rng.standard_normal((e, 3)).astype(np.float32)
    vec[::29] = 0.0
    vec[1::31] = (0.0, 0.0, 1.5)
    vec[2::37] = (0.0, 0.0, -0.5)
    d1, d2 = (l_in + 1) ** 2, (l_sh + 1) ** 2
    return dict(n_nodes=n, n_edges=e, row_ptr=og.row_ptr_from_receivers(recv, n), senders=send, vec=vec,
                x=rng.standard_normal((n, d1, c)).astype(np.float32),
                w=rng.standard_normal((e, n_paths, c)).astype(np.float32),
                grad_out=rng.standard_normal((n, out_dim, c)).astype(np.float32))


@pytest.mark.parametrize("c", [16, 64, 100, 128, 192, 256, 320])
def test_frame_small_grid_split(ctp, dev, c):
    """Edge-frame forward and backward on grids small enough to split every
    edge list between two workgroups (lists of 0, 1, 2, ... edges and a hub),
    at one to five waves of channels: element by element against the oracle,
    bitwise equal reruns."""
    deg = (3, 3, 3) if c <= 128 else (2, 3, 1)
    prob = oc.Problem(*deg)
    n = 40
    d = skewed_graph(n, c, deg[0], deg[1], prob.P, prob.D3, seed=c)
    v64 = d["vec"].astype(np.float64)
    Y = osh.real_sh(deg[1], v64)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G, vt = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev), T(d["vec"], dev)
    print(f"[frame split] deg={deg} n={n} e={d['n_edges']} c={c}", flush=True)
    out = ctp.conv_tp_fwd(x, vt, w, g, deg, ctp.VEC_GIVEN, ctp.ALGO_FRAME)
    close("out", host(out), oc.fwd(prob, d["x"], Y, d["w"], d["row_ptr"], d["senders"]))
    assert torch.equal(out, ctp.conv_tp_fwd(x, vt, w, g, deg, ctp.VEC_GIVEN, ctp.ALGO_FRAME))
    dx, dw, dvec = ctp.conv_tp_bwd(G, x, vt, w, g, deg, ctp.VEC_GIVEN, algo=ctp.ALGO_FRAME)
    sp, pe, sr = og.transpose(n, d["row_ptr"], d["senders"])
    close("dx", host(dx), oc.bwd_dx(prob, Y, d["w"], d["grad_out"], sp, pe, sr))
    ref_dw, ref_dY = oc.bwd_edges(prob, d["x"], Y, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    close("dw", host(dw), ref_dw)
    close("dvec", host(dvec), osh.vec_grad_from_sh_grad(deg[1], v64, ref_dY))
    for u, v in zip((dx, dw, dvec), ctp.conv_tp_bwd(G, x, vt, w, g, deg, ctp.VEC_GIVEN, algo=ctp.ALGO_FRAME)):
        assert torch.equal(u, v)

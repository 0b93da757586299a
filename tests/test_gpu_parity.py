"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bar: for every output tensor, max |gpu - oracle| <= 1e-4 * max |oracle|
(fp32 kernels vs fp64 oracle); index arrays bit-exact; the deterministic
kernels bitwise reproducible run to run.  Small workloads are compared
element by element; full-size workloads on seeded samples of receivers,
senders and edges that the oracle evaluates one by one.
"""
import math

import numpy as np
import pytest
import torch

from oracle import convtp as oc
from oracle import graph as og
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


def close(name, got, ref, nonzero=True):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if nonzero:
        assert scale > 0.0, f"{name}: reference is identically zero"
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert np.isfinite(got).all(), name
    assert err <= RTOL * scale or err == 0.0, f"{name}: max err {err:.3e} vs scale {scale:.3e}"


def T(a, dev, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev)


def host(t):
    return t.detach().cpu().numpy()


def sh32(L, vec):
    return osh.real_sh(L, np.asarray(vec, dtype=np.float64)).astype(np.float32)


# ------------------------------------------------------------ small workloads, full comparison


def run_small(ctp, dev, d, L, y_mode, algo=0, bwd=True, variant=0):
    n, e = d["n_nodes"], d["n_edges"]
    prob = oc.Problem(L, L, L, variant=variant)
    vec = d["vec"]
    Y = sh32(L, vec)
    yin = Y if y_mode == 0 else vec
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w = T(d["x"], dev), T(d["w"], dev)
    yv = T(yin, dev)
    out = ctp.conv_tp_fwd(x, yv, w, g, L, y_mode, algo, variant=variant)
    # oracle: Y mode sees the same fp32 Y; vec mode sees fp64 harmonics of the same vec
    Yref = Y.astype(np.float64) if y_mode == 0 else osh.real_sh(L, vec.astype(np.float64))
    ref = oc.fwd(prob, d["x"], Yref, d["w"], d["row_ptr"], d["senders"])
    close("out", host(out), ref)
    if not bwd:
        return
    G = T(d["grad_out"], dev)
    dx, dw, dy = ctp.conv_tp_bwd(G, x, yv, w, g, L, y_mode, variant=variant)
    sp, pe, sr = og.transpose(n, d["row_ptr"], d["senders"])
    close("dx", host(dx), oc.bwd_dx(prob, Yref, d["w"], d["grad_out"], sp, pe, sr))
    dw_ref, dY_ref = oc.bwd_edges(prob, d["x"], Yref, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    close("dw", host(dw), dw_ref)
    if y_mode == 0:
        close("dY", host(dy), dY_ref)
    else:
        # lmax = 0: Y_00 is constant, so the edge-vector gradient is exactly zero
        close("dvec", host(dy), osh.vec_grad_from_sh_grad(L, vec.astype(np.float64), dY_ref), nonzero=L > 0)


@pytest.mark.parametrize("y_mode", [0, 1])
@pytest.mark.parametrize("algo", [0, 1])
def test_tiny(ctp, dev, y_mode, algo):
    run_small(ctp, dev, gen.tiny(), 1, y_mode, algo, bwd=(algo == 0))


SMALL = [  # (N, C, L): several channel tiles, ragged lane tails, every degree
    (90, 16, 1), (150, 48, 2), (120, 128, 2), (100, 128, 3), (70, 64, 3),
    (60, 192, 3), (50, 256, 2), (40, 512, 2), (30, 1024, 2), (40, 96, 0), (60, 128, 0),
]


@pytest.mark.parametrize("n,c,L", SMALL)
@pytest.mark.parametrize("y_mode", [0, 1])
def test_small_poisson(ctp, dev, n, c, L, y_mode):
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=n + c + L)
    run_small(ctp, dev, d, L, y_mode, 0, bwd=True)
    run_small(ctp, dev, d, L, y_mode, 1, bwd=False)


@pytest.mark.parametrize("L", [2, 3])
@pytest.mark.parametrize("y_mode", [0, 1])
def test_many_receivers(ctp, dev, L, y_mode):
    # 8192 receivers at C = 128 (16384 forward waves, the full-size grid's
    # shape), element by element; a sparse graph keeps the oracle fast.
    d = gen.poisson_small(8192, 128, L, mean_deg=3.0, seed=7 + L)
    run_small(ctp, dev, d, L, y_mode, 0, bwd=False)


@pytest.mark.parametrize("n,c,L", [(4096, 64, 3), (2048, 128, 2)])
@pytest.mark.parametrize("y_mode", [0, 1])
def test_unsplit_rows(ctp, dev, n, c, L, y_mode):
    # Grids of fewer than 4096 waves split every edge list between two
    # workgroups (partial sums added with two fp32 atomics onto zero); these
    # sizes are just large enough to take the unsplit path, element by element.
    d = gen.poisson_small(n, c, L, mean_deg=3.0, seed=n + c)
    run_small(ctp, dev, d, L, y_mode, 0, bwd=True)


def test_deterministic_reruns(ctp, dev):
    d = gen.poisson_small(300, 128, 3, mean_deg=45.0, seed=5)
    g = ctp.Graph(300, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev)
    for y_mode, y in ((0, T(sh32(3, d["vec"]), dev)), (1, T(d["vec"], dev))):
        a = ctp.conv_tp_fwd(x, y, w, g, 3, y_mode)
        b = ctp.conv_tp_fwd(x, y, w, g, 3, y_mode)
        assert torch.equal(a, b)
        r1 = ctp.conv_tp_bwd(G, x, y, w, g, 3, y_mode)
        r2 = ctp.conv_tp_bwd(G, x, y, w, g, 3, y_mode)
        for u, v in zip(r1, r2):
            assert torch.equal(u, v)


@pytest.mark.parametrize("n,c", [(300, 128), (4096, 64)])
def test_hip_graph_replays(ctp, dev, n, c):
    """The forward and both backward entry points enqueue kernels only, so a
    HIP graph (torch.cuda.graph) captures them; every replay, with eager work
    on the outputs in between, gives the eager results bitwise.  (300, 128)
    takes the small-grid split, whose zeroing is a kernel, not a memset;
    (4096, 64) the unsplit path."""
    L = 3
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=n + c)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    g.transpose
    x, w, G = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev)
    y = T(sh32(L, d["vec"]), dev)
    e = d["n_edges"]
    ws = torch.empty(e * 16 * c, device=dev)
    outs = [torch.empty_like(x)] + [torch.empty_like(t) for t in (x, w, y)] + [torch.empty_like(t) for t in (x, w, y)]

    def run():
        ctp.conv_tp_fwd(x, y, w, g, L, 0, out=outs[0])
        ctp.conv_tp_bwd(G, x, y, w, g, L, 0, dx=outs[1], dw=outs[2], dy=outs[3])
        ctp.conv_tp_bwd_msg(G, x, y, w, g, L, 0, dx=outs[4], dw=outs[5], dy=outs[6], workspace=ws)

    print(f"graph capture n={n} c={c}", flush=True)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for k in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "dx", "dw", "dY", "dx msg", "dw msg", "dY msg"), outs, ref):
            assert torch.equal(a, b), (k, name)


def test_hip_graph_replays_frame_and_dy(ctp, dev):
    """The edge-frame forward (small-grid split: its zero fill is a kernel) and
    dY alone, captured in a HIP graph and replayed with eager work between."""
    L, n, c = 3, 300, 128
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=77)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G, v = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev), T(d["vec"], dev)
    out, dy = torch.empty_like(x), torch.empty(d["n_edges"], 16, device=dev)

    def run():
        ctp.conv_tp_fwd(x, v, w, g, L, 1, ctp.ALGO_FRAME, out=out)
        ctp.conv_tp_bwd_dy(G, x, w, g, L, dy=dy)

    print("graph capture frame + dy", flush=True)
    run()
    torch.cuda.synchronize()
    ref = (out.clone(), dy.clone())
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for k in range(3):
        out.fill_(float("nan"))
        dy.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(dy, ref[1]), k


def test_hip_graph_replays_frame_bwd_atomic_bwd_and_vec_double_bwd(ctp, dev):
    """The edge-frame backward (small-grid split, dx zero fill), the atomic
    backward (algo 1, dx zero fill) and the one-call edge-vector double
    backward (workspace, first backward's dY given), captured in one HIP graph
    and replayed three times: every output equals the eager run bitwise,
    except the atomic backward's dx (additions in any order: to tolerance)."""
    L, n, c = 3, 300, 128
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=78)
    e = d["n_edges"]
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G, v = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev), T(d["vec"], dev)
    rng = np.random.default_rng(5)
    ax, aw = T(rng.standard_normal(d["x"].shape, dtype=np.float32), dev), T(rng.standard_normal(d["w"].shape, dtype=np.float32), dev)
    av = T(rng.standard_normal((e, 3), dtype=np.float32), dev)
    Y = ctp.spherical_harmonics(v, L)
    dY = ctp.conv_tp_bwd(G, x, Y, w, g, L, ctp.Y_GIVEN)[2]
    outs = [torch.empty_like(x), torch.empty_like(w), torch.empty_like(v),                 # frame bwd
            torch.empty_like(x), torch.empty_like(w), torch.empty_like(Y),                 # atomic bwd
            torch.empty_like(x), torch.empty_like(w), torch.empty_like(v), torch.empty_like(G)]   # dd vec
    ws = torch.empty(3 * e * 16, device=dev)

    def run():
        ctp.conv_tp_bwd(G, x, v, w, g, L, ctp.VEC_GIVEN, dx=outs[0], dw=outs[1], dy=outs[2], algo=ctp.ALGO_FRAME)
        ctp.conv_tp_bwd(G, x, Y, w, g, L, ctp.Y_GIVEN, dx=outs[3], dw=outs[4], dy=outs[5], algo=ctp.ALGO_ATOMIC)
        ctp.conv_tp_bwd_bwd_vec(G, x, v, w, ax, aw, av, g, L, dY=dY, out=tuple(outs[6:]), workspace=ws)

    print("graph capture frame bwd + atomic bwd + dd vec", flush=True)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            run()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for k in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for q, (a, b) in enumerate(zip(outs, ref)):
            if q == 3:
                close("atomic dx", host(a), host(b))
            else:
                assert torch.equal(a, b), (k, q)


def test_random_shapes_every_entry_point(ctp, dev):
    """Seeded random problems (independent degrees, channel count including
    ragged ones and two backward channel tiles, graph size with empty rows,
    both Y modes, both variants) through every conv entry point: forward algos
    0/1/2, backward algos 0/1/2, message backward and dY alone, each against
    the oracle."""
    rng = np.random.default_rng(2024)
    for case in range(32):
        deg = tuple(int(v) for v in rng.integers(0, 4, size=3))
        L = deg[1]          # harmonics degree
        c = int(rng.choice([1, 3, 17, 64, 65, 100, 128, 129, 200, 256, 300, 513, 700, 1024]))
        n = int(rng.integers(2, 60))
        e = int(rng.integers(0, 4 * n))
        variant = int(rng.integers(0, 2))
        y_mode = int(rng.integers(0, 2))
        recv = np.sort(rng.integers(0, n, size=e))
        pr = oc.Problem(*deg, variant=variant)
        d = dict(n_nodes=n, n_edges=e, row_ptr=og.row_ptr_from_receivers(recv, n),
                 senders=rng.integers(0, n, size=e).astype(np.int32),
                 vec=rng.standard_normal((e, 3)).astype(np.float32),
                 x=rng.standard_normal((n, pr.D1, c)).astype(np.float32),
                 w=rng.standard_normal((e, pr.P, c)).astype(np.float32),
                 grad_out=rng.standard_normal((n, pr.D3, c)).astype(np.float32))
        print(f"case {case}: deg={deg} c={c} n={n} e={e} variant={variant} y_mode={y_mode}", flush=True)
        Y = sh32(L, d["vec"])
        yin = Y if y_mode == 0 else d["vec"]
        Yref = Y.astype(np.float64) if y_mode == 0 else osh.real_sh(L, d["vec"].astype(np.float64))
        g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
        x, w, G, yv = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev), T(yin, dev)
        nz = e > 0
        ref = oc.fwd(pr, d["x"], Yref, d["w"], d["row_ptr"], d["senders"])
        algos = [0, 1] + ([2] if y_mode == 1 and variant == 0 else [])
        for algo in algos:
            close(f"out algo {algo}", host(ctp.conv_tp_fwd(x, yv, w, g, deg, y_mode, algo, variant=variant)), ref,
                  nonzero=nz)
        sp, pe, sr = og.transpose(n, d["row_ptr"], d["senders"])
        dx_ref = oc.bwd_dx(pr, Yref, d["w"], d["grad_out"], sp, pe, sr)
        dw_ref, dY_ref = oc.bwd_edges(pr, d["x"], Yref, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
        dy_ref = dY_ref if y_mode == 0 else osh.vec_grad_from_sh_grad(L, d["vec"].astype(np.float64), dY_ref)
        bwds = [("bwd", ctp.conv_tp_bwd), ("bwd_msg", ctp.conv_tp_bwd_msg),
                ("bwd algo 1", lambda *a, **k: ctp.conv_tp_bwd(*a, **k, algo=ctp.ALGO_ATOMIC))]
        if y_mode == 1 and variant == 0:
            bwds.append(("bwd algo 2", lambda *a, **k: ctp.conv_tp_bwd(*a, **k, algo=ctp.ALGO_FRAME)))
        for name, fn in bwds:
            dx, dw, dy = fn(G, x, yv, w, g, deg, y_mode, variant=variant)
            close(f"{name} dx", host(dx), dx_ref, nonzero=nz)
            close(f"{name} dw", host(dw), dw_ref, nonzero=nz)
            # with edge vectors dvec is exactly zero unless some path has l2 > 0
            close(f"{name} dy", host(dy), dy_ref, nonzero=nz and (y_mode == 0 or any(p[1] > 0 for p in pr.paths)))
        if y_mode == 0:
            close("dY alone", host(ctp.conv_tp_bwd_dy(G, x, w, g, deg, variant=variant)), dY_ref, nonzero=nz)


# ------------------------------------------------------------ bookkeeping and harmonics


@pytest.mark.parametrize("which", ["tiny", "poisson", "water", "skewed", "hubs"])
def test_transpose_bit_exact(ctp, dev, which):
    if which == "tiny":
        d = gen.tiny()
        n, rp, s = d["n_nodes"], d["row_ptr"], d["senders"]
    elif which == "poisson":
        n = 20000
        rp, s = gen.poisson_graph(n, 45.0, np.random.default_rng(3))
    elif which == "water":
        d = gen.water_box_graph()
        n, rp, s = d["n_nodes"], d["row_ptr"], d["senders"]
    else:   # one sender with 3000 out-edges, many isolated nodes
        n = 500
        rng = np.random.default_rng(4)
        recv = np.sort(rng.integers(0, n, size=4000))
        s = rng.integers(0, n, size=4000).astype(np.int32)
        s[rng.choice(4000, 3000, replace=False)] = 7
        rp = og.row_ptr_from_receivers(recv, n)
    if which == "hubs":
        # segments above the in-LDS sort size: one sender with 50,000 out-edges,
        # one with 4097 (just above 4096) and one with exactly 4096
        n = 3000
        rng = np.random.default_rng(12)
        e = 70000
        recv = np.sort(rng.integers(0, n, size=e))
        s = rng.integers(0, n, size=e).astype(np.int32)
        pick = rng.permutation(e)
        s[pick[:50000]] = 11
        s[pick[50000:54097]] = 12
        s[pick[54097:58193]] = 13
        s[pick[58193:]] = rng.integers(14, n, size=e - 58193)
        rp = og.row_ptr_from_receivers(recv, n)
    ref = og.transpose(n, rp, s)
    got = ctp.build_transpose(n, T(rp, dev), T(s, dev))
    for a, b in zip(got, ref):
        assert np.array_equal(host(a), b)
    assert ctp.check_graph(n, T(rp, dev), T(s, dev)) == 0


def test_check_graph_counts_defects(ctp, dev):
    n = 50
    rp, s = gen.poisson_graph(n, 6.0, np.random.default_rng(8))
    bad_s = s.copy()
    bad_s[[1, 5, 9]] = [n, -2, n + 100]
    bad_rp = rp.copy()
    bad_rp[10] = bad_rp[11] + 3
    for r, q in ((rp, bad_s), (bad_rp, s), (bad_rp, bad_s)):
        assert ctp.check_graph(n, T(r, dev), T(q, dev)) == og.check_graph(n, r, q)


@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_spherical_harmonics(ctp, dev, L):
    rng = np.random.default_rng(L)
    vec = (rng.standard_normal((5000, 3)) * rng.uniform(0.1, 10, size=(5000, 1))).astype(np.float32)
    vec[0] = 0.0
    vec[1] = (0.0, 0.0, 2.5)       # pole
    vec[2] = (0.0, 0.0, -1e-3)
    Y = ctp.spherical_harmonics(T(vec, dev), L)
    close("Y", host(Y), osh.real_sh(L, vec.astype(np.float64)))
    dY = rng.standard_normal((5000, (L + 1) ** 2)).astype(np.float32)
    dv = ctp.spherical_harmonics_backward(T(vec, dev), T(dY, dev), L)
    close("dvec", host(dv), osh.vec_grad_from_sh_grad(L, vec.astype(np.float64), dY), nonzero=L > 0)
    assert not host(dv)[0].any()


# ------------------------------------------------------------ edge cases


def test_empty_graph_gives_zeros(ctp, dev):
    n, c, L = 5, 128, 2
    rp = np.zeros(n + 1, dtype=np.int32)
    s = np.zeros(0, dtype=np.int32)
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    x = torch.randn(n, 9, c, device=dev)
    w = torch.empty(0, 15, c, device=dev)
    y = torch.empty(0, 9, device=dev)
    for algo in (0, 1):
        out = ctp.conv_tp_fwd(x, y, w, g, L, 0, algo)
        assert not out.any()
    dx, dw, dy = ctp.conv_tp_bwd(torch.randn_like(x), x, y, w, g, L, 0)
    assert not dx.any() and dw.numel() == 0 and dy.numel() == 0


def test_hub_self_edges_duplicates_and_zero_vectors(ctp, dev):
    """One receiver with in-degree 1000, isolated nodes, explicit self-edges,
    duplicate edges, zero-weight edges and zero edge vectors."""
    rng = np.random.default_rng(12)
    n, c, L = 40, 128, 3
    recv = np.concatenate([np.full(1000, 3), rng.integers(0, n, size=300)])
    recv[recv == 17] = 18                        # node 17 has no incoming edge
    recv = np.sort(recv)
    s = rng.integers(0, n, size=recv.size)
    s[s == 21] = 22                              # node 21 sends nothing
    s[:10] = recv[:10]                           # self-edges
    s[10:20] = s[20:30]
    rp = og.row_ptr_from_receivers(recv, n)
    e = recv.size
    vec = rng.standard_normal((e, 3)).astype(np.float32)
    vec[::37] = 0.0
    w = rng.standard_normal((e, 34, c)).astype(np.float32)
    w[::5] = 0.0
    d = dict(n_nodes=n, n_edges=e, row_ptr=rp, senders=s.astype(np.int32), vec=vec,
             x=rng.standard_normal((n, 16, c)).astype(np.float32), w=w,
             grad_out=rng.standard_normal((n, 16, c)).astype(np.float32))
    for y_mode in (0, 1):
        run_small(ctp, dev, d, L, y_mode, 0)
        run_small(ctp, dev, d, L, y_mode, 1, bwd=False)


# ------------------------------------------------------------ full-size workloads, sampled


def _sub_fwd(prob, rp, s, Yref, w_dev, x_host, rows):
    edges = np.concatenate([np.arange(rp[i], rp[i + 1]) for i in rows]).astype(np.int64)
    rp_sub = np.zeros(len(rows) + 1, dtype=np.int32)
    rp_sub[1:] = np.cumsum([rp[i + 1] - rp[i] for i in rows])
    w_sub = host(w_dev[torch.as_tensor(edges, device=w_dev.device)])
    # receivers renumbered 0..len(rows)-1; senders stay global
    return oc.fwd(prob, x_host, Yref[edges], w_sub, rp_sub, s[edges], rows=np.arange(len(rows)))


def _sub_dx(prob, rp, s, Yref, w_dev, G_host, senders_sel):
    recv = og.receivers_of(rp)
    pos = {j: k for k, j in enumerate(senders_sel)}
    edges = np.nonzero(np.isin(s, senders_sel))[0]
    loc = np.array([pos[j] for j in s[edges]], dtype=np.int64)
    order = np.argsort(loc, kind="stable")
    send_ptr = np.zeros(len(senders_sel) + 1, dtype=np.int32)
    send_ptr[1:] = np.cumsum(np.bincount(loc, minlength=len(senders_sel)))
    w_sub = host(w_dev[torch.as_tensor(edges, device=w_dev.device)])
    return oc.bwd_dx(prob, Yref[edges], w_sub, G_host, send_ptr, order.astype(np.int32),
                     recv[edges][order].astype(np.int32), rows=np.arange(len(senders_sel)))


def _sub_edges(prob, rp, s, Yref, w_dev, x_host, G_host, edges):
    recv = og.receivers_of(rp)[edges]
    rp_sub = og.row_ptr_from_receivers(recv, len(rp) - 1)
    w_sub = host(w_dev[torch.as_tensor(edges, device=w_dev.device)])
    return oc.bwd_edges(prob, x_host, Yref[edges], w_sub, G_host, rp_sub, s[edges])


def run_full(ctp, dev, n, c, L, y_mode, algo=0, bwd=False, seed=0, n_sample=48):
    d = gen.poisson_full(n, c, L, dev, seed=seed, need_grad=bwd)
    rp, s, vec = d["row_ptr"], d["senders"], d["vec"]
    prob = oc.Problem(L, L, L)
    Y = sh32(L, vec)
    yin = T(Y if y_mode == 0 else vec, dev)
    Yref = Y.astype(np.float64) if y_mode == 0 else osh.real_sh(L, vec.astype(np.float64))
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    out = ctp.conv_tp_fwd(d["x"], yin, d["w"], g, L, y_mode, algo)
    rng = np.random.default_rng(seed + 99)
    rows = np.sort(rng.choice(n, n_sample, replace=False))
    x_host = host(d["x"])
    close("out[sample]", host(out[torch.as_tensor(rows, device=dev)]),
          _sub_fwd(prob, rp, s, Yref, d["w"], x_host, rows))
    del out
    if not bwd:
        return
    dx, dw, dy = ctp.conv_tp_bwd(d["grad_out"], d["x"], yin, d["w"], g, L, y_mode, algo=algo)
    G_host = host(d["grad_out"])
    close("dx[sample]", host(dx[torch.as_tensor(rows, device=dev)]),
          _sub_dx(prob, rp, s, Yref, d["w"], G_host, rows))
    edges = np.sort(rng.choice(len(s), 4 * n_sample, replace=False))
    dw_ref, dY_ref = _sub_edges(prob, rp, s, Yref, d["w"], x_host, G_host, edges)
    ei = torch.as_tensor(edges, device=dev)
    close("dw[sample]", host(dw[ei]), dw_ref)
    if y_mode == 0:
        close("dY[sample]", host(dy[ei]), dY_ref)
    else:
        close("dvec[sample]", host(dy[ei]), osh.vec_grad_from_sh_grad(L, vec[edges].astype(np.float64), dY_ref))


def test_full_l2_forward(ctp, dev):
    """lmax=2, N=32768, C=128 (N*C = 2^22), Poisson(45) in-degrees."""
    run_full(ctp, dev, 32768, 128, 2, 0)


@pytest.mark.parametrize("y_mode", [0, 1])
def test_full_l3_forward_backward(ctp, dev, y_mode):
    """lmax=3, N=16384, C=128 (N*C = 2^21), forward and backward."""
    run_full(ctp, dev, 16384, 128, 3, y_mode, bwd=True)


def test_full_l3_edge_frame_forward_backward(ctp, dev):
    """lmax=3, N=16384, C=128, edge vectors, forward and backward in each
    edge's frame (algo 2), as `bench.py --vec --frame` times them."""
    run_full(ctp, dev, 16384, 128, 3, 1, algo=2, bwd=True, seed=3)


@pytest.mark.parametrize("c", gen.SWEEP_CHANNELS)
@pytest.mark.parametrize("algo", [0, 1])
def test_full_channel_sweep(ctp, dev, c, algo):
    """lmax=2 forward, N = 2^22 / C, both the CSR and the atomic variant."""
    run_full(ctp, dev, (1 << 22) // c, c, 2, 0, algo=algo, n_sample=24)
    torch.cuda.empty_cache()


class _DevRows:
    """Rows of a device array fetched when indexed (fp64 on the host), mapped
    by `fn` if given (edge vectors -> harmonics), so that the sampled oracle
    helpers never copy a multi-GB array whole."""

    def __init__(self, t, fn=None):
        self.t, self.fn = t, fn

    def __getitem__(self, idx):
        i = torch.as_tensor(np.asarray(idx, dtype=np.int64), device=self.t.device)
        a = host(self.t[i]).astype(np.float64)
        return a if self.fn is None else self.fn(a)


def test_offsets_beyond_int32(ctp, dev):
    """lmax=3, C=2, 2^20 receivers of in-degree 40: E = 41.9M edges, so w and
    dw hold E*P*C = 2.85e9 elements (11.4 GB) and the rows of the last edges
    lie beyond 2^31 elements and 2^32 bytes.  Every entry point that indexes
    edge rows (forward CSR and atomic; backward direct, atomic and through
    messages; dY alone; the VJP of the VJP; edge vectors direct and in the
    edge frame) is compared with the oracle on samples that include the last
    receivers, the last edges and the senders of the last edges."""
    n, deg, c, L = 1 << 20, 40, 2, 3
    print("large offsets: inputs", flush=True)
    d = gen.fixed_degree_large(n, deg, c, L, dev, seed=5)
    rp, s, e = d["row_ptr"], d["senders"], d["n_edges"]
    assert e * gen.num_paths(L) * c > 2**31
    prob = oc.Problem(L, L, L)
    x, w, G, Y, vec = d["x"], d["w"], d["grad_out"], d["y"], d["vec"]
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([np.arange(n - 6, n), rng.choice(n, 10, replace=False)]))
    edges = np.unique(np.concatenate([np.arange(e - 12, e), rng.choice(e, 36, replace=False)]))
    send_sel = np.unique(np.concatenate([s[e - 6:], rng.choice(n, 6, replace=False)]))
    ri, si, ei = (torch.as_tensor(a, device=dev) for a in (rows, send_sel, edges))
    x_h, G_h = host(x), host(G)
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    g.transpose

    Yr = _DevRows(Y)
    ref_out = _sub_fwd(prob, rp, s, Yr, w, x_h, rows)
    ref_dx = _sub_dx(prob, rp, s, Yr, w, G_h, send_sel)
    ref_dw, ref_dY = _sub_edges(prob, rp, s, Yr, w, x_h, G_h, edges)
    for algo in (ctp.ALGO_CSR, ctp.ALGO_ATOMIC):
        print(f"large offsets: forward algo {algo}", flush=True)
        out = ctp.conv_tp_fwd(x, Y, w, g, L, ctp.Y_GIVEN, algo)
        close(f"out[sample] algo {algo}", host(out[ri]), ref_out)
        del out
    bwds = (("bwd algo 0", lambda: ctp.conv_tp_bwd(G, x, Y, w, g, L)),
            ("bwd algo 1", lambda: ctp.conv_tp_bwd(G, x, Y, w, g, L, algo=ctp.ALGO_ATOMIC)),
            ("bwd_msg", lambda: ctp.conv_tp_bwd_msg(G, x, Y, w, g, L)))
    for name, run in bwds:
        print(f"large offsets: {name}", flush=True)
        dx, dw, dy = run()
        close(f"dx[sample] {name}", host(dx[si]), ref_dx)
        close(f"dw[sample] {name}", host(dw[ei]), ref_dw)
        close(f"dY[sample] {name}", host(dy[ei]), ref_dY)
        del dx, dw, dy
        torch.cuda.empty_cache()
    print("large offsets: bwd_dy", flush=True)
    close("dY[sample] bwd_dy", host(ctp.conv_tp_bwd_dy(G, x, w, g, L)[ei]), ref_dY)

    print("large offsets: double backward", flush=True)
    ax = gen.normal_tensor(x.shape, 5, 26, dev)
    aw = gen.normal_tensor(w.shape, 5, 27, dev)
    aY = gen.normal_tensor(Y.shape, 5, 28, dev)
    gx, gw, gy, gG = ctp.conv_tp_bwd_bwd(G, x, Y, w, ax, aw, aY, g, L)
    ax_h, aYr = host(ax), _DevRows(aY)
    close("g_grad[sample]", host(gG[ri]),
          _sub_fwd(prob, rp, s, Yr, w, ax_h, rows) + _sub_fwd(prob, rp, s, Yr, aw, x_h, rows)
          + _sub_fwd(prob, rp, s, aYr, w, x_h, rows))
    close("g_x[sample]", host(gx[si]),
          _sub_dx(prob, rp, s, Yr, aw, G_h, send_sel) + _sub_dx(prob, rp, s, aYr, w, G_h, send_sel))
    dw1, dY1 = _sub_edges(prob, rp, s, Yr, w, ax_h, G_h, edges)
    dw2, _ = _sub_edges(prob, rp, s, aYr, w, x_h, G_h, edges)
    _, dY3 = _sub_edges(prob, rp, s, Yr, aw, x_h, G_h, edges)
    close("g_w[sample]", host(gw[ei]), dw1 + dw2)
    close("g_y[sample]", host(gy[ei]), dY1 + dY3)
    del ax, aw, aY, gx, gw, gy, gG, Y
    torch.cuda.empty_cache()

    Vr = _DevRows(vec, lambda v: osh.real_sh(L, v))
    ref_out = _sub_fwd(prob, rp, s, Vr, w, x_h, rows)
    ref_dx = _sub_dx(prob, rp, s, Vr, w, G_h, send_sel)
    ref_dw, ref_dY = _sub_edges(prob, rp, s, Vr, w, x_h, G_h, edges)
    ref_dvec = osh.vec_grad_from_sh_grad(L, host(vec[ei]).astype(np.float64), ref_dY)
    for algo in (ctp.ALGO_CSR, ctp.ALGO_FRAME):
        print(f"large offsets: edge vectors algo {algo}", flush=True)
        out = ctp.conv_tp_fwd(x, vec, w, g, L, ctp.VEC_GIVEN, algo)
        close(f"out[sample] vec algo {algo}", host(out[ri]), ref_out)
        del out
        dx, dw, dv = ctp.conv_tp_bwd(G, x, vec, w, g, L, ctp.VEC_GIVEN, algo=algo)
        close(f"dx[sample] vec algo {algo}", host(dx[si]), ref_dx)
        close(f"dw[sample] vec algo {algo}", host(dw[ei]), ref_dw)
        close(f"dvec[sample] vec algo {algo}", host(dv[ei]), ref_dvec)
        del dx, dw, dv
        torch.cuda.empty_cache()
    del d, x, w, G, vec
    torch.cuda.empty_cache()


def test_water_box_two_layers(ctp, dev):
    """1503 atoms, 83,325 padded edges, C=128, lmax=3, vec mode: two chained
    layers forward, then backward to the edge vectors (sum of both layers)."""
    wb = gen.water_box(seed=0, device="cpu")
    n, L = wb["n_nodes"], 3
    prob = oc.Problem(L, L, L)
    vec = wb["vec"]
    g = ctp.Graph(n, T(wb["row_ptr"], dev), T(wb["senders"], dev))
    v = T(vec, dev)
    w1, w2 = wb["w1"].numpy(), wb["w2"].numpy()
    x0 = T(wb["x"], dev)
    h1 = ctp.conv_tp_fwd(x0, v, T(w1, dev), g, L, 1)
    h2 = ctp.conv_tp_fwd(h1, v, T(w2, dev), g, L, 1)
    G = T(wb["grad_out"], dev)
    dh1, dw2, dv2 = ctp.conv_tp_bwd(G, h1, v, T(w2, dev), g, L, 1)
    dx0, dw1, dv1 = ctp.conv_tp_bwd(dh1, x0, v, T(w1, dev), g, L, 1)
    # oracle chain from the same inputs (C edge loop, fp64 accumulation; its
    # fp64 layer-1 results are rounded to fp32 where they feed layer 2)
    Yref = osh.real_sh(L, vec.astype(np.float64))
    rp, s = wb["row_ptr"], wb["senders"]
    sp, pe, sr = og.transpose(n, rp, s)
    r1 = oc.fwd(prob, wb["x"], Yref, w1, rp, s)
    r2 = oc.fwd(prob, r1, Yref, w2, rp, s)
    close("h1", host(h1), r1)
    close("h2", host(h2), r2)
    rdh1 = oc.bwd_dx(prob, Yref, w2, wb["grad_out"], sp, pe, sr)
    rdw2, rdY2 = oc.bwd_edges(prob, r1, Yref, w2, wb["grad_out"], rp, s)
    rdx0 = oc.bwd_dx(prob, Yref, w1, rdh1, sp, pe, sr)
    rdw1, rdY1 = oc.bwd_edges(prob, wb["x"], Yref, w1, rdh1, rp, s)
    close("dh1", host(dh1), rdh1)
    close("dx0", host(dx0), rdx0)
    close("dw1", host(dw1), rdw1)
    close("dw2", host(dw2), rdw2)
    dvec_ref = osh.vec_grad_from_sh_grad(L, vec.astype(np.float64), rdY1 + rdY2)
    close("dvec", host(dv1) + host(dv2), dvec_ref)
    # padded edges (zero weight) contribute no weight gradient to the model: w is masked
    assert not host(T(w1, dev))[wb["mask"] == 0].any()
    assert math.isfinite(float(host(h2).sum()))


def test_stream_probes(ctp, dev):
    # measurement helper: the copy is exact, read and write run to completion
    n = (1 << 20) + 4 * 1000 + 4      # ragged against the grid stride and the 4-deep copy loop
    src = torch.randn(n, device=dev)
    dst = torch.zeros(n, device=dev)
    ctp.stream_probe(ctp.STREAM_COPY, src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    sink = torch.zeros(4, device=dev)
    ctp.stream_probe(ctp.STREAM_READ, src, sink)
    ctp.stream_probe(ctp.STREAM_WRITE, None, dst)
    torch.cuda.synchronize()
    assert float(sink.abs().sum()) == 0.0
    assert torch.equal(dst[:8].cpu(), torch.tensor([1.0, 2.0, 3.0, 4.0] * 2))
    assert bool((dst.view(-1, 4) == torch.tensor([1.0, 2.0, 3.0, 4.0], device=dev)).all())
    # the 4-byte-access variants
    dst.zero_()
    ctp.stream_probe(ctp.STREAM_COPY + ctp.STREAM_DWORD, src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    ctp.stream_probe(ctp.STREAM_READ + ctp.STREAM_DWORD, src, sink)
    ctp.stream_probe(ctp.STREAM_WRITE + ctp.STREAM_DWORD, None, dst)
    torch.cuda.synchronize()
    assert float(sink.abs().sum()) == 0.0
    assert bool((dst == 1.0).all())


# ------------------------------------------------------------ VJP of the VJP (Y given)


def run_double_small(ctp, dev, d, L):
    n = d["n_nodes"]
    prob = oc.Problem(L, L, L)
    Y = sh32(L, d["vec"])
    ax, aw, aY = gen.cotangents_small(d, seed=n)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    res = ctp.conv_tp_bwd_bwd(T(d["grad_out"], dev), T(d["x"], dev), T(Y, dev), T(d["w"], dev),
                              T(ax, dev), T(aw, dev), T(aY, dev), g, L)
    ref = oc.materialised_double_bwd(prob, d["x"], Y, d["w"], d["grad_out"], ax, aw, aY,
                                     d["row_ptr"], d["senders"])
    for name, got, want in zip(("g_x", "g_w", "g_y", "g_grad"), res, ref):
        close(name, host(got), want)
    return res


def test_double_bwd_tiny(ctp, dev):
    run_double_small(ctp, dev, gen.tiny(), 1)


@pytest.mark.parametrize("n,c,L", [(90, 16, 1), (150, 48, 2), (120, 128, 2), (100, 128, 3), (70, 64, 3),
                                   (60, 192, 3), (40, 96, 0), (36, 512, 2)])
def test_double_bwd_small(ctp, dev, n, c, L):
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=n + c + L)
    a = run_double_small(ctp, dev, d, L)
    b = run_double_small(ctp, dev, d, L)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_double_bwd_full_l3_sampled(ctp, dev):
    """lmax=3, N=16384, C=128, Poisson(45): every output on seeded samples,
    the oracle composed from the C edge loop with swapped operands."""
    n, c, L = 16384, 128, 3
    d = gen.poisson_full(n, c, L, dev, seed=0)
    rp, s = d["row_ptr"], d["senders"]
    prob = oc.Problem(L, L, L)
    Y = sh32(L, d["vec"])
    ax, aw, aY = gen.cotangents_full(d, dev, seed=0)
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    gx, gw, gy, gG = ctp.conv_tp_bwd_bwd(d["grad_out"], d["x"], T(Y, dev), d["w"], ax, aw, T(aY, dev), g, L)
    Yr, aYr = Y.astype(np.float64), aY.astype(np.float64)
    x_h, ax_h, G_h = host(d["x"]), host(ax), host(d["grad_out"])
    rng = np.random.default_rng(123)
    rows = np.sort(rng.choice(n, 24, replace=False))
    ri = torch.as_tensor(rows, device=dev)
    ref_G = (_sub_fwd(prob, rp, s, Yr, d["w"], ax_h, rows) + _sub_fwd(prob, rp, s, Yr, aw, x_h, rows)
             + _sub_fwd(prob, rp, s, aYr, d["w"], x_h, rows))
    close("g_grad[sample]", host(gG[ri]), ref_G)
    ref_x = _sub_dx(prob, rp, s, Yr, aw, G_h, rows) + _sub_dx(prob, rp, s, aYr, d["w"], G_h, rows)
    close("g_x[sample]", host(gx[ri]), ref_x)
    edges = np.sort(rng.choice(len(s), 96, replace=False))
    dw1, dY1 = _sub_edges(prob, rp, s, Yr, d["w"], ax_h, G_h, edges)
    dw2, _ = _sub_edges(prob, rp, s, aYr, d["w"], x_h, G_h, edges)
    _, dY3 = _sub_edges(prob, rp, s, Yr, aw, x_h, G_h, edges)
    ei = torch.as_tensor(edges, device=dev)
    close("g_w[sample]", host(gw[ei]), dw1 + dw2)
    close("g_y[sample]", host(gy[ei]), dY1 + dY3)


def test_double_bwd_edge_vectors_full_l3(ctp, dev):
    """lmax=3, N=16384, C=128, as `bench.py --workload l3ddvec` runs it: the
    one-call edge-vector VJP of the VJP (first backward's dY given) equals,
    bit for bit, its steps called one by one (harmonics, harmonic JVP, the
    Y-given double backward sampled against the oracle above, second-order
    term); g_vec is also checked on sampled edges against the oracle's
    harmonic terms applied to the library's g_y and dY."""
    n, c, L = 16384, 128, 3
    d = gen.poisson_full(n, c, L, dev, seed=0)
    rp, s = d["row_ptr"], d["senders"]
    ax, aw, _ = gen.cotangents_full(d, dev, seed=0)
    v = T(d["vec"], dev)
    av = torch.randn(v.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev)
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    G, x, w = d["grad_out"], d["x"], d["w"]
    print("double bwd edge vectors full l3", flush=True)
    Y = ctp.spherical_harmonics(v, L)
    dY = ctp.conv_tp_bwd(G, x, Y, w, g, L, ctp.Y_GIVEN)[2]
    res = ctp.conv_tp_bwd_bwd_vec(G, x, v, w, ax, aw, av, g, L, dY=dY)
    aY = ctp.spherical_harmonics_jvp(v, av, L)
    gx, gw, gy, gG = ctp.conv_tp_bwd_bwd(G, x, Y, w, ax, aw, aY, g, L)
    gv = ctp.spherical_harmonics_bwd_bwd(v, dY, av, gy, L)
    for name, a, b in zip(("g_x", "g_w", "g_vec", "g_grad"), res, (gx, gw, gv, gG)):
        assert torch.equal(a, b), name
    rng = np.random.default_rng(8)
    edges = np.sort(rng.choice(len(s), 256, replace=False))
    ei = torch.as_tensor(edges, device=dev)
    v64 = d["vec"][edges].astype(np.float64)
    ref = (osh.vec_grad_from_sh_grad(L, v64, host(gy[ei]).astype(np.float64))
           + osh.vec_hess_term(L, v64, host(dY[ei]).astype(np.float64), host(av[ei]).astype(np.float64)))
    close("g_vec[sample]", host(res[2][ei]), ref)


# ------------------------------------------------------------ MACE variant (natural parity, slots)


def _variant_inputs(d, L):
    """Resize w and grad_out of a summed-variant workload to the slot variant
    (the generators draw the summed shapes; the extra values are simply not used)."""
    pr = oc.Problem(L, L, L, variant=1)
    rng = np.random.default_rng(d["n_nodes"] + 17)
    d = dict(d)
    d["w"] = rng.standard_normal((d["n_edges"], pr.P, d["x"].shape[2]), dtype=np.float32)
    d["grad_out"] = rng.standard_normal((d["n_nodes"], pr.D3, d["x"].shape[2]), dtype=np.float32)
    return d


@pytest.mark.parametrize("n,c,L", [(90, 16, 1), (150, 48, 2), (100, 128, 3), (70, 64, 3), (60, 192, 3),
                                   (40, 96, 0), (30, 512, 2)])
@pytest.mark.parametrize("y_mode", [0, 1])
def test_variant_slots_small(ctp, dev, n, c, L, y_mode):
    d = _variant_inputs(gen.poisson_small(n, c, L, mean_deg=12.0, seed=n + c + L), L)
    run_small(ctp, dev, d, L, y_mode, 0, bwd=True, variant=1)
    run_small(ctp, dev, d, L, y_mode, 1, bwd=False, variant=1)


def test_variant_slots_full_l3_sampled(ctp, dev):
    """lmax=3, N=16384, C=128, Poisson(45), Y given, natural-parity paths with slots."""
    n, c, L = 16384, 128, 3
    d = gen.poisson_full(n, c, L, dev, seed=0, need_grad=False)
    pr = oc.Problem(L, L, L, variant=1)
    rp, s = d["row_ptr"], d["senders"]
    e = len(s)
    w = gen.normal_tensor((e, pr.P, c), 0, 21, dev)
    G = gen.normal_tensor((n, pr.D3, c), 0, 23, dev)
    Y = sh32(L, d["vec"])
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    out = ctp.conv_tp_fwd(d["x"], T(Y, dev), w, g, L, 0, variant=1)
    dx, dw, dy = ctp.conv_tp_bwd(G, d["x"], T(Y, dev), w, g, L, 0, variant=1)
    Yr = Y.astype(np.float64)
    x_h, G_h = host(d["x"]), host(G)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(n, 32, replace=False))
    ri = torch.as_tensor(rows, device=dev)
    close("out[sample]", host(out[ri]), _sub_fwd(pr, rp, s, Yr, w, x_h, rows))
    close("dx[sample]", host(dx[ri]), _sub_dx(pr, rp, s, Yr, w, G_h, rows))
    edges = np.sort(rng.choice(e, 128, replace=False))
    dw_ref, dY_ref = _sub_edges(pr, rp, s, Yr, w, x_h, G_h, edges)
    ei = torch.as_tensor(edges, device=dev)
    close("dw[sample]", host(dw[ei]), dw_ref)
    close("dY[sample]", host(dy[ei]), dY_ref)


# ------------------------------------------------------------ harmonic gradient alone


@pytest.mark.parametrize("n,c,L", [(90, 16, 1), (150, 48, 2), (100, 128, 3), (60, 192, 3), (40, 96, 0),
                                   (30, 512, 2), (50, 7, 2)])
@pytest.mark.parametrize("variant", [0, 1])
def test_bwd_dy_small(ctp, dev, n, c, L, variant):
    """conv_tp_bwd_dy against the oracle's dY and bitwise against conv_tp_bwd's."""
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=n + c + L + 9)
    if variant == 1:
        d = _variant_inputs(d, L)
    prob = oc.Problem(L, L, L, variant=variant)
    Y = sh32(L, d["vec"])
    g = ctp.Graph(d["n_nodes"], T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev)
    print(f"bwd_dy n={n} c={c} L={L} variant={variant}", flush=True)
    dy = ctp.conv_tp_bwd_dy(G, x, w, g, L, variant=variant)
    _, dY_ref = oc.bwd_edges(prob, d["x"], Y.astype(np.float64), d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    close("dY", host(dy), dY_ref)
    _, _, dy0 = ctp.conv_tp_bwd(G, x, T(Y, dev), w, g, L, 0, variant=variant)
    assert torch.equal(dy, dy0)


def test_bwd_dy_full_l3_and_isolated_receivers(ctp, dev):
    """lmax=3, N=16384, C=128: bitwise equal to the full backward's dY; and a
    graph with receivers that have no in-edges."""
    n, c, L = 16384, 128, 3
    d = gen.poisson_full(n, c, L, dev, seed=4, need_grad=True)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    Y = T(sh32(L, d["vec"]), dev)
    print("bwd_dy full l3", flush=True)
    dy = ctp.conv_tp_bwd_dy(d["grad_out"], d["x"], d["w"], g, L)
    _, _, dy0 = ctp.conv_tp_bwd(d["grad_out"], d["x"], Y, d["w"], g, L, 0)
    assert torch.equal(dy, dy0)
    rng = np.random.default_rng(3)
    recv = np.sort(rng.integers(0, 10, size=200))        # receivers 10..39 have no in-edges
    dd = dict(n_nodes=40, n_edges=200, row_ptr=og.row_ptr_from_receivers(recv, 40),
              senders=rng.integers(0, 40, size=200).astype(np.int32),
              vec=rng.standard_normal((200, 3)).astype(np.float32),
              x=rng.standard_normal((40, 16, 64)).astype(np.float32),
              w=rng.standard_normal((200, 34, 64)).astype(np.float32),
              grad_out=rng.standard_normal((40, 16, 64)).astype(np.float32))
    g2 = ctp.Graph(40, T(dd["row_ptr"], dev), T(dd["senders"], dev))
    dy2 = ctp.conv_tp_bwd_dy(T(dd["grad_out"], dev), T(dd["x"], dev), T(dd["w"], dev), g2, L)
    _, ref = oc.bwd_edges(oc.Problem(L, L, L), dd["x"], sh32(L, dd["vec"]).astype(np.float64), dd["w"],
                          dd["grad_out"], dd["row_ptr"], dd["senders"])
    close("dY", host(dy2), ref)


# ------------------------------------------------------------ forward in each edge's frame (algo 2)


@pytest.mark.parametrize("n,c,L", SMALL)
def test_frame_forward_small(ctp, dev, n, c, L):
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=n + c + L + 5)
    run_small(ctp, dev, d, L, 1, ctp.ALGO_FRAME, bwd=False)


def test_frame_forward_poles_zero_vectors_and_hub(ctp, dev):
    """Edge vectors along +z and -z (exact and within 1e-7 of them), zero
    vectors, a 1000-in-degree hub, self and duplicate edges."""
    rng = np.random.default_rng(44)
    n, c, L = 40, 96, 3
    recv = np.sort(np.concatenate([np.full(1000, 3), rng.integers(0, n, size=300)]))
    s = rng.integers(0, n, size=recv.size)
    s[:10] = recv[:10]
    e = recv.size
    vec = rng.standard_normal((e, 3)).astype(np.float32)
    vec[::37] = 0.0
    vec[1::41] = (0.0, 0.0, 2.5)
    vec[2::41] = (0.0, 0.0, -0.5)
    vec[3::41] = (1e-7, -1e-7, -1.0)
    vec[4::41] = (-1e-7, 0.0, 1.0)
    vec[5::41] = (1.0, 0.0, 0.0)
    d = dict(n_nodes=n, n_edges=e, row_ptr=og.row_ptr_from_receivers(recv, n), senders=s.astype(np.int32), vec=vec,
             x=rng.standard_normal((n, 16, c)).astype(np.float32),
             w=rng.standard_normal((e, 34, c)).astype(np.float32))
    run_small(ctp, dev, d, L, 1, ctp.ALGO_FRAME, bwd=False)


def test_frame_forward_full_l3_sampled_and_deterministic(ctp, dev):
    """lmax=3, N=16384, C=128, Poisson(45), edge vectors: sampled receivers
    against the oracle, the whole output against the direct forward, and
    bitwise equal reruns."""
    n, c, L = 16384, 128, 3
    d = gen.poisson_full(n, c, L, dev, seed=2, need_grad=False)
    rp, s, vec = d["row_ptr"], d["senders"], d["vec"]
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    v = T(vec, dev)
    print("frame forward full l3", flush=True)
    out = ctp.conv_tp_fwd(d["x"], v, d["w"], g, L, 1, ctp.ALGO_FRAME)
    again = ctp.conv_tp_fwd(d["x"], v, d["w"], g, L, 1, ctp.ALGO_FRAME)
    assert torch.equal(out, again)
    direct = ctp.conv_tp_fwd(d["x"], v, d["w"], g, L, 1, ctp.ALGO_CSR)
    close("out vs direct forward", host(out), host(direct))
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(n, 32, replace=False))
    close("out[sample]", host(out[torch.as_tensor(rows, device=dev)]),
          _sub_fwd(oc.Problem(L, L, L), rp, s, osh.real_sh(L, vec.astype(np.float64)), d["w"], host(d["x"]), rows))


def test_frame_forward_water_box(ctp, dev):
    """The water box (1503 receivers: the small-grid split) with edge vectors."""
    wb = gen.water_box(seed=0, device="cpu")
    n, L = wb["n_nodes"], 3
    g = ctp.Graph(n, T(wb["row_ptr"], dev), T(wb["senders"], dev))
    w1 = wb["w1"].numpy()
    x, v, w = T(wb["x"], dev), T(wb["vec"], dev), T(w1, dev)
    print("frame forward water box", flush=True)
    out = ctp.conv_tp_fwd(x, v, w, g, L, 1, ctp.ALGO_FRAME)
    ref = oc.fwd(oc.Problem(L, L, L), wb["x"], osh.real_sh(L, wb["vec"].astype(np.float64)), w1,
                 wb["row_ptr"], wb["senders"])
    close("out", host(out), ref)


# ------------------------------------------------------------ backward through edge messages


def run_msg(ctp, dev, d, L, y_mode, variant, ws=None):
    """conv_tp_bwd_msg against the oracle (dx, dw, dY) and against conv_tp_bwd
    (dw and dY bitwise: the same per-edge arithmetic); conv_tp_bwd algo 1 (the
    receiver-major pass with atomics into dx) likewise."""
    n, e = d["n_nodes"], d["n_edges"]
    prob = oc.Problem(L, L, L, variant=variant)
    vec = d["vec"]
    Y = sh32(L, vec)
    yv = T(Y if y_mode == 0 else vec, dev)
    Yref = Y.astype(np.float64) if y_mode == 0 else osh.real_sh(L, vec.astype(np.float64))
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x, w, G = T(d["x"], dev), T(d["w"], dev), T(d["grad_out"], dev)
    print(f"bwd_msg n={n} e={e} c={x.shape[2]} L={L} y_mode={y_mode} variant={variant}", flush=True)
    dx, dw, dy = ctp.conv_tp_bwd_msg(G, x, yv, w, g, L, y_mode, variant=variant, workspace=ws)
    sp, pe, sr = og.transpose(n, d["row_ptr"], d["senders"])
    close("dx", host(dx), oc.bwd_dx(prob, Yref, d["w"], d["grad_out"], sp, pe, sr), nonzero=e > 0)
    dw_ref, dY_ref = oc.bwd_edges(prob, d["x"], Yref, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    close("dw", host(dw), dw_ref, nonzero=e > 0)
    if y_mode == 0:
        close("dY", host(dy), dY_ref, nonzero=e > 0)
    else:
        close("dvec", host(dy), osh.vec_grad_from_sh_grad(L, vec.astype(np.float64), dY_ref), nonzero=e > 0 and L > 0)
    dx0, dw0, dy0 = ctp.conv_tp_bwd(G, x, yv, w, g, L, y_mode, variant=variant)
    assert torch.equal(dw, dw0) and torch.equal(dy, dy0)
    # algo 1: the same receiver-major pass with dx added by atomics (dw, dY the same bits)
    dx1, dw1, dy1 = ctp.conv_tp_bwd(G, x, yv, w, g, L, y_mode, variant=variant, algo=ctp.ALGO_ATOMIC)
    close("dx (algo 1)", host(dx1), oc.bwd_dx(prob, Yref, d["w"], d["grad_out"], sp, pe, sr), nonzero=e > 0)
    assert torch.equal(dw1, dw) and torch.equal(dy1, dy)


@pytest.mark.parametrize("n,c,L", [(90, 16, 1), (150, 48, 2), (100, 128, 3), (60, 192, 3), (40, 96, 0),
                                   (30, 512, 2), (50, 7, 2), (45, 5, 0)])
@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("y_mode", [0, 1])
def test_bwd_msg_small(ctp, dev, n, c, L, variant, y_mode):
    d = gen.poisson_small(n, c, L, mean_deg=12.0, seed=n + c + L)
    if variant == 1:
        d = _variant_inputs(d, L)
    run_msg(ctp, dev, d, L, y_mode, variant)


def test_bwd_msg_edge_cases_and_reused_workspace(ctp, dev):
    """Hub receiver, isolated nodes, self and duplicate edges, zero vectors;
    the same workspace reused by a second, smaller call; an empty graph."""
    rng = np.random.default_rng(31)
    n, c, L = 40, 128, 3
    recv = np.concatenate([np.full(700, 3), rng.integers(0, n, size=300)])
    recv[recv == 17] = 18
    recv = np.sort(recv)
    s = rng.integers(0, n, size=recv.size)
    s[s == 21] = 22
    s[:10] = recv[:10]
    s[10:20] = s[20:30]
    e = recv.size
    vec = rng.standard_normal((e, 3)).astype(np.float32)
    vec[::37] = 0.0
    d = dict(n_nodes=n, n_edges=e, row_ptr=og.row_ptr_from_receivers(recv, n), senders=s.astype(np.int32), vec=vec,
             x=rng.standard_normal((n, 16, c)).astype(np.float32))
    d = _variant_inputs(d, L)
    ws = torch.full((e * 16 * c,), float("nan"), device=dev)
    for y_mode in (0, 1):
        run_msg(ctp, dev, d, L, y_mode, 1, ws=ws)
    small = _variant_inputs(gen.poisson_small(20, c, L, mean_deg=6.0, seed=3), L)
    run_msg(ctp, dev, small, L, 0, 1, ws=ws)
    g = ctp.Graph(5, T(np.zeros(6, dtype=np.int32), dev), T(np.zeros(0, dtype=np.int32), dev))
    x = torch.randn(5, 16, c, device=dev)
    dx, dw, dy = ctp.conv_tp_bwd_msg(torch.randn(5, 99, c, device=dev), x, torch.empty(0, 16, device=dev),
                                     torch.empty(0, 23, c, device=dev), g, L, 0, variant=1)
    assert not dx.any() and dw.numel() == 0 and dy.numel() == 0


def test_bwd_msg_full_l3_sampled(ctp, dev):
    """lmax=3, N=16384, C=128, Poisson(45), Y given, natural-parity paths with
    slots, as the timed variant-1 backward runs it."""
    n, c, L = 16384, 128, 3
    d = gen.poisson_full(n, c, L, dev, seed=0, need_grad=False)
    pr = oc.Problem(L, L, L, variant=1)
    rp, s = d["row_ptr"], d["senders"]
    e = len(s)
    w = gen.normal_tensor((e, pr.P, c), 0, 21, dev)
    G = gen.normal_tensor((n, pr.D3, c), 0, 23, dev)
    Y = sh32(L, d["vec"])
    g = ctp.Graph(n, T(rp, dev), T(s, dev))
    print("bwd_msg full l3 variant 1", flush=True)
    dx, dw, dy = ctp.conv_tp_bwd_msg(G, d["x"], T(Y, dev), w, g, L, 0, variant=1)
    Yr = Y.astype(np.float64)
    x_h, G_h = host(d["x"]), host(G)
    rng = np.random.default_rng(6)
    rows = np.sort(rng.choice(n, 32, replace=False))
    close("dx[sample]", host(dx[torch.as_tensor(rows, device=dev)]), _sub_dx(pr, rp, s, Yr, w, G_h, rows))
    edges = np.sort(rng.choice(e, 128, replace=False))
    dw_ref, dY_ref = _sub_edges(pr, rp, s, Yr, w, x_h, G_h, edges)
    ei = torch.as_tensor(edges, device=dev)
    close("dw[sample]", host(dw[ei]), dw_ref)
    close("dY[sample]", host(dy[ei]), dY_ref)
    dx0, dw0, dy0 = ctp.conv_tp_bwd(G, d["x"], T(Y, dev), w, g, L, 0, variant=1)
    assert torch.equal(dw, dw0) and torch.equal(dy, dy0)
    close("dx vs conv_tp_bwd", host(dx), host(dx0))
    # algo 1 (receiver-major, dx by atomics), as `bench.py --workload l3mace --bwd atomic` times it
    dx1, dw1, dy1 = ctp.conv_tp_bwd(G, d["x"], T(Y, dev), w, g, L, 0, variant=1, algo=ctp.ALGO_ATOMIC)
    assert torch.equal(dw1, dw) and torch.equal(dy1, dy)
    close("dx (algo 1)[sample]", host(dx1[torch.as_tensor(rows, device=dev)]), _sub_dx(pr, rp, s, Yr, w, G_h, rows))
    close("dx (algo 1) vs conv_tp_bwd_msg", host(dx1), host(dx))


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("y_mode", [0, 1])
def test_autograd_wrapper(ctp, dev, variant, y_mode):
    """conv_tp (torch.autograd) gives the library's forward and the oracle's
    gradients of <G, out> in x, w and Y (or vec)."""
    L = 2
    d = gen.poisson_small(80, 64, L, mean_deg=10.0, seed=41)
    if variant == 1:
        d = _variant_inputs(d, L)
    n = d["n_nodes"]
    prob = oc.Problem(L, L, L, variant=variant)
    vec = d["vec"]
    Y = sh32(L, vec)
    Yref = Y.astype(np.float64) if y_mode == 0 else osh.real_sh(L, vec.astype(np.float64))
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    x = T(d["x"], dev).requires_grad_(True)
    w = T(d["w"], dev).requires_grad_(True)
    yv = T(Y if y_mode == 0 else vec, dev).requires_grad_(True)
    print(f"autograd variant={variant} y_mode={y_mode}", flush=True)
    out = ctp.conv_tp(x, yv, w, g, L, y_mode, variant=variant)
    (out * T(d["grad_out"], dev)).sum().backward()
    close("out", host(out), oc.fwd(prob, d["x"], Yref, d["w"], d["row_ptr"], d["senders"]))
    sp, pe, sr = og.transpose(n, d["row_ptr"], d["senders"])
    close("x.grad", host(x.grad), oc.bwd_dx(prob, Yref, d["w"], d["grad_out"], sp, pe, sr))
    dw_ref, dY_ref = oc.bwd_edges(prob, d["x"], Yref, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    close("w.grad", host(w.grad), dw_ref)
    if y_mode == 0:
        close("Y.grad", host(yv.grad), dY_ref)
    else:
        close("vec.grad", host(yv.grad), osh.vec_grad_from_sh_grad(L, vec.astype(np.float64), dY_ref))


# ------------------------------------------------------------ edge-vector VJP of the VJP


@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_harmonic_second_order_terms(ctp, dev, L):
    rng = np.random.default_rng(60 + L)
    e = 5000
    vec = rng.standard_normal((e, 3)).astype(np.float32) * rng.uniform(0.3, 3.0, (e, 1)).astype(np.float32)
    vec[0] = 0.0                      # zero vector: zeros by convention
    vec[1] = [0.0, 0.0, 2.0]          # poles
    vec[2] = [0.0, 0.0, -0.5]
    av = rng.standard_normal((e, 3)).astype(np.float32)
    dY = rng.standard_normal((e, (L + 1) ** 2)).astype(np.float32)
    gY = rng.standard_normal((e, (L + 1) ** 2)).astype(np.float32)
    v64 = vec.astype(np.float64)
    aY = ctp.spherical_harmonics_jvp(T(vec, dev), T(av, dev), L)
    gv = ctp.spherical_harmonics_bwd_bwd(T(vec, dev), T(dY, dev), T(av, dev), T(gY, dev), L)
    ref_aY = osh.real_sh_jvp(L, v64, av)
    ref_gv = osh.vec_grad_from_sh_grad(L, v64, gY) + osh.vec_hess_term(L, v64, dY, av)
    close("aY", host(aY), ref_aY, nonzero=L > 0)
    close("gvec", host(gv), ref_gv, nonzero=L > 0)
    assert np.all(host(aY)[0] == 0.0) and np.all(host(gv)[0] == 0.0)


@pytest.mark.parametrize("n,c,L", [(60, 16, 1), (80, 64, 2), (70, 128, 3)])
def test_double_bwd_edge_vectors(ctp, dev, n, c, L):
    d = gen.poisson_small(n, c, L, mean_deg=10.0, seed=n + L)
    prob = oc.Problem(L, L, L)
    ax, aw, _ = gen.cotangents_small(d, seed=n)
    av = np.random.default_rng(n + 1).standard_normal((d["n_edges"], 3)).astype(np.float32)
    g = ctp.Graph(n, T(d["row_ptr"], dev), T(d["senders"], dev))
    gx, gw, gvec, gG = ctp.conv_tp_bwd_bwd_vec(T(d["grad_out"], dev), T(d["x"], dev), T(d["vec"], dev),
                                               T(d["w"], dev), T(ax, dev), T(aw, dev), T(av, dev), g, L)
    v64 = d["vec"].astype(np.float64)
    Y = osh.real_sh(L, v64)
    aY = osh.real_sh_jvp(L, v64, av)
    rx, rw, rY, rG = oc.materialised_double_bwd(prob, d["x"], Y, d["w"], d["grad_out"], ax, aw, aY,
                                                d["row_ptr"], d["senders"])
    _, _, dY = oc.materialised_bwd(prob, d["x"], Y, d["w"], d["grad_out"], d["row_ptr"], d["senders"])
    rvec = osh.vec_grad_from_sh_grad(L, v64, rY) + osh.vec_hess_term(L, v64, dY, av)
    for name, got, ref in (("g_x", gx, rx), ("g_w", gw, rw), ("g_vec", gvec, rvec), ("g_grad", gG, rG)):
        close(name, host(got), ref)
    # with the first backward's dY passed in (Y given): the same bits
    vt = T(d["vec"], dev)
    _, _, dYt = ctp.conv_tp_bwd(T(d["grad_out"], dev), T(d["x"], dev), ctp.spherical_harmonics(vt, L),
                                T(d["w"], dev), g, L, ctp.Y_GIVEN)
    again = ctp.conv_tp_bwd_bwd_vec(T(d["grad_out"], dev), T(d["x"], dev), vt, T(d["w"], dev), T(ax, dev),
                                    T(aw, dev), T(av, dev), g, L, dY=dYt)
    for u, v in zip((gx, gw, gvec, gG), again):
        assert torch.equal(u, v)

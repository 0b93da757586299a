#!/usr/bin/env python3
"""Benchmark of the fused conv tensor product on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM.  Default workload (`l3fb`): lmax = 3, N = 16384
nodes, C = 128 channels (N*C = 2^21), Poisson(45) in-degrees, Y given,
forward (CSR, deterministic) + backward (dx, dw, dY).  Other workloads:
`l2fwd` (lmax 2, N = 32768, forward), `sweepC` (lmax 2, N = 2^22/C, forward,
CSR and atomic timed, C in 64..1024), `water` (1503 atoms, 83,325 edges,
two lmax-3 layers forward + backward to edge vectors, in each edge's frame;
`--direct` for the direct kernels), `tiny`, and the diagnostics listed
under --workload.

Throughput is algorithmic bytes / time (the byte model counts every array
the method must touch once: w, Y or vec, index arrays, x and G once, outputs
once) and edges / time.  Kernel times come from HIP events recorded on the
stream the kernels run on.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv TP fwd/bwd effective GB/s (% of MI355X HBM peak); edges/s"
HBM_PEAK_GBS = 8000.0
# fp32 VALU peak without packed math (the kernels are built with packed fp32
# switched off): 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz
VALU_PEAK_TFLOPS = 78.6432


def fwd_bytes(N, E, C, D1, D2, D3, P, S):
    return 4 * (E * P * C + E * S + E + (N + 1) + N * C * D1 + N * C * D3)


def bwd_bytes(N, E, C, D1, D2, D3, P, S):
    return 4 * (2 * E * P * C + 2 * E * S + 2 * E + (N + 1) + 2 * N * C * D1 + N * C * D3)


# every source a workload's kernels are compiled or dispatched from
COMMON_SOURCES = ("device_common.hpp", "tables.hpp", "kernels.hpp", "convtp_api.hip")
CONV_SOURCES = ("convtp_triple.hip", "convtp_common.hip", "conv_fwd.hpp", "conv_bwd.hpp", "conv_dy.hpp",
                "conv_dd.hpp", "conv_frame.hpp")
WORKLOAD_SOURCES = {"node3": ("nodetp_kernels.hip",), "hbm": ("stream_probe.hip",)}


def kernel_sources_sha(workload="l3fb"):
    """Hash of every source the workload's kernels are compiled or dispatched from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_product_message_amd", "csrc")
    for f in WORKLOAD_SOURCES.get(workload.split("-")[0], CONV_SOURCES) + COMMON_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def run_tag(args):
    """Name of what a run measures: the workload plus the options that change
    which kernels run (edge vectors, edge-frame forward, sender-major MACE
    backward).  Traffic records are stored and looked up under it."""
    tag = args.workload
    if getattr(args, "vec", False):
        tag += "-vec"
    if getattr(args, "frame", False) and args.workload != "water":
        tag += "-frame"
    if args.workload == "water" and getattr(args, "direct", False):
        tag += "-direct"
    if args.workload == "l3mace" and getattr(args, "bwd", "msg") != "msg":
        tag += "-" + args.bwd
    return tag


class Timer:
    """Per-kernel HIP events on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        r = fn()
        ev1.record()
        self.pairs.setdefault(name, []).append((ev0, ev1))
        return r

    def mean_ms(self, name):
        p = self.pairs.get(name, [])
        return sum(a.elapsed_time(b) for a, b in p) / len(p) if p else float("nan")

    def reset(self):
        self.pairs = {}


# ------------------------------------------------------------ workloads


def make_poisson(ctp, torch, dev, n, c, L, y_mode, with_bwd, seed=0):
    from workloads import gen
    d = gen.poisson_full(n, c, L, dev, seed=seed, need_grad=with_bwd)
    g = ctp.Graph(n, torch.as_tensor(d["row_ptr"]).to(dev), torch.as_tensor(d["senders"]).to(dev))
    vec = torch.as_tensor(d["vec"]).to(dev)
    y = ctp.spherical_harmonics(vec, L) if y_mode == ctp.Y_GIVEN else vec
    if with_bwd:
        g.transpose  # built once per static graph, outside the timed region
    torch.cuda.synchronize()
    return d, g, y


def shape_of(d, ctp, L, y_mode, variant=0):
    N, E, C = d["n_nodes"], d["n_edges"], d["channels"]
    D = ctp.dim(L)
    paths, DO = ctp.layout(L, variant)
    S = D if y_mode == ctp.Y_GIVEN else 3
    return N, E, C, D, D, DO, len(paths), S


def fma_per_edge_channel(ctp, L, variant=0):
    """FMAs per (edge, channel) of the plain sparse schedule, from the coupling
    tables: forward = T entries + min(2l1+1, 2l3+1) per path; backward = T
    entries (v = T^T g) + 2 * sum(2l1+1) (dw, dx) + x(x)g products per (l1, l3)
    pair + coupling non-zeros (B) + sum(2l2+1) (dY)."""
    import numpy as np
    fwd = bwd = 0
    pairs = set()
    for k, (l1, l2, l3) in enumerate(ctp.layout(L, variant)[0]):
        c = ctp.coupling(l1, l2, l3)
        slots = int(np.count_nonzero(np.abs(c).sum(axis=1) > 0))
        nnz = int(np.count_nonzero(c))
        n1, n2, n3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
        fwd += slots + min(n1, n3)
        bwd += slots + 2 * n1 + nnz + n2
        # products x (x) g are shared by the paths reading the same G block
        pairs.add((l1, l3) if variant == 0 else (l1, l3, k))
    bwd += sum((2 * q[0] + 1) * (2 * q[1] + 1) for q in pairs)
    return fwd, bwd


def workload_l3fb(ctp, torch, dev, args):
    L, y_mode = 3, (ctp.VEC_GIVEN if args.vec else ctp.Y_GIVEN)
    d, g, y = make_poisson(ctp, torch, dev, 16384, 128, L, y_mode, True)
    x, w, G = d["x"], d["w"], d["grad_out"]
    out = torch.empty_like(x)
    dx, dw, dy = torch.empty_like(x), torch.empty_like(w), torch.empty_like(y)
    shp = shape_of(d, ctp, L, y_mode)

    if args.frame and not args.vec:
        raise SystemExit("--frame needs --vec (the edge-frame forward takes edge vectors)")
    fwd_algo = ctp.ALGO_FRAME if args.frame else ctp.ALGO_CSR

    def step(t):
        t.run("fwd", lambda: ctp.conv_tp_fwd(x, y, w, g, L, y_mode, fwd_algo, out=out))
        t.run("bwd", lambda: ctp.conv_tp_bwd(G, x, y, w, g, L, y_mode, dx=dx, dw=dw, dy=dy, algo=fwd_algo))

    kb = {"fwd": fwd_bytes(*shp), "bwd": bwd_bytes(*shp)}
    ffma, bfma = fma_per_edge_channel(ctp, L)
    # the direct kernels' FMAs (the edge-frame kernels do fewer: no VALU figure for them)
    kf = None if args.frame else {"fwd": 2.0 * ffma * shp[1] * 128, "bwd": 2.0 * bfma * shp[1] * 128}
    cfg = {"workload": f"lmax=3 conv TP forward+backward, N=16384, C=128, E={shp[1]}, "
                       f"Poisson(45) in-degree, {'vec' if args.vec else 'Y'} given, fp32",
           "n_nodes": shp[0], "n_edges": shp[1], "channels": 128, "lmax": 3,
           "y_mode": "vec" if args.vec else "Y", "paths": shp[6],
           "algo": "edge frame (algo 2), forward and backward" if args.frame else "direct (algo 0)"}
    # the direct backward issues VALU instructions at about 0.9 of the rate the
    # VALU probe sustains (SQ counters), the unit nearest its ceiling; its HBM
    # streams, a little further from theirs, are reported beside it
    return dict(step=step, kernel_bytes=kb, kernel_flops=kf, dominant="bwd", edges=shp[1], cfg=cfg,
                cpu=dict(kind="poisson", d=d, L=L, y_mode=y_mode, shp=shp, fb=True),
                bound=None if args.frame else "alu")


def workload_l3dd(ctp, torch, dev, args):
    """VJP of the VJP at lmax=3, N=16384, C=128, Poisson(45), Y given: the
    gradients of <ax, dx> + <aw, dw> + <aY, dY> in x, w, Y and G."""
    from workloads import gen
    L = 3
    d, g, y = make_poisson(ctp, torch, dev, 16384, 128, L, ctp.Y_GIVEN, True)
    ax, aw, aY = gen.cotangents_full(d, dev, seed=0)
    aY = torch.as_tensor(aY).to(dev)
    x, w, G = d["x"], d["w"], d["grad_out"]
    outs = (torch.empty_like(x), torch.empty_like(w), torch.empty_like(y), torch.empty_like(G))
    n, e, c = 16384, d["n_edges"], 128
    D, P = (L + 1) ** 2, ctp.num_paths(L)

    def step(t):
        t.run("dd", lambda: ctp.conv_tp_bwd_bwd(G, x, y, w, ax, aw, aY, g, L, out=outs))

    # each input read once and each output written once: x, ax, G, w, aw, Y, aY,
    # row_ptr, senders, send_ptr/perm/recv; gx, gG, gw, gY
    kb = {"dd": 4 * (3 * e * P * c + 3 * e * D + 4 * e + 2 * (n + 1) + 5 * n * D * c)}
    kf = {"dd": 2.0 * dd_fma_per_edge_channel(ctp, L) * e * c}
    cfg = {"workload": f"lmax=3 conv TP VJP-of-VJP, N=16384, C=128, E={e}, Poisson(45) in-degree, Y given, fp32",
           "n_nodes": n, "n_edges": e, "channels": c, "lmax": L, "paths": P}
    # k_dd_send (two thirds of the time) runs at about 80% of the VALU peak; k_dd_recv at the read ceiling
    return dict(step=step, kernel_bytes=kb, kernel_flops=kf, dominant="dd", edges=e, cfg=cfg, cpu=None, bound="alu")


def workload_l3ddvec(ctp, torch, dev, args):
    """VJP of the edge-vector backward at lmax=3, N=16384, C=128, Poisson(45):
    the gradients of <ax, dx> + <aw, dw> + <avec, dvec> in x, w, vec and G in
    one conv_tp_bwd_bwd_vec call (harmonics, harmonic JVP, the double backward,
    harmonic second-order term), given the first backward's harmonic gradient
    dY as force training keeps it (computed once, before the timed steps)."""
    from workloads import gen
    L = 3
    d, g, vec = make_poisson(ctp, torch, dev, 16384, 128, L, ctp.VEC_GIVEN, True)
    ax, aw, _ = gen.cotangents_full(d, dev, seed=0)
    avec = torch.randn(vec.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev)
    x, w, G = d["x"], d["w"], d["grad_out"]
    n, e, c = 16384, d["n_edges"], 128
    D, P = (L + 1) ** 2, ctp.num_paths(L)

    _, _, dY = ctp.conv_tp_bwd(G, x, ctp.spherical_harmonics(vec, L), w, g, L, ctp.Y_GIVEN)
    ws = torch.empty(4 * e * D, dtype=torch.float32, device=dev)
    outs = (torch.empty_like(x), torch.empty_like(w), torch.empty_like(vec), torch.empty_like(G))

    def step(t):
        t.run("ddvec", lambda: ctp.conv_tp_bwd_bwd_vec(G, x, vec, w, ax, aw, avec, g, L, dY=dY, out=outs,
                                                       workspace=ws))

    # inputs read once and outputs written once: x, ax, G, w, aw, vec, avec, dY and
    # the graph arrays; gx, gG, gw, gvec
    kb = {"ddvec": 4 * (3 * e * P * c + 4 * e * 3 + e * D + 4 * e + 2 * (n + 1) + 5 * n * D * c)}
    cfg = {"workload": f"lmax=3 conv TP VJP-of-VJP with edge vectors, N=16384, C=128, E={e}, Poisson(45) "
                       "in-degree, the first backward's dY given, fp32",
           "n_nodes": n, "n_edges": e, "channels": c, "lmax": L, "paths": P}
    return dict(step=step, kernel_bytes=kb, dominant="ddvec", edges=e, cfg=cfg, cpu=None)


def workload_l3mace(ctp, torch, dev, args):
    """MACE variant at lmax=3, N=16384, C=128, Poisson(45), Y given: natural-parity
    paths (P=23), one output slot per path (99 components per channel)."""
    from workloads import gen
    L, V = 3, ctp.SLOTS
    d, g, y = make_poisson(ctp, torch, dev, 16384, 128, L, ctp.Y_GIVEN, False)
    shp = shape_of(d, ctp, L, ctp.Y_GIVEN, V)
    n, e, c = shp[0], shp[1], shp[2]
    x = d["x"]
    w = gen.normal_tensor((e, shp[6], c), 0, 21, dev)
    G = gen.normal_tensor((n, shp[5], c), 0, 23, dev)
    g.transpose
    out, dx, dw, dy = torch.empty_like(G), torch.empty_like(x), torch.empty_like(w), torch.empty_like(y)
    if args.bwd == "msg":
        # backward through edge messages: the workspace is allocated once, outside the timed steps
        ws = torch.empty(ctp.conv_tp_bwd_msg_workspace(n, e, c, L, ctp.Y_GIVEN, V) // 4, dtype=torch.float32,
                         device=dev)
        bwd = lambda: ctp.conv_tp_bwd_msg(G, x, y, w, g, L, ctp.Y_GIVEN, dx=dx, dw=dw, dy=dy,  # noqa: E731
                                          variant=V, workspace=ws)
    elif args.bwd == "atomic":
        bwd = lambda: ctp.conv_tp_bwd(G, x, y, w, g, L, ctp.Y_GIVEN, dx=dx, dw=dw, dy=dy, variant=V,  # noqa: E731
                                      algo=ctp.ALGO_ATOMIC)
    else:
        bwd = lambda: ctp.conv_tp_bwd(G, x, y, w, g, L, ctp.Y_GIVEN, dx=dx, dw=dw, dy=dy, variant=V)  # noqa: E731

    def step(t):
        t.run("fwd", lambda: ctp.conv_tp_fwd(x, y, w, g, L, ctp.Y_GIVEN, out=out, variant=V))
        t.run("bwd", bwd)

    kb = {"fwd": fwd_bytes(*shp), "bwd": bwd_bytes(*shp)}
    ffma, bfma = fma_per_edge_channel(ctp, L, V)
    kf = {"fwd": 2.0 * ffma * e * c, "bwd": 2.0 * bfma * e * c}
    cfg = {"workload": f"MACE variant (natural-parity paths, per-path output slots), lmax=3, N=16384, C=128, "
                       f"E={e}, Poisson(45) in-degree, Y given, fp32",
           "n_nodes": n, "n_edges": e, "channels": c, "lmax": L, "paths": shp[6], "out_dim": shp[5],
           "backward": {"msg": "edge messages (conv_tp_bwd_msg)", "sender": "sender-major (conv_tp_bwd)",
                        "atomic": "receiver-major, dx by atomics (conv_tp_bwd algo 1, not reproducible)"}[args.bwd]}
    return dict(step=step, kernel_bytes=kb, kernel_flops=kf, dominant="bwd", edges=e, cfg=cfg, cpu=None)


def workload_gather(ctp, torch, dev, args):
    """Cache-footprint diagnostic at the lmax=3 step's sizes: the forward on a
    graph whose senders are nodes 0..K-1 and the backward on one whose
    receivers are nodes 0..K-1 (K = --gather-nodes), so the per-edge row
    gathers (x, then G) come from K rows of 8 KB; w, dw and the other streams
    are those of the real workload."""
    from workloads import gen
    L, n, c, k = 3, 16384, 128, args.gather_nodes
    (rp_a, s_a), (rp_b, s_b) = gen.gather_limited_graphs(n, 45.0, k, gen.rng_for(0))
    e = len(s_a)
    ga = ctp.Graph(n, torch.as_tensor(rp_a).to(dev), torch.as_tensor(s_a).to(dev))
    gb = ctp.Graph(n, torch.as_tensor(rp_b).to(dev), torch.as_tensor(s_b).to(dev))
    gb.transpose
    x = gen.normal_tensor((n, 16, c), 0, 1, dev)
    w = gen.normal_tensor((e, ctp.num_paths(L), c), 0, 2, dev)
    G = gen.normal_tensor((n, 16, c), 0, 3, dev)
    vec = torch.as_tensor(gen.unit_vectors(e, gen.rng_for(1))).to(dev)
    y = ctp.spherical_harmonics(vec, L)
    out, dx, dw, dy = torch.empty_like(x), torch.empty_like(x), torch.empty_like(w), torch.empty_like(y)
    torch.cuda.synchronize()

    def step(t):
        t.run("fwd", lambda: ctp.conv_tp_fwd(x, y, w, ga, L, ctp.Y_GIVEN, out=out))
        t.run("bwd", lambda: ctp.conv_tp_bwd(G, x, y, w, gb, L, ctp.Y_GIVEN, dx=dx, dw=dw, dy=dy))

    d = dict(n_nodes=n, n_edges=e, channels=c)
    shp = shape_of(d, ctp, L, ctp.Y_GIVEN)
    kb = {"fwd": fwd_bytes(*shp), "bwd": bwd_bytes(*shp)}
    cfg = {"workload": f"gather-footprint diagnostic: lmax=3, N=16384, C=128, E={e}, node-row gathers "
                       f"limited to {k} nodes ({k * 16 * c * 4 / 2**20:.1f} MiB), Y given, fp32",
           "n_nodes": n, "n_edges": e, "channels": c, "lmax": L, "gather_nodes": k}
    return dict(step=step, kernel_bytes=kb, dominant="bwd", edges=e, cfg=cfg, cpu=None)


def workload_l2fwd(ctp, torch, dev, args):
    L, y_mode = 2, ctp.Y_GIVEN
    d, g, y = make_poisson(ctp, torch, dev, 32768, 128, L, y_mode, False)
    x, w = d["x"], d["w"]
    out = torch.empty_like(x)
    shp = shape_of(d, ctp, L, y_mode)

    def step(t):
        t.run("fwd", lambda: ctp.conv_tp_fwd(x, y, w, g, L, y_mode, out=out))

    cfg = {"workload": f"lmax=2 conv TP forward, N=32768, C=128, E={shp[1]}, Poisson(45), Y given, fp32",
           "n_nodes": shp[0], "n_edges": shp[1], "channels": 128, "lmax": 2, "paths": shp[6]}
    return dict(step=step, kernel_bytes={"fwd": fwd_bytes(*shp)}, dominant="fwd", edges=shp[1], cfg=cfg,
                cpu=dict(kind="poisson", d=d, L=L, y_mode=y_mode, shp=shp, fb=False))


def workload_sweep(ctp, torch, dev, args):
    L, y_mode, c = 2, ctp.Y_GIVEN, args.channels
    n = (1 << 22) // c
    d, g, y = make_poisson(ctp, torch, dev, n, c, L, y_mode, False)
    x, w = d["x"], d["w"]
    out, out2 = torch.empty_like(x), torch.empty_like(x)
    shp = shape_of(d, ctp, L, y_mode)

    def step(t):
        t.run("fwd", lambda: ctp.conv_tp_fwd(x, y, w, g, L, y_mode, ctp.ALGO_CSR, out=out))
        t.run("fwd_atomic", lambda: ctp.conv_tp_fwd(x, y, w, g, L, y_mode, ctp.ALGO_ATOMIC, out=out2))

    fb = fwd_bytes(*shp)
    cfg = {"workload": f"channel sweep lmax=2 forward, C={c}, N={n}, E={shp[1]}, Poisson(45), "
                       "CSR and atomic both timed, fp32",
           "n_nodes": n, "n_edges": shp[1], "channels": c, "lmax": 2, "paths": shp[6]}
    return dict(step=step, kernel_bytes={"fwd": fb, "fwd_atomic": fb}, dominant="fwd", edges=shp[1], cfg=cfg,
                cpu=None, value_kernels=("fwd",))


def workload_water(ctp, torch, dev, args):
    from workloads import gen
    L, y_mode = 3, ctp.VEC_GIVEN
    wb = gen.water_box(seed=0, device=dev)
    n = wb["n_nodes"]
    g = ctp.Graph(n, torch.as_tensor(wb["row_ptr"]).to(dev), torch.as_tensor(wb["senders"]).to(dev))
    g.transpose
    v = torch.as_tensor(wb["vec"]).to(dev)
    x0 = torch.as_tensor(wb["x"]).to(dev)
    G = torch.as_tensor(wb["grad_out"]).to(dev)
    w1, w2 = wb["w1"], wb["w2"]
    h1, h2 = torch.empty_like(x0), torch.empty_like(x0)
    dh1, dx0 = torch.empty_like(x0), torch.empty_like(x0)
    dw1, dw2 = torch.empty_like(w1), torch.empty_like(w2)
    dv1, dv2 = torch.empty_like(v), torch.empty_like(v)
    torch.cuda.synchronize()

    # edge vectors: the edge-frame kernels by default (the same result up to
    # rounding, fewer FMAs); --direct times the direct kernels
    fwd_algo = ctp.ALGO_CSR if args.direct else ctp.ALGO_FRAME

    def step(t):
        t.run("fwd1", lambda: ctp.conv_tp_fwd(x0, v, w1, g, L, y_mode, fwd_algo, out=h1))
        t.run("fwd2", lambda: ctp.conv_tp_fwd(h1, v, w2, g, L, y_mode, fwd_algo, out=h2))
        t.run("bwd2", lambda: ctp.conv_tp_bwd(G, h1, v, w2, g, L, y_mode, dx=dh1, dw=dw2, dy=dv2, algo=fwd_algo))
        t.run("bwd1", lambda: ctp.conv_tp_bwd(dh1, x0, v, w1, g, L, y_mode, dx=dx0, dw=dw1, dy=dv1, algo=fwd_algo))

    E = wb["n_edges"]
    shp = (n, E, 128, 16, 16, 16, ctp.num_paths(L), 3)
    kb = {"fwd1": fwd_bytes(*shp), "fwd2": fwd_bytes(*shp), "bwd1": bwd_bytes(*shp), "bwd2": bwd_bytes(*shp)}
    cfg = {"workload": f"water-box-shaped step: 1503 atoms, {E} edges (10% zero-weight padding), "
                       "C=128, lmax=3, vec given, two layers forward + backward to edge vectors, fp32",
           "n_nodes": n, "n_edges": E, "channels": 128, "lmax": 3, "layers": 2,
           "algo": "direct (algo 0)" if args.direct else "edge frame (algo 2), forward and backward"}
    return dict(step=step, kernel_bytes=kb, dominant="bwd1", edges=E, cfg=cfg, cpu=None)


def workload_tiny(ctp, torch, dev, args):
    from workloads import gen
    d = gen.tiny()
    L, y_mode = 1, ctp.VEC_GIVEN
    g = ctp.Graph(64, torch.as_tensor(d["row_ptr"]).to(dev), torch.as_tensor(d["senders"]).to(dev))
    g.transpose
    x, w, G, v = (torch.as_tensor(d[k]).to(dev) for k in ("x", "w", "grad_out", "vec"))
    shp = (64, d["n_edges"], 16, 4, 4, 4, 5, 3)

    def step(t):
        t.run("fwd", lambda: ctp.conv_tp_fwd(x, v, w, g, L, y_mode))
        t.run("bwd", lambda: ctp.conv_tp_bwd(G, x, v, w, g, L, y_mode))

    cfg = {"workload": "tiny: 64 nodes, 16 channels, lmax=1, 16 distinct senders, vec given, fp32"}
    return dict(step=step, kernel_bytes={"fwd": fwd_bytes(*shp), "bwd": bwd_bytes(*shp)}, dominant="bwd",
                edges=d["n_edges"], cfg=cfg, cpu=None)


def workload_copy(ctp, torch, dev, args):
    """Calibration only: a plain 1 GiB device-to-device copy (reads 1 GiB,
    writes 1 GiB), used to scale the HBM byte counters of the profiler."""
    n = (1 << 30) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)

    def step(t):
        t.run("copy", lambda: dst.copy_(src))

    return dict(step=step, kernel_bytes={"copy": 2 * 4 * n}, dominant="copy", edges=0,
                cfg={"workload": "calibration: 1 GiB fp32 device copy"}, cpu=None)


def node_fma_per_node_channel(ctp, L):
    """FMAs per (node, channel) of the node-local product: forward = x*y
    products per (l1, l2) pair + coupling non-zeros + sum(2l3+1) (w scaling);
    backward = that for dw (plus sum(2l3+1) for the dot with g), and the same
    count for dx (y*g products per (l2, l3)) and dy (x*g per (l1, l3))."""
    import numpy as np
    ps = ctp.paths(L)
    nnz = sum(int(np.count_nonzero(ctp.coupling(*p))) for p in ps)
    def prod(i, j):
        return sum((2 * a + 1) * (2 * b + 1) for a, b in {(p[i], p[j]) for p in ps})
    s1 = sum(2 * p[0] + 1 for p in ps)
    s2 = sum(2 * p[1] + 1 for p in ps)
    s3 = sum(2 * p[2] + 1 for p in ps)
    fwd = prod(0, 1) + nnz + s3
    bwd = (prod(0, 1) + nnz + s3) + (prod(1, 2) + nnz + s1) + (prod(0, 2) + nnz + s2)
    return fwd, bwd


def dd_fma_per_edge_channel(ctp, L):
    """FMAs per (edge, channel) of the VJP of the VJP: receiver kernel
    3 sum(2l1+1) + 2 T entries; sender kernel 2 T entries + 4 sum(2l1+1) +
    2 (x*g products per (l1, l3) + coupling non-zeros + sum(2l2+1))."""
    import numpy as np
    ps = ctp.paths(L)
    slots = sum(int(np.count_nonzero(np.abs(ctp.coupling(*p)).sum(axis=1) > 0)) for p in ps)
    nnz = sum(int(np.count_nonzero(ctp.coupling(*p))) for p in ps)
    s1 = sum(2 * p[0] + 1 for p in ps)
    s2 = sum(2 * p[1] + 1 for p in ps)
    pairs = sum((2 * a + 1) * (2 * b + 1) for a, b in {(p[0], p[2]) for p in ps})
    return 3 * s1 + 2 * slots + 2 * slots + 4 * s1 + 2 * (pairs + nnz + s2)


def workload_node(ctp, torch, dev, args):
    """Node-local channelwise tensor product, lmax=3, C=128, N=131072 (no graph):
    forward + backward; every (node, channel) streams its rows once."""
    from workloads import gen
    s = gen.NODE
    L, n, c = s["lmax"], s["n_nodes"], s["channels"]
    d = gen.node_full(n, c, L, dev, seed=0)
    x, y, w, G = d["x"], d["y"], d["w"], d["grad_out"]
    out, dx, dy, dw = torch.empty_like(x), torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)
    D, P = (L + 1) ** 2, ctp.num_paths(L)

    def step(t):
        t.run("fwd", lambda: ctp.node_tp_fwd(x, y, w, L, out=out))
        t.run("bwd", lambda: ctp.node_tp_bwd(G, x, y, w, L, dx=dx, dy=dy, dw=dw))

    kb = {"fwd": 4 * n * c * (3 * D + P), "bwd": 4 * n * c * (5 * D + 2 * P)}
    ff, bf = node_fma_per_node_channel(ctp, L)
    kf = {"fwd": 2.0 * ff * n * c, "bwd": 2.0 * bf * n * c}
    cfg = {"workload": f"node-local channelwise tensor product, lmax=3, N={n}, C={c}, forward+backward, fp32",
           "n_nodes": n, "channels": c, "lmax": L, "paths": P}
    return dict(step=step, kernel_bytes=kb, kernel_flops=kf, dominant="bwd", edges=0, cfg=cfg, cpu=None)


def workload_hbm(ctp, torch, dev, args):
    """Practical HBM ceilings: the library's stream probes (non-temporal read,
    write and copy of 2 GiB, grid-stride), with 16-byte accesses per lane and
    with 4-byte ones (`*_b32`: the width of the kernels' row accesses)."""
    n = (1 << 31) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    D = ctp.STREAM_DWORD

    def step(t):
        t.run("read", lambda: ctp.stream_probe(ctp.STREAM_READ, src, dst))
        t.run("write", lambda: ctp.stream_probe(ctp.STREAM_WRITE, None, dst))
        t.run("copy", lambda: ctp.stream_probe(ctp.STREAM_COPY, src, dst))
        t.run("read_b32", lambda: ctp.stream_probe(ctp.STREAM_READ + D, src, dst))
        t.run("write_b32", lambda: ctp.stream_probe(ctp.STREAM_WRITE + D, None, dst))
        t.run("copy_b32", lambda: ctp.stream_probe(ctp.STREAM_COPY + D, src, dst))

    kb = {"read": 4 * n, "write": 4 * n, "copy": 8 * n, "read_b32": 4 * n, "write_b32": 4 * n, "copy_b32": 8 * n}
    return dict(step=step, kernel_bytes=kb, dominant="copy", edges=0,
                cfg={"workload": "HBM stream probes: 2 GiB fp32 read, write and copy, 16- and 4-byte accesses"},
                cpu=None)


def measured_valu_ceiling(ctp, torch, dev, iters=20000, reps=5):
    """fp32 FMA rate (TFLOP/s) the library's VALU probe sustains on this
    device right after the timed steps: HIP events around single launches on
    the current stream, best of reps."""
    sink = torch.zeros(4, device=dev)
    fmas = ctp.valu_probe(iters, sink)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ctp.valu_probe(iters, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2.0 * fmas / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def workload_valu(ctp, torch, dev, args):
    """Arithmetic ceiling: the library's fp32 FMA probe (non-packed, eight
    chains per lane, eight waves per SIMD on every CU)."""
    sink = torch.zeros(4, device=dev)
    iters = 20000
    fmas = ctp.valu_probe(iters, sink)   # one launch; the library reports the FMAs it performs

    def step(t):
        t.run("valu", lambda: ctp.valu_probe(iters, sink))

    return dict(step=step, kernel_bytes={}, kernel_flops={"valu": 2.0 * fmas}, dominant="valu", edges=0,
                cfg={"workload": "VALU probe: non-packed fp32 FMA, 8 chains per lane, 2048 x 256 threads"},
                cpu=None, flops_metric=True)


WORKLOADS = {"l3fb": workload_l3fb, "l2fwd": workload_l2fwd, "sweepC": workload_sweep,
             "water": workload_water, "tiny": workload_tiny, "copy": workload_copy, "hbm": workload_hbm,
             "node3": workload_node, "l3dd": workload_l3dd, "l3mace": workload_l3mace,
             "gather": workload_gather, "l3ddvec": workload_l3ddvec, "valu": workload_valu}


# ------------------------------------------------------------ CPU baseline (oracle)


def cpu_baseline(spec, sample_nodes):
    """Time the fp64 oracle (C edge loop, OpenMP) on a bounded sample of the
    same workload and scale to the benchmark's units."""
    import numpy as np
    from oracle import convtp as oc
    from oracle import graph as og
    from oracle import sh as osh

    d, L, shp, fb = spec["d"], spec["L"], spec["shp"], spec["fb"]
    N, E = shp[0], shp[1]
    rp, s = d["row_ptr"], d["senders"]
    rows = np.arange(min(sample_nodes, N) if sample_nodes > 0 else N)
    e_lo, e_hi = 0, int(rp[rows[-1] + 1])
    Y = osh.real_sh(L, d["vec"][e_lo:e_hi].astype(np.float64))
    x = d["x"].cpu().numpy()
    w = d["w"][e_lo:e_hi].cpu().numpy()
    prob = oc.Problem(L, L, L)
    rp_sub = rp[:rows[-1] + 2]
    s_sub = s[e_lo:e_hi]
    nt = oc.max_threads()
    t0 = time.perf_counter()
    oc.fwd(prob, x, Y, w, rp_sub, s_sub, rows=rows)
    t_fwd = time.perf_counter() - t0
    t_bwd = 0.0
    if fb:
        G = d["grad_out"].cpu().numpy()
        # the sampled edges grouped by sender (stable), as the backward walks them
        recv = og.receivers_of(rp_sub)
        order = np.argsort(s_sub, kind="stable")
        send_ptr = np.zeros(N + 1, dtype=np.int64)
        send_ptr[1:] = np.cumsum(np.bincount(s_sub, minlength=N))
        senders_hit = np.unique(s_sub)
        t0 = time.perf_counter()
        oc.bwd_dx(prob, Y, w, G, send_ptr.astype(np.int32), order.astype(np.int32),
                  recv[order].astype(np.int32), rows=senders_hit)
        oc.bwd_edges(prob, x, Y, w, G, rp_sub, s_sub)
        t_bwd = time.perf_counter() - t0
    e_sample = e_hi - e_lo
    t = t_fwd + t_bwd
    step_bytes = fwd_bytes(*shp) + (bwd_bytes(*shp) if fb else 0)
    edges_per_s = e_sample / t
    gbs = edges_per_s * (step_bytes / E) / 1e9
    what = "forward + backward (dx, dw, dY)" if fb else "forward"
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": nt, "kind": "oracle", "cpu_model": cpu_model,
            "edges_per_s": round(edges_per_s, 1), "seconds": round(t, 2),
            "forward_seconds": round(t_fwd, 2), "backward_seconds": round(t_bwd, 2),
            "sample": f"{what} over the {e_sample} in-edges of the first {len(rows)} receivers "
                      f"({e_sample / E:.1%} of the edges), fp64 C edge loop, {nt} OpenMP threads; "
                      "GB/s = edges/s x the step's algorithmic bytes per edge"}


# ------------------------------------------------------------ traffic from committed counters


def committed_traffic(tag, kernel):
    """HBM bytes per launch from profiles/traffic_<tag>_<kernel>.json, only if
    that record was taken for this run tag on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("tag", rec.get("workload")) != tag:
        return None
    if rec.get("source_sha") != kernel_sources_sha(tag):
        return None        # kernels changed since the counters were taken
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="l3fb", choices=sorted(WORKLOADS))
    ap.add_argument("--channels", type=int, default=128, help="sweepC only")
    ap.add_argument("--gather-nodes", type=int, default=64, help="gather only: nodes the row gathers touch")
    ap.add_argument("--vec", action="store_true", help="l3fb with edge vectors instead of Y")
    ap.add_argument("--frame", action="store_true",
                    help="l3fb --vec: forward and backward in each edge's frame (algo 2; the water box's default)")
    ap.add_argument("--direct", action="store_true",
                    help="water: the direct kernels (algo 0) instead of the edge frame")
    ap.add_argument("--bwd", choices=("msg", "sender", "atomic"), default="msg",
                    help="l3mace: backward through edge messages (conv_tp_bwd_msg), sender-major (conv_tp_bwd) "
                         "or receiver-major with dx by atomics (conv_tp_bwd algo 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-nodes", type=int, default=0,
                    help="receivers in the CPU-oracle sample (0: all of them)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the conv TP path here is "
              "single-device and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import tensor_product_message_amd as ctp
    dev = torch.device("cuda:0")
    print(f"[bench] workload {args.workload}: generating inputs", file=sys.stderr, flush=True)
    wl = WORKLOADS[args.workload](ctp, torch, dev, args)
    timer = Timer(torch)
    for _ in range(args.warmup):
        wl["step"](timer)
    torch.cuda.synchronize()
    timer.reset()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    s0.record()
    for _ in range(args.steps):
        wl["step"](timer)
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = s0.elapsed_time(s1) / args.steps

    if wl.get("flops_metric"):
        k = wl["dominant"]
        tf = wl["kernel_flops"][k] / (timer.mean_ms(k) * 1e-3) / 1e12
        print(json.dumps({"metric": "fp32 VALU FMA rate (measurement probe)", "value": round(tf, 2),
                          "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": wl["cfg"],
                          "roofline": {"bound": "alu", "kernel": k, "achieved": round(tf, 2),
                                       "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(tf / VALU_PEAK_TFLOPS, 4), "traffic": None},
                          "cpu_baseline": None}), flush=True)
        return
    value_kernels = wl.get("value_kernels", tuple(wl["kernel_bytes"]))
    step_bytes = sum(wl["kernel_bytes"][k] for k in value_kernels)
    if value_kernels != tuple(wl["kernel_bytes"]):
        ms_value = sum(timer.mean_ms(k) for k in value_kernels)
    else:
        ms_value = ms_step
    gbs = step_bytes / (ms_value * 1e-3) / 1e9
    dom = wl["dominant"]
    dom_ms = timer.mean_ms(dom)
    dom_gbs = wl["kernel_bytes"][dom] / (dom_ms * 1e-3) / 1e9
    kernels = {k: {"ms": round(timer.mean_ms(k), 4), "alg_bytes": wl["kernel_bytes"][k],
                   "GB_s": round(wl["kernel_bytes"][k] / (timer.mean_ms(k) * 1e-3) / 1e9, 1),
                   "pct_hbm_peak": round(100 * wl["kernel_bytes"][k] / (timer.mean_ms(k) * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 1)}
               for k in wl["kernel_bytes"]}
    tag = run_tag(args)
    traffic = committed_traffic(tag, dom)
    wl["cfg"].setdefault("seed", 0)     # graphs and features drawn with seed 0 (fixed seeds elsewhere)
    line = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_value, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": wl["cfg"],
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
        "edges_per_s": round(wl["edges"] / (ms_value * 1e-3), 1) if wl["edges"] else None,
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "wall_s": round(wall, 3), "run_tag": tag, "kernel_sources_sha": kernel_sources_sha(tag),
    }
    if wl.get("kernel_flops"):
        # the second bound: fp32 VALU arithmetic of the same kernel
        tf = wl["kernel_flops"][dom] / (dom_ms * 1e-3) / 1e12
        alu = {"achieved": round(tf, 2), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": round(tf / VALU_PEAK_TFLOPS, 4), "flops": wl["kernel_flops"][dom]}
        if wl.get("bound") == "alu":
            # arithmetic holds this kernel: the VALU figure is the roofline, HBM the second
            # bound; the probe's rate on this device is the practical VALU ceiling
            hbm = {k: line["roofline"][k] for k in ("achieved", "peak", "unit", "frac")}
            ceil = measured_valu_ceiling(ctp, torch, dev)
            line["roofline"] = {"bound": "alu", "kernel": dom, **{k: alu[k] for k in ("achieved", "peak", "unit", "frac")},
                                "traffic": traffic, "flops": alu["flops"], "hbm": hbm,
                                "measured_ceiling": round(ceil, 2), "frac_of_measured": round(tf / ceil, 4)}
        else:
            line["roofline"]["alu"] = alu
    if wl.get("cpu") and not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl["cpu"], args.cpu_sample_nodes)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs for the conv tensor-product workloads.

This module only draws random inputs and builds graph index arrays.  It holds
none of the method's arithmetic (no Clebsch-Gordan coefficients, no spherical
harmonics, no convolution): both the oracle and the HIP path are fed from here.

Workload shapes follow the e3j paper (arXiv 2609.35099): Table 1 (convolution
throughput at 45 average neighbours, N*C = 2^22 at lmax=2 and 2^21 at lmax=3)
and Table 2 / Table 3 (a 1503-atom, 25 A water box with a 5 A cutoff and a
static edge count of 83,325 after 10% padding).  The pages give no graphs or
structures, so every input here is synthetic:

* graph: every receiver i draws deg_i ~ Poisson(mean_deg) senders uniformly,
  with replacement, from the other N-1 nodes (draw in [0, N-1), values >= i
  shifted up by one, so no self-edges).  Edges are receiver-major, so they
  are already in CSR order.
* tiny graph: every receiver gets exactly `deg` distinct senders.
* edge vectors: normalised Gaussian (uniform on the sphere).
* features, weights, output gradients: standard normal, fp32.
* water box: uniform positions in a periodic cube, minimum-image neighbour
  list, padding edges (zero weight) spread round-robin over receivers.

Small arrays come from numpy's PCG64 (`numpy.random.default_rng(seed)`), drawn
in the order graph -> vec -> x -> w -> G.  Arrays too large to draw on the host
in reasonable time (full-size w and G) come from torch's generator on the
target device, seeded from (seed, tag); `normal_tensor` documents the scheme.
"""
from __future__ import annotations

import numpy as np

# (l_in, l_sh, l_out) are equal in the named workloads below; poisson_degrees
# draws small graphs with independent degrees.
TINY = dict(name="tiny", n_nodes=64, channels=16, lmax=1, deg=16)
L2_FWD = dict(name="l2fwd", n_nodes=32768, channels=128, lmax=2, mean_deg=45.0)
L3_FB = dict(name="l3fb", n_nodes=16384, channels=128, lmax=3, mean_deg=45.0)
SWEEP_CHANNELS = (64, 128, 256, 512, 1024)
# node-local tensor product (no graph): x, y, G ~ N(0,1) [N][D][C], w [N][P][C]
NODE = dict(name="node3", n_nodes=131072, channels=128, lmax=3)
WATER = dict(name="water", n_atoms=1503, box=25.0, cutoff=5.0, n_edges=83325,
             channels=128, lmax=3, n_bessel=8, hidden=64)


def rng_for(seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(seed)


def csr_from_degrees(deg: np.ndarray) -> np.ndarray:
    row_ptr = np.zeros(deg.size + 1, dtype=np.int64)
    np.cumsum(deg, out=row_ptr[1:])
    if row_ptr[-1] >= 2**31:
        raise ValueError("edge count does not fit int32")
    return row_ptr.astype(np.int32)


def poisson_graph(n_nodes: int, mean_deg: float, rng: np.random.Generator):
    """CSR-by-receiver graph with Poisson in-degrees and uniform senders."""
    if n_nodes < 2:
        raise ValueError("need at least two nodes")
    deg = rng.poisson(mean_deg, size=n_nodes).astype(np.int64)
    row_ptr = csr_from_degrees(deg)
    recv = np.repeat(np.arange(n_nodes, dtype=np.int64), deg)
    s = rng.integers(0, n_nodes - 1, size=recv.size, dtype=np.int64)
    s = s + (s >= recv)
    return row_ptr, s.astype(np.int32)


def gather_limited_graphs(n_nodes: int, mean_deg: float, k: int, rng: np.random.Generator):
    """Two graphs of the Poisson workload's size whose node-row gathers touch
    only nodes 0..k-1 (a cache-footprint diagnostic, not a workload of the
    method): (a) Poisson(mean_deg) in-degrees over all receivers with senders
    uniform over 0..k-1, so the forward gathers x from k rows; (b) as many
    edges with receivers uniform over 0..k-1 (CSR order) and senders uniform
    over all nodes, so the backward gathers G from k rows.  Self-edges are
    allowed.  Returns ((row_ptr, senders), (row_ptr, senders))."""
    deg = rng.poisson(mean_deg, size=n_nodes).astype(np.int64)
    rp_a = csr_from_degrees(deg)
    e = int(rp_a[-1])
    s_a = rng.integers(0, k, size=e, dtype=np.int64).astype(np.int32)
    recv_b = np.sort(rng.integers(0, k, size=e, dtype=np.int64))
    rp_b = csr_from_degrees(np.bincount(recv_b, minlength=n_nodes).astype(np.int64))
    s_b = rng.integers(0, n_nodes, size=e, dtype=np.int64).astype(np.int32)
    return (rp_a, s_a), (rp_b, s_b)


def distinct_sender_graph(n_nodes: int, deg: int, rng: np.random.Generator):
    """Every receiver gets `deg` distinct senders drawn from the other nodes."""
    if deg > n_nodes - 1:
        raise ValueError("degree exceeds the number of other nodes")
    row_ptr = csr_from_degrees(np.full(n_nodes, deg, dtype=np.int64))
    senders = np.empty(n_nodes * deg, dtype=np.int32)
    for i in range(n_nodes):
        s = rng.choice(n_nodes - 1, size=deg, replace=False)
        senders[i * deg:(i + 1) * deg] = s + (s >= i)
    return row_ptr, senders


def unit_vectors(n: int, rng: np.random.Generator) -> np.ndarray:
    v = rng.standard_normal((n, 3))
    norm = np.linalg.norm(v, axis=1, keepdims=True)
    # A zero draw has probability zero; guard anyway so no zero vector leaves.
    norm[norm == 0] = 1.0
    v[(v == 0).all(axis=1)] = (0.0, 0.0, 1.0)
    return (v / norm).astype(np.float32)


def normal(shape, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def normal_tensor(shape, seed: int, tag: int, device):
    """Standard-normal fp32 tensor drawn by torch's generator on `device`.

    The generator is seeded with seed * 1000003 + tag, so each array of a
    workload (tag 1: x, 2: w, 3: G) has its own reproducible stream.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(tag))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)


def num_paths(lmax: int) -> int:
    """Number of (l1, l2, l3) triples with all l <= lmax obeying the triangle rule.

    Only a count, used to size the weight array; the path list itself belongs
    to the oracle and to the library.
    """
    return sum(1 for a in range(lmax + 1) for b in range(lmax + 1)
               for c in range(lmax + 1) if abs(a - b) <= c <= a + b)


# ---------------------------------------------------------------- workloads


def tiny(seed: int = 0):
    """64 nodes, 16 channels, l <= 1, 16 distinct senders per node."""
    cfg = TINY
    rng = rng_for(seed)
    n, c, L = cfg["n_nodes"], cfg["channels"], cfg["lmax"]
    row_ptr, senders = distinct_sender_graph(n, cfg["deg"], rng)
    e = senders.size
    vec = unit_vectors(e, rng)
    d = (L + 1) ** 2
    x = normal((n, d, c), rng)
    w = normal((e, num_paths(L), c), rng)
    g = normal((n, d, c), rng)
    return dict(name="tiny", n_nodes=n, n_edges=e, channels=c, lmax=L,
                row_ptr=row_ptr, senders=senders, vec=vec, x=x, w=w, grad_out=g)


def poisson_small(n_nodes: int, channels: int, lmax: int, mean_deg: float = 45.0,
                  seed: int = 0):
    """Same law as the full-size graphs, at a size the oracle finishes quickly."""
    rng = rng_for(seed)
    row_ptr, senders = poisson_graph(n_nodes, mean_deg, rng)
    e = senders.size
    vec = unit_vectors(e, rng)
    d = (lmax + 1) ** 2
    x = normal((n_nodes, d, channels), rng)
    w = normal((e, num_paths(lmax), channels), rng)
    g = normal((n_nodes, d, channels), rng)
    return dict(name=f"poisson_n{n_nodes}_c{channels}_l{lmax}", n_nodes=n_nodes,
                n_edges=e, channels=channels, lmax=lmax, row_ptr=row_ptr,
                senders=senders, vec=vec, x=x, w=w, grad_out=g)


def poisson_degrees(n_nodes: int, channels: int, l_in: int, l_sh: int, n_paths: int, out_dim: int,
                    mean_deg: float = 12.0, seed: int = 0):
    """Small Poisson workload with independent degrees: x [N][(l_in+1)^2][C],
    vec [E][3] (the caller evaluates Y up to l_sh), w [E][n_paths][C] and
    grad_out [N][out_dim][C].  The path count and output width are passed in
    (they belong to the oracle and the library), so this draws only shapes."""
    rng = rng_for(seed)
    row_ptr, senders = poisson_graph(n_nodes, mean_deg, rng)
    e = senders.size
    vec = unit_vectors(e, rng)
    x = normal((n_nodes, (l_in + 1) ** 2, channels), rng)
    w = normal((e, n_paths, channels), rng)
    g = normal((n_nodes, out_dim, channels), rng)
    return dict(name=f"poisson_n{n_nodes}_c{channels}_deg{l_in}{l_sh}", n_nodes=n_nodes, n_edges=e,
                channels=channels, lmax=None, l_sh=l_sh, row_ptr=row_ptr, senders=senders, vec=vec, x=x, w=w,
                grad_out=g)


def poisson_full(n_nodes: int, channels: int, lmax: int, device, mean_deg: float = 45.0,
                 seed: int = 0, need_grad: bool = True):
    """Full-size Poisson workload: graph and vec on the host (PCG64), x, w and
    G drawn on `device` by torch (see `normal_tensor`)."""
    rng = rng_for(seed)
    row_ptr, senders = poisson_graph(n_nodes, mean_deg, rng)
    e = senders.size
    vec = unit_vectors(e, rng)
    d = (lmax + 1) ** 2
    out = dict(name=f"poisson_n{n_nodes}_c{channels}_l{lmax}", n_nodes=n_nodes,
               n_edges=e, channels=channels, lmax=lmax, row_ptr=row_ptr,
               senders=senders, vec=vec)
    out["x"] = normal_tensor((n_nodes, d, channels), seed, 1, device)
    out["w"] = normal_tensor((e, num_paths(lmax), channels), seed, 2, device)
    if need_grad:
        out["grad_out"] = normal_tensor((n_nodes, d, channels), seed, 3, device)
    return out


def fixed_degree_large(n_nodes: int, deg: int, channels: int, lmax: int, device, seed: int = 0):
    """Large-offset workload: every receiver draws `deg` senders uniformly from
    the other nodes (host PCG64, as poisson_graph), so E = n_nodes * deg; x, w,
    G, a Y-given array (standard normal values, not harmonics: the Y-given
    operation takes any Y) and Gaussian edge vectors are drawn on `device`
    (tags 21..25).  Sized so that E * P * C passes 2^31, the edge rows of w and
    dw lie beyond 32-bit element offsets."""
    rng = rng_for(seed)
    e = n_nodes * deg
    if e >= 2**31:
        raise ValueError("edge count does not fit int32")
    row_ptr = (np.arange(n_nodes + 1, dtype=np.int64) * deg).astype(np.int32)
    recv = np.repeat(np.arange(n_nodes, dtype=np.int32), deg)
    s = rng.integers(0, n_nodes - 1, size=e, dtype=np.int32)
    s += (s >= recv)
    del recv
    d = (lmax + 1) ** 2
    return dict(name=f"fixed_n{n_nodes}_deg{deg}_c{channels}_l{lmax}", n_nodes=n_nodes, n_edges=e,
                channels=channels, lmax=lmax, row_ptr=row_ptr, senders=s,
                x=normal_tensor((n_nodes, d, channels), seed, 21, device),
                w=normal_tensor((e, num_paths(lmax), channels), seed, 22, device),
                grad_out=normal_tensor((n_nodes, d, channels), seed, 23, device),
                y=normal_tensor((e, d), seed, 24, device),
                vec=normal_tensor((e, 3), seed, 25, device))


def water_box_graph(seed: int = 0, n_atoms: int = 1503, box: float = 25.0,
                    cutoff: float = 5.0, n_edges: int = 83325):
    """Periodic random 'water box': CSR neighbour list padded to n_edges.

    Real edges are ordered pairs i != j with minimum-image distance < cutoff,
    receiver i, sender j, vec = pos[j] - pos[i] (minimum image).  Padding
    edges go to receivers round-robin (k mod N) with sender (i+1) mod N and
    their true minimum-image vector; `mask` is 0 on them.  Edges are then
    re-sorted stably by receiver.
    """
    rng = rng_for(seed)
    pos = rng.uniform(0.0, box, size=(n_atoms, 3))
    recv_l, send_l, vec_l = [], [], []
    for i in range(n_atoms):
        d = pos - pos[i]
        d -= box * np.round(d / box)
        r = np.linalg.norm(d, axis=1)
        nb = np.nonzero((r < cutoff) & (np.arange(n_atoms) != i))[0]
        recv_l.append(np.full(nb.size, i))
        send_l.append(nb)
        vec_l.append(d[nb])
    recv = np.concatenate(recv_l)
    send = np.concatenate(send_l)
    vec = np.concatenate(vec_l)
    n_real = recv.size
    if n_real > n_edges:
        raise ValueError(f"{n_real} real edges exceed the static count {n_edges}")
    n_pad = n_edges - n_real
    pr = np.arange(n_pad) % n_atoms
    ps = (pr + 1) % n_atoms
    pd = pos[ps] - pos[pr]
    pd -= box * np.round(pd / box)
    recv = np.concatenate([recv, pr])
    send = np.concatenate([send, ps])
    vec = np.concatenate([vec, pd])
    mask = np.concatenate([np.ones(n_real), np.zeros(n_pad)])
    order = np.argsort(recv, kind="stable")
    recv, send, vec, mask = recv[order], send[order], vec[order], mask[order]
    row_ptr = csr_from_degrees(np.bincount(recv, minlength=n_atoms))
    return dict(n_nodes=n_atoms, n_edges=n_edges, n_real=n_real, pos=pos,
                row_ptr=row_ptr, senders=send.astype(np.int32),
                vec=vec.astype(np.float32), mask=mask.astype(np.float32), rng=rng)


def radial_mlp_weights(vec: np.ndarray, mask: np.ndarray, n_paths: int, channels: int,
                       rng: np.random.Generator, cutoff: float = 5.0, n_bessel: int = 8,
                       hidden: int = 64, device="cpu"):
    """Per-edge weights w[E, P, C] from a random radial MLP.

    Features: sqrt(2/rc) sin(n pi r / rc) / r for n = 1..n_bessel.  MLP
    n_bessel -> hidden -> hidden -> P*C with SiLU after both hidden layers,
    weights ~ N(0, 1/fan_in), zero biases.  Padded edges (mask 0) get w = 0.
    The MLP is part of the synthetic input, not of the convolution.
    """
    import torch
    r = np.linalg.norm(vec.astype(np.float64), axis=1)
    n = np.arange(1, n_bessel + 1)
    feat = np.sqrt(2.0 / cutoff) * np.sin(np.outer(r, n) * np.pi / cutoff) / r[:, None]
    w1 = rng.standard_normal((n_bessel, hidden)) / np.sqrt(n_bessel)
    w2 = rng.standard_normal((hidden, hidden)) / np.sqrt(hidden)
    w3 = rng.standard_normal((hidden, n_paths * channels)) / np.sqrt(hidden)
    t = lambda a: torch.as_tensor(a, dtype=torch.float32, device=device)
    h = torch.nn.functional.silu(t(feat) @ t(w1))
    h = torch.nn.functional.silu(h @ t(w2))
    out = (h @ t(w3)) * t(mask)[:, None]
    return out.reshape(vec.shape[0], n_paths, channels).contiguous()


def water_box(seed: int = 0, device="cpu", channels: int = 128, lmax: int = 3):
    """The two-layer water-box workload: graph, x0, w1, w2 and G."""
    g = water_box_graph(seed)
    rng = g.pop("rng")
    P = num_paths(lmax)
    d = (lmax + 1) ** 2
    x0 = normal((g["n_nodes"], d, channels), rng)
    w1 = radial_mlp_weights(g["vec"], g["mask"], P, channels, rng, device=device)
    w2 = radial_mlp_weights(g["vec"], g["mask"], P, channels, rng, device=device)
    grad = normal((g["n_nodes"], d, channels), rng)
    g.update(name="water", channels=channels, lmax=lmax, x=x0, w1=w1, w2=w2, grad_out=grad)
    return g


def node_small(n_nodes: int, channels: int, lmax: int, seed: int = 0):
    """Node-local tensor-product inputs drawn on the host: x, y, w, G."""
    rng = rng_for(seed)
    d = (lmax + 1) ** 2
    x = normal((n_nodes, d, channels), rng)
    y = normal((n_nodes, d, channels), rng)
    w = normal((n_nodes, num_paths(lmax), channels), rng)
    g = normal((n_nodes, d, channels), rng)
    return dict(name=f"node_n{n_nodes}_c{channels}_l{lmax}", n_nodes=n_nodes, channels=channels,
                lmax=lmax, x=x, y=y, w=w, grad_out=g)


def node_full(n_nodes: int, channels: int, lmax: int, device, seed: int = 0):
    """Full-size node-local inputs drawn on `device` (tags 11 x, 12 y, 13 w, 14 G)."""
    d = (lmax + 1) ** 2
    return dict(name=f"node_n{n_nodes}_c{channels}_l{lmax}", n_nodes=n_nodes, channels=channels,
                lmax=lmax,
                x=normal_tensor((n_nodes, d, channels), seed, 11, device),
                y=normal_tensor((n_nodes, d, channels), seed, 12, device),
                w=normal_tensor((n_nodes, num_paths(lmax), channels), seed, 13, device),
                grad_out=normal_tensor((n_nodes, d, channels), seed, 14, device))


def cotangents_small(d: dict, seed: int = 0):
    """Cotangents (ax, aw, aY) of the backward's outputs for a small workload,
    N(0,1) fp32 from their own PCG64 stream."""
    rng = rng_for(seed + 7919)
    return (normal(d["x"].shape, rng), normal(d["w"].shape, rng),
            normal((d["n_edges"], (d["lmax"] + 1) ** 2), rng))


def cotangents_full(d: dict, device, seed: int = 0):
    """Full-size cotangents: ax and aw on `device` (tags 4, 5), aY on the host."""
    n, e, c, L = d["n_nodes"], d["n_edges"], d["x"].shape[2], d["lmax"]
    ax = normal_tensor(d["x"].shape, seed, 4, device)
    aw = normal_tensor((e, num_paths(L), c), seed, 5, device)
    aY = normal((e, (L + 1) ** 2), rng_for(seed + 7919))
    return ax, aw, aY

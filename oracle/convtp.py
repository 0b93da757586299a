"""The convolution tensor product and its VJP, two plain fp64 forms.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

1. `materialised_*` (numpy): the definition as e3nn evaluates it (e3j paper,
   arXiv 2609.35099, Table 1 caption: messages are materialised), i.e.
   build every per-edge message, then scatter-add into receivers.  Vectorised
   with einsum per path; memory grows with E * D * C, so small inputs only.
2. `fwd`, `bwd_dx`, `bwd_edges` (C, OpenMP): a naive per-receiver /
   per-sender / per-edge loop over the same definition (convtp_oracle.c) that
   can evaluate any subset of rows of a full-size workload.

Both take x[N][D1][C], Y[E][D2], w[E][P][C], G[N][D3][C] and CSR-by-receiver
(row_ptr, senders); component index d(l, m) = l^2 + l + m; paths in
lexicographic (l1, l2, l3) order; all paths that share l3 are summed into the
same output block.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import cg as _cg
from . import graph as _graph

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB names another build of the C loop (the sanitizer test's)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "convtp_oracle.c")


def build(force: bool = True) -> str:
    """Compile convtp_oracle.c into liboracle.so with gcc (-O2 -fopenmp)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.oracle_fwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, I, P, P, I]
        L.oracle_bwd_dx.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, I, P, P, I]
        L.oracle_bwd_edge.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, I, P, P, P, I]
        for f in (L.oracle_fwd, L.oracle_bwd_dx, L.oracle_bwd_edge):
            f.restype = I
        L.oracle_max_threads.restype = I
        _lib = L
    return _lib


def max_threads() -> int:
    return int(lib().oracle_max_threads())


class Problem:
    """Path list, output blocks and dense coupling blocks for (l_in, l_sh, l_out).

    variant 0: every triangle path; paths sharing l3 add into one output block
    (l3^2 .. (l3+1)^2 - 1).  variant 1 (MACE's convolution, the implementation
    e3j's Table 2 matches): natural-parity paths only, each writing an output
    slot of its own, slots in path order; out and G then have D3 = sum of
    2 l3 + 1 components."""

    def __init__(self, l_in: int, l_sh: int, l_out: int, variant: int = 0):
        self.l_in, self.l_sh, self.l_out, self.variant = l_in, l_sh, l_out, variant
        self.paths = _cg.paths(l_in, l_sh, l_out, natural=(variant == 1))
        self.P = len(self.paths)
        self.D1, self.D2 = _cg.dim(l_in), _cg.dim(l_sh)
        if variant == 0:
            self.o3 = np.array([l3 * l3 for (_, _, l3) in self.paths], dtype=np.int32)
            self.D3 = _cg.dim(l_out)
        else:
            sizes = [2 * l3 + 1 for (_, _, l3) in self.paths]
            self.o3 = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int32) if sizes else \
                np.zeros(0, dtype=np.int32)
            self.D3 = int(sum(sizes))
        blocks = [_cg.real_cg(*p) for p in self.paths]
        self.blocks = blocks
        offs = np.zeros(self.P, dtype=np.int64)
        if self.P:
            offs[1:] = np.cumsum([b.size for b in blocks])[:-1]
        self.cg_off = offs
        self.cg_flat = (np.concatenate([b.ravel() for b in blocks]) if blocks
                        else np.zeros(0)).astype(np.float64)
        self.l123 = np.array(self.paths, dtype=np.int32).reshape(-1, 3)

    def oslice(self, p: int) -> slice:
        """Output components of path p."""
        l3 = self.paths[p][2]
        return slice(int(self.o3[p]), int(self.o3[p]) + 2 * l3 + 1)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _c64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# ------------------------------------------------------------ numpy definition


def materialised_fwd(prob: Problem, x, Y, w, row_ptr, senders):
    """out[N][D3][C]: every message built explicitly, then scatter-added.

    einsum(optimize=True) only picks the pairwise contraction order of each
    path's product; the arithmetic is the definition term by term."""
    x = np.asarray(x, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n, _, c = x.shape
    e = len(senders)
    recv = _graph.receivers_of(row_ptr)
    msg = np.zeros((e, prob.D3, c))
    for p, (l1, l2, l3) in enumerate(prob.paths):
        Cp = prob.blocks[p]
        xs = x[senders, l1 * l1:(l1 + 1) ** 2, :]
        ys = Y[:, l2 * l2:(l2 + 1) ** 2]
        msg[:, prob.oslice(p), :] += w[:, p, None, :] * np.einsum(
            "abk,eac,eb->ekc", Cp, xs, ys, optimize=True)
    out = np.zeros((n, prob.D3, c))
    np.add.at(out, recv, msg)
    return out


def materialised_bwd(prob: Problem, x, Y, w, G, row_ptr, senders):
    """(dx, dw, dY): the VJP of materialised_fwd for upstream gradient G."""
    x = np.asarray(x, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    n, _, c = x.shape
    recv = _graph.receivers_of(row_ptr)
    gd = G[recv]
    dx_e = np.zeros((len(senders), prob.D1, c))
    dw = np.zeros_like(w)
    dY = np.zeros_like(Y)
    for p, (l1, l2, l3) in enumerate(prob.paths):
        Cp = prob.blocks[p]
        s1 = slice(l1 * l1, (l1 + 1) ** 2)
        s2 = slice(l2 * l2, (l2 + 1) ** 2)
        s3 = prob.oslice(p)
        xs, ys, gs = x[senders, s1, :], Y[:, s2], gd[:, s3, :]
        dx_e[:, s1, :] += w[:, p, None, :] * np.einsum("abk,eb,ekc->eac", Cp, ys, gs, optimize=True)
        dw[:, p, :] = np.einsum("abk,eac,eb,ekc->ec", Cp, xs, ys, gs, optimize=True)
        dY[:, s2] += np.einsum("abk,ec,eac,ekc->eb", Cp, w[:, p, :], xs, gs,
                                 optimize=True)
    dx = np.zeros((n, prob.D1, c))
    np.add.at(dx, senders, dx_e)
    return dx, dw, dY


# ------------------------------------------------------------ C edge loop


def fwd(prob: Problem, x, Y, w, row_ptr, senders, rows=None, n_threads=None):
    """out rows (receivers `rows`, default all) via the C edge loop, fp64."""
    x, w, Y = _c32(x), _c32(w), _c64(Y)
    row_ptr, senders = _i32(row_ptr), _i32(senders)
    n, _, c = x.shape
    rows = _i32(np.arange(n) if rows is None else rows)
    out = np.zeros((rows.size, prob.D3, c))
    nt = n_threads or max_threads()
    rc = lib().oracle_fwd(c, prob.D1, prob.D2, prob.D3, prob.P, _ptr(prob.l123), _ptr(prob.o3),
                          _ptr(prob.cg_flat), _ptr(prob.cg_off), _ptr(x), _ptr(Y), _ptr(w),
                          _ptr(row_ptr), _ptr(senders), rows.size, _ptr(rows), _ptr(out), nt)
    if rc:
        raise MemoryError("oracle_fwd could not allocate its message buffer")
    return out


def bwd_dx(prob: Problem, Y, w, G, send_ptr, send_perm, send_recv, rows=None,
           n_threads=None):
    """dx rows (senders `rows`, default all), fp64."""
    w, G, Y = _c32(w), _c32(G), _c64(Y)
    send_ptr, send_perm, send_recv = _i32(send_ptr), _i32(send_perm), _i32(send_recv)
    n = send_ptr.size - 1
    c = G.shape[2]
    rows = _i32(np.arange(n) if rows is None else rows)
    dx = np.zeros((rows.size, prob.D1, c))
    nt = n_threads or max_threads()
    lib().oracle_bwd_dx(c, prob.D1, prob.D2, prob.D3, prob.P, _ptr(prob.l123), _ptr(prob.o3),
                        _ptr(prob.cg_flat), _ptr(prob.cg_off), _ptr(Y), _ptr(w), _ptr(G),
                        _ptr(send_ptr), _ptr(send_perm), _ptr(send_recv),
                        rows.size, _ptr(rows), _ptr(dx), nt)
    return dx


def bwd_edges(prob: Problem, x, Y, w, G, row_ptr, senders, rows=None, n_threads=None):
    """(dw, dY) rows (edges `rows`, default all), fp64."""
    x, w, G, Y = _c32(x), _c32(w), _c32(G), _c64(Y)
    senders = _i32(senders)
    recv = _i32(_graph.receivers_of(row_ptr))
    e = senders.size
    c = x.shape[2]
    rows = _i32(np.arange(e) if rows is None else rows)
    dw = np.zeros((rows.size, prob.P, c))
    dY = np.zeros((rows.size, prob.D2))
    nt = n_threads or max_threads()
    lib().oracle_bwd_edge(c, prob.D1, prob.D2, prob.D3, prob.P, _ptr(prob.l123), _ptr(prob.o3),
                          _ptr(prob.cg_flat), _ptr(prob.cg_off), _ptr(x), _ptr(Y), _ptr(w),
                          _ptr(G), _ptr(senders), _ptr(recv), rows.size, _ptr(rows),
                          _ptr(dw), _ptr(dY), nt)
    return dw, dY


# ------------------------------------------------------------ VJP of the VJP (numpy)


def materialised_double_bwd(prob: Problem, x, Y, w, G, ax, aw, aY, row_ptr, senders):
    """Gradients of  L2 = <ax, dx> + <aw, dw> + <aY, dY>  (the backward's
    outputs (dx, dw, dY) of materialised_bwd, paired with cotangents ax, aw,
    aY) with respect to x, w, Y and G: returns (gx, gw, gY, gG).

    The forward is trilinear in (x, w, Y), so each derivative is a sum of the
    backward's contractions with one operand replaced by its cotangent; the
    terms are written out per path, message by message (FlashCart, arXiv
    2610.06409, section on symbolic VJPs: the VJP-of-VJP of the edge
    convolution)."""
    x, Y, w, G = (np.asarray(a, dtype=np.float64) for a in (x, Y, w, G))
    ax, aw, aY = (np.asarray(a, dtype=np.float64) for a in (ax, aw, aY))
    n, _, c = x.shape
    recv = _graph.receivers_of(row_ptr)
    gd = G[recv]
    gx_e = np.zeros((len(senders), prob.D1, c))
    gG_e = np.zeros((len(senders), prob.D3, c))
    gw = np.zeros_like(w)
    gY = np.zeros_like(Y)
    for p, (l1, l2, l3) in enumerate(prob.paths):
        Cp = prob.blocks[p]
        s1 = slice(l1 * l1, (l1 + 1) ** 2)
        s2 = slice(l2 * l2, (l2 + 1) ** 2)
        s3 = prob.oslice(p)
        xs, axs, ys, ays, gs = x[senders, s1, :], ax[senders, s1, :], Y[:, s2], aY[:, s2], gd[:, s3, :]
        wp, awp = w[:, p, None, :], aw[:, p, None, :]
        # G enters every term of L2 linearly: gG = the three forwards with one
        # operand replaced by its cotangent
        gG_e[:, s3, :] += (wp * np.einsum("abk,eac,eb->ekc", Cp, axs, ys, optimize=True)
                           + awp * np.einsum("abk,eac,eb->ekc", Cp, xs, ys, optimize=True)
                           + wp * np.einsum("abk,eac,eb->ekc", Cp, xs, ays, optimize=True))
        # x appears in <aw, dw> and <aY, dY>
        gx_e[:, s1, :] += (awp * np.einsum("abk,eb,ekc->eac", Cp, ys, gs, optimize=True)
                           + wp * np.einsum("abk,eb,ekc->eac", Cp, ays, gs, optimize=True))
        # w appears in <ax, dx> and <aY, dY>
        gw[:, p, :] = (np.einsum("abk,eac,eb,ekc->ec", Cp, axs, ys, gs, optimize=True)
                       + np.einsum("abk,eac,eb,ekc->ec", Cp, xs, ays, gs, optimize=True))
        # Y appears in <ax, dx> and <aw, dw>
        gY[:, s2] += (np.einsum("abk,ec,eac,ekc->eb", Cp, w[:, p, :], axs, gs, optimize=True)
                      + np.einsum("abk,ec,eac,ekc->eb", Cp, aw[:, p, :], xs, gs, optimize=True))
    gx = np.zeros((n, prob.D1, c))
    np.add.at(gx, senders, gx_e)
    gG = np.zeros((n, prob.D3, c))
    np.add.at(gG, recv, gG_e)
    return gx, gw, gY, gG

"""Torch-facing binding of libconvtp.so: argument marshalling only.

Every computation runs in the library's HIP kernels; this module checks
tensor metadata, passes raw device pointers and the current HIP stream, and
turns a non-zero status into `ConvTPError`.  PyTorch provides device memory
and streams, nothing else.

Degrees: every call takes `lmax`, either one int L (l_in = l_sh = l_out = L)
or a tuple (l_in, l_sh, l_out), each in 0..3.

Shapes (channel index fastest, D_l = (l+1)^2, P and D_out from `layout`):
    x, dx                : [N, D_in, C]  float32
    out, grad_out        : [N, D_out, C] float32 (D_out = D_{l_out} for variant 0)
    w, dw                : [E, P, C]     float32
    Y, dY                : [E, D_sh]     float32  (y_mode 0)
    vec, dvec            : [E, 3]        float32  (y_mode 1)
    row_ptr [N+1], senders [E], send_ptr [N+1], send_perm [E], send_recv [E]: int32
"""
from __future__ import annotations

import ctypes
import functools

import numpy as np
import torch

from . import _capi
from ._capi import ConvTPError, Problem, check, lib  # noqa: F401

Y_GIVEN, VEC_GIVEN = 0, 1
ALGO_CSR, ALGO_ATOMIC, ALGO_FRAME = 0, 1, 2   # ALGO_FRAME: edge-frame forward (edge vectors)
SUMMED, SLOTS = 0, 1          # path variants (conv_tp_problem.variant)


def _p(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)



def _want(t, name, shape, dtype=torch.float32, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def dim(l: int) -> int:
    return (l + 1) ** 2


def degrees(lmax):
    """(l_in, l_sh, l_out) from an int L or a 3-tuple."""
    if isinstance(lmax, (tuple, list)):
        if len(lmax) != 3:
            raise ValueError("lmax must be an int or (l_in, l_sh, l_out)")
        return tuple(int(v) for v in lmax)
    return (int(lmax),) * 3


def num_paths(l_in: int, l_sh: int = None, l_out: int = None) -> int:
    l_sh = l_in if l_sh is None else l_sh
    l_out = l_in if l_out is None else l_out
    n = lib().conv_tp_num_paths(l_in, l_sh, l_out)
    if n < 0:
        raise ConvTPError(_capi.CTP_EUNSUPPORTED, lib().conv_tp_last_error().decode())
    return n


def paths(l_in: int, l_sh: int = None, l_out: int = None):
    l_sh = l_in if l_sh is None else l_sh
    l_out = l_in if l_out is None else l_out
    n = num_paths(l_in, l_sh, l_out)
    buf = np.zeros((n, 3), dtype=np.int32)
    check(lib().conv_tp_paths(l_in, l_sh, l_out, buf.ctypes.data_as(ctypes.c_void_p)))
    return [tuple(int(v) for v in r) for r in buf]


def layout(lmax, variant: int = SUMMED):
    """(paths, out_dim) of a variant: the path list in w's order and the
    number of output components per channel."""
    ps, d = _layout(degrees(lmax), int(variant))
    return list(ps), d


@functools.lru_cache(maxsize=None)
def _layout(deg, variant):
    # the library's answer for a (degrees, variant) pair never changes: asked once
    a, b, c = deg
    n, d = ctypes.c_int32(0), ctypes.c_int32(0)
    check(lib().conv_tp_layout(variant, a, b, c, ctypes.byref(n), ctypes.byref(d), None))
    buf = np.zeros((n.value, 3), dtype=np.int32)
    check(lib().conv_tp_layout(variant, a, b, c, ctypes.byref(n), ctypes.byref(d),
                               buf.ctypes.data_as(ctypes.c_void_p)))
    return tuple(tuple(int(v) for v in r) for r in buf), int(d.value)


def coupling(l1: int, l2: int, l3: int) -> np.ndarray:
    out = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1), dtype=np.float64)
    check(lib().conv_tp_coupling(l1, l2, l3, out.ctypes.data_as(ctypes.c_void_p)))
    return out


class Graph:
    """A static CSR-by-receiver graph on a device, with its sender transpose.

    The transpose (send_ptr, send_perm, send_recv) is built once by
    conv_tp_build_transpose and reused by every backward pass.
    """

    def __init__(self, n_nodes: int, row_ptr: torch.Tensor, senders: torch.Tensor):
        self.n_nodes = int(n_nodes)
        self.n_edges = int(senders.numel())
        _want(row_ptr, "row_ptr", (self.n_nodes + 1,), torch.int32)
        _want(senders, "senders", (self.n_edges,), torch.int32, row_ptr.device)
        self.row_ptr, self.senders = row_ptr, senders
        self.device = row_ptr.device
        self._t = None

    @property
    def transpose(self):
        if self._t is None:
            self._t = build_transpose(self.n_nodes, self.row_ptr, self.senders)
        return self._t

    def check(self) -> int:
        return check_graph(self.n_nodes, self.row_ptr, self.senders)


def build_transpose(n_nodes: int, row_ptr: torch.Tensor, senders: torch.Tensor):
    n_edges = senders.numel()
    _want(row_ptr, "row_ptr", (n_nodes + 1,), torch.int32)
    _want(senders, "senders", (n_edges,), torch.int32, row_ptr.device)
    dev = row_ptr.device
    send_ptr = torch.empty(n_nodes + 1, dtype=torch.int32, device=dev)
    send_perm = torch.empty(n_edges, dtype=torch.int32, device=dev)
    send_recv = torch.empty(n_edges, dtype=torch.int32, device=dev)
    check(lib().conv_tp_build_transpose(n_nodes, n_edges, _p(row_ptr), _p(senders), _p(send_ptr),
                                        _p(send_perm), _p(send_recv), _stream(row_ptr)))
    return send_ptr, send_perm, send_recv


def check_graph(n_nodes: int, row_ptr: torch.Tensor, senders: torch.Tensor) -> int:
    n_edges = senders.numel()
    _want(row_ptr, "row_ptr", (n_nodes + 1,), torch.int32)
    _want(senders, "senders", (n_edges,), torch.int32, row_ptr.device)
    bad = ctypes.c_int64(0)
    check(lib().conv_tp_check_graph(n_nodes, n_edges, _p(row_ptr), _p(senders), ctypes.byref(bad),
                                    _stream(row_ptr)))
    return int(bad.value)


def _problem(n_nodes, n_edges, channels, lmax, y_mode, algo, variant=SUMMED) -> Problem:
    a, b, c = degrees(lmax)
    return Problem(n_nodes, n_edges, channels, a, b, c, y_mode, algo, variant)


def _shapes(x, y_or_vec, w, graph, lmax, y_mode, variant=SUMMED):
    n, e = graph.n_nodes, graph.n_edges
    l_in, l_sh, _ = degrees(lmax)
    if x.dim() != 3:
        raise ValueError("x must be [N, D, C]")
    c = x.shape[2]
    _want(x, "x", (n, dim(l_in), c), device=graph.device)
    _want(y_or_vec, "y_or_vec", (e, dim(l_sh) if y_mode == Y_GIVEN else 3), device=graph.device)
    _want(w, "w", (e, len(_layout(degrees(lmax), int(variant))[0]), c), device=graph.device)
    return n, e, c


def out_dim(lmax, variant: int = SUMMED) -> int:
    return _layout(degrees(lmax), int(variant))[1]


def conv_tp_fwd(x, y_or_vec, w, graph: Graph, lmax: int, y_mode: int = Y_GIVEN, algo: int = ALGO_CSR,
                out=None, variant: int = SUMMED):
    """out[N, D_out, C] = conv(x, Y or vec, w) on `graph` (see include/convtp.h)."""
    n, e, c = _shapes(x, y_or_vec, w, graph, lmax, y_mode, variant)
    do = out_dim(lmax, variant)
    if out is None:
        out = torch.empty((n, do, c), dtype=torch.float32, device=x.device)
    _want(out, "out", (n, do, c), device=x.device)
    prob = _problem(n, e, c, lmax, y_mode, algo, variant)
    check(lib().conv_tp_fwd(ctypes.byref(prob), _p(x), _p(y_or_vec), _p(w), _p(graph.row_ptr),
                            _p(graph.senders), _p(out), _stream(x)))
    return out


def conv_tp_bwd(grad_out, x, y_or_vec, w, graph: Graph, lmax: int, y_mode: int = Y_GIVEN,
                dx=None, dw=None, dy=None, variant: int = SUMMED, algo: int = ALGO_CSR):
    """(dx, dw, dY or dvec) for upstream gradient grad_out (see include/convtp.h);
    algo ALGO_FRAME computes it in each edge's frame (edge vectors); ALGO_ATOMIC walks
    receivers and adds dx with atomics (dx not bitwise reproducible)."""
    n, e, c = _shapes(x, y_or_vec, w, graph, lmax, y_mode, variant)
    _want(grad_out, "grad_out", (n, out_dim(lmax, variant), c), device=x.device)
    send_ptr, send_perm, send_recv = graph.transpose
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w) if dw is None else dw
    dy = torch.empty_like(y_or_vec) if dy is None else dy
    _want(dx, "dx", x.shape, device=x.device)
    _want(dw, "dw", w.shape, device=x.device)
    _want(dy, "dy", y_or_vec.shape, device=x.device)
    prob = _problem(n, e, c, lmax, y_mode, algo, variant)
    check(lib().conv_tp_bwd(ctypes.byref(prob), _p(grad_out), _p(x), _p(y_or_vec), _p(w),
                            _p(graph.row_ptr), _p(graph.senders), _p(send_ptr), _p(send_perm),
                            _p(send_recv), _p(dx), _p(dw), _p(dy), _stream(x)))
    return dx, dw, dy


def conv_tp_bwd_dy(grad_out, x, w, graph: Graph, lmax: int, dy=None, variant: int = SUMMED):
    """dY alone (Y given): the harmonic gradient of conv_tp_bwd without dx and dw."""
    n, e, c = x.shape[0], w.shape[0], x.shape[2]
    l_in, l_sh, _ = degrees(lmax)
    if graph.n_nodes != n or graph.senders.numel() != e:
        raise ValueError("graph does not match x / w")
    _want(x, "x", (n, dim(l_in), c))
    _want(w, "w", (e, len(_layout(degrees(lmax), int(variant))[0]), c), device=x.device)
    _want(grad_out, "grad_out", (n, out_dim(lmax, variant), c), device=x.device)
    dy = torch.empty((e, dim(l_sh)), dtype=torch.float32, device=x.device) if dy is None else dy
    _want(dy, "dy", (e, dim(l_sh)), device=x.device)
    prob = _problem(n, e, c, lmax, Y_GIVEN, ALGO_CSR, variant)
    check(lib().conv_tp_bwd_dy(ctypes.byref(prob), _p(grad_out), _p(x), _p(w), _p(graph.row_ptr),
                               _p(graph.senders), _p(dy), _stream(x)))
    return dy


def conv_tp_bwd_msg_workspace(n_nodes: int, n_edges: int, channels: int, lmax, y_mode: int = Y_GIVEN,
                              variant: int = SUMMED) -> int:
    """Bytes of device workspace conv_tp_bwd_msg needs (E * (l_in+1)^2 * C * 4)."""
    prob = _problem(n_nodes, n_edges, channels, lmax, y_mode, ALGO_CSR, variant)
    out = ctypes.c_int64(0)
    check(lib().conv_tp_bwd_msg_workspace(ctypes.byref(prob), ctypes.byref(out)))
    return out.value


def conv_tp_bwd_msg(grad_out, x, y_or_vec, w, graph: Graph, lmax: int, y_mode: int = Y_GIVEN,
                    dx=None, dw=None, dy=None, variant: int = SUMMED, workspace=None):
    """conv_tp_bwd through an edge-message workspace (receiver-major products,
    then per-sender sums; see include/convtp.h).  workspace: a float32 device
    tensor of at least conv_tp_bwd_msg_workspace bytes, allocated here if None."""
    n, e, c = _shapes(x, y_or_vec, w, graph, lmax, y_mode, variant)
    _want(grad_out, "grad_out", (n, out_dim(lmax, variant), c), device=x.device)
    send_ptr, send_perm, send_recv = graph.transpose
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w) if dw is None else dw
    dy = torch.empty_like(y_or_vec) if dy is None else dy
    _want(dx, "dx", x.shape, device=x.device)
    _want(dw, "dw", w.shape, device=x.device)
    _want(dy, "dy", y_or_vec.shape, device=x.device)
    prob = _problem(n, e, c, lmax, y_mode, ALGO_CSR, variant)
    if workspace is None:
        workspace = torch.empty(max(1, e * dim(degrees(lmax)[0]) * c), dtype=torch.float32, device=x.device)
    if workspace.dtype != torch.float32 or workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 tensor on x's device")
    check(lib().conv_tp_bwd_msg(ctypes.byref(prob), _p(grad_out), _p(x), _p(y_or_vec), _p(w),
                                _p(graph.row_ptr), _p(graph.senders), _p(send_ptr), _p(send_perm),
                                _p(send_recv), _p(dx), _p(dw), _p(dy), _p(workspace),
                                workspace.numel() * 4, _stream(x)))
    return dx, dw, dy


def conv_tp_bwd_msg_noalloc(grad_out, x, y_or_vec, w, graph: Graph, lmax, y_mode: int = Y_GIVEN,
                            dx=None, dw=None, dy=None, variant: int = SUMMED):
    """conv_tp_bwd_msg with the library's fixed per-device scratch instead of a
    workspace (see include/convtp.h; rejects problems whose messages exceed it)."""
    n, e, c = _shapes(x, y_or_vec, w, graph, lmax, y_mode, variant)
    _want(grad_out, "grad_out", (n, out_dim(lmax, variant), c), device=x.device)
    send_ptr, send_perm, send_recv = graph.transpose
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w) if dw is None else dw
    dy = torch.empty_like(y_or_vec) if dy is None else dy
    _want(dx, "dx", x.shape, device=x.device)
    _want(dw, "dw", w.shape, device=x.device)
    _want(dy, "dy", y_or_vec.shape, device=x.device)
    prob = _problem(n, e, c, lmax, y_mode, ALGO_CSR, variant)
    check(lib().conv_tp_bwd_msg_noalloc(ctypes.byref(prob), _p(grad_out), _p(x), _p(y_or_vec), _p(w),
                                        _p(graph.row_ptr), _p(graph.senders), _p(send_ptr), _p(send_perm),
                                        _p(send_recv), _p(dx), _p(dw), _p(dy), _stream(x)))
    return dx, dw, dy


def conv_tp_bwd_bwd(grad_out, x, Y, w, a_x, a_w, a_y, graph: Graph, lmax, out=None, variant: int = SUMMED):
    """VJP of conv_tp_bwd (Y given): gradients (g_x, g_w, g_y, g_grad) of
    <a_x, dx> + <a_w, dw> + <a_y, dY> (see include/convtp.h)."""
    n, e, c = _shapes(x, Y, w, graph, lmax, Y_GIVEN, variant)
    _want(grad_out, "grad_out", (n, out_dim(lmax, variant), c), device=x.device)
    _want(a_x, "a_x", x.shape, device=x.device)
    _want(a_w, "a_w", w.shape, device=x.device)
    _want(a_y, "a_y", Y.shape, device=x.device)
    send_ptr, send_perm, send_recv = graph.transpose
    if out is None:
        out = (torch.empty_like(x), torch.empty_like(w), torch.empty_like(Y), torch.empty_like(grad_out))
    g_x, g_w, g_y, g_grad = out
    for name, t, ref in (("g_x", g_x, x), ("g_w", g_w, w), ("g_y", g_y, Y), ("g_grad", g_grad, grad_out)):
        _want(t, name, ref.shape, device=x.device)
    prob = _problem(n, e, c, lmax, Y_GIVEN, ALGO_CSR, variant)
    check(lib().conv_tp_bwd_bwd(ctypes.byref(prob), _p(grad_out), _p(x), _p(Y), _p(w), _p(a_x), _p(a_w),
                                _p(a_y), _p(graph.row_ptr), _p(graph.senders), _p(send_ptr), _p(send_perm),
                                _p(send_recv), _p(g_x), _p(g_w), _p(g_y), _p(g_grad), _stream(x)))
    return g_x, g_w, g_y, g_grad


def spherical_harmonics(vec, lmax: int, out=None):
    e = vec.shape[0]
    _want(vec, "vec", (e, 3))
    out = torch.empty((e, dim(lmax)), dtype=torch.float32, device=vec.device) if out is None else out
    _want(out, "Y", (e, dim(lmax)), device=vec.device)
    check(lib().conv_tp_sh(e, lmax, _p(vec), _p(out), _stream(vec)))
    return out


def spherical_harmonics_backward(vec, dY, lmax: int, out=None):
    e = vec.shape[0]
    _want(vec, "vec", (e, 3))
    _want(dY, "dY", (e, dim(lmax)), device=vec.device)
    out = torch.empty_like(vec) if out is None else out
    _want(out, "dvec", (e, 3), device=vec.device)
    check(lib().conv_tp_sh_bwd(e, lmax, _p(vec), _p(dY), _p(out), _stream(vec)))
    return out


def _node_problem(n, c, lmax):
    return _capi.NodeProblem(n, c, lmax, lmax, lmax)


def node_tp_fwd(x, y, w, lmax: int, out=None):
    """Node-local channelwise tensor product: out[i] = sum_p w[i,p] (.) C_p(x[i], y[i])."""
    n, d, c = x.shape
    _want(x, "x", (n, dim(lmax), c))
    _want(y, "y", (n, dim(lmax), c), device=x.device)
    _want(w, "w", (n, num_paths(lmax), c), device=x.device)
    out = torch.empty_like(x) if out is None else out
    _want(out, "out", (n, dim(lmax), c), device=x.device)
    prob = _node_problem(n, c, lmax)
    check(lib().conv_tp_node_fwd(ctypes.byref(prob), _p(x), _p(y), _p(w), _p(out), _stream(x)))
    return out


def node_tp_bwd(grad_out, x, y, w, lmax: int, dx=None, dy=None, dw=None):
    """VJP of node_tp_fwd: (dx, dy, dw)."""
    n, d, c = x.shape
    for name, t in (("grad_out", grad_out), ("x", x), ("y", y)):
        _want(t, name, (n, dim(lmax), c), device=x.device)
    _want(w, "w", (n, num_paths(lmax), c), device=x.device)
    dx = torch.empty_like(x) if dx is None else dx
    dy = torch.empty_like(y) if dy is None else dy
    dw = torch.empty_like(w) if dw is None else dw
    for name, t, ref in (("dx", dx, x), ("dy", dy, y), ("dw", dw, w)):
        _want(t, name, tuple(ref.shape), device=x.device)
    prob = _node_problem(n, c, lmax)
    check(lib().conv_tp_node_bwd(ctypes.byref(prob), _p(grad_out), _p(x), _p(y), _p(w), _p(dx), _p(dy), _p(dw),
                                 _stream(x)))
    return dx, dy, dw


STREAM_READ, STREAM_WRITE, STREAM_COPY = 0, 1, 2
STREAM_DWORD = 3   # added to a kind: the same stream with 4-byte accesses per lane


def stream_probe(kind: int, src, dst):
    """HBM stream probe (measurement only): kind STREAM_READ reads src,
    STREAM_WRITE writes dst, STREAM_COPY copies src into dst (16-byte
    accesses per lane; kind + STREAM_DWORD: 4-byte accesses)."""
    t = dst if kind % 3 == STREAM_WRITE else src
    n = t.numel()
    for name, a in (("src", src), ("dst", dst)):
        if a is not None:
            _want(a, name, (a.numel(),), device=t.device)
    check(lib().conv_tp_stream_probe(kind, _p(src), _p(dst), n, _stream(t)))


def valu_probe(iterations: int, sink):
    """fp32 FMA probe (measurement only): launches it on sink's device and
    returns the number of FMAs the launch performs."""
    _want(sink, "sink", (sink.numel(),))
    fmas = ctypes.c_int64(0)
    check(lib().conv_tp_valu_probe(int(iterations), _p(sink), ctypes.byref(fmas), _stream(sink)))
    return int(fmas.value)


def spherical_harmonics_jvp(vec, a_vec, lmax: int, out=None):
    """a_Y = (dY/dvec) a_vec per edge."""
    e = vec.shape[0]
    _want(vec, "vec", (e, 3))
    _want(a_vec, "a_vec", (e, 3), device=vec.device)
    out = torch.empty((e, dim(lmax)), dtype=torch.float32, device=vec.device) if out is None else out
    _want(out, "a_y", (e, dim(lmax)), device=vec.device)
    check(lib().conv_tp_sh_jvp(e, lmax, _p(vec), _p(a_vec), _p(out), _stream(vec)))
    return out


def spherical_harmonics_bwd_bwd(vec, dY, a_vec, g_y, lmax: int, out=None):
    """g_vec = J^T g_y + d/dvec <J a_vec, dY> per edge."""
    e = vec.shape[0]
    _want(vec, "vec", (e, 3))
    for name, t, sh_ in (("dY", dY, (e, dim(lmax))), ("a_vec", a_vec, (e, 3)), ("g_y", g_y, (e, dim(lmax)))):
        _want(t, name, sh_, device=vec.device)
    out = torch.empty_like(vec) if out is None else out
    _want(out, "g_vec", (e, 3), device=vec.device)
    check(lib().conv_tp_sh_bwd_bwd(e, lmax, _p(vec), _p(dY), _p(a_vec), _p(g_y), _p(out), _stream(vec)))
    return out


def conv_tp_bwd_bwd_vec(grad_out, x, vec, w, a_x, a_w, a_vec, graph: Graph, lmax, variant: int = SUMMED,
                        dY=None, out=None, workspace=None):
    """VJP of the edge-vector backward in one library call
    (conv_tp_bwd_bwd_vec, include/convtp.h): (g_x, g_w, g_vec, g_grad) for
    cotangents (a_x, a_w, a_vec) of (dx, dw, dvec).  dY: the first backward's
    harmonic gradient [E][(l_sh+1)^2] if the caller kept it (else the library
    recomputes it).  workspace: a float32 device tensor of at least
    conv_tp_bwd_bwd_vec_workspace bytes, allocated here if None."""
    n, e, c = _shapes(x, vec, w, graph, lmax, VEC_GIVEN, variant)
    _want(grad_out, "grad_out", (n, out_dim(lmax, variant), c), device=x.device)
    _want(a_x, "a_x", x.shape, device=x.device)
    _want(a_w, "a_w", w.shape, device=x.device)
    _want(a_vec, "a_vec", vec.shape, device=x.device)
    if dY is not None:
        _want(dY, "dY", (e, dim(degrees(lmax)[1])), device=x.device)
    send_ptr, send_perm, send_recv = graph.transpose
    if out is None:
        out = (torch.empty_like(x), torch.empty_like(w), torch.empty_like(vec), torch.empty_like(grad_out))
    g_x, g_w, g_vec, g_grad = out
    for name, t, ref in (("g_x", g_x, x), ("g_w", g_w, w), ("g_vec", g_vec, vec), ("g_grad", g_grad, grad_out)):
        _want(t, name, ref.shape, device=x.device)
    prob = _problem(n, e, c, lmax, VEC_GIVEN, ALGO_CSR, variant)
    if workspace is None:
        nbytes = ctypes.c_int64()
        check(lib().conv_tp_bwd_bwd_vec_workspace(ctypes.byref(prob), int(dY is not None), ctypes.byref(nbytes)))
        workspace = torch.empty(max(1, nbytes.value // 4), dtype=torch.float32, device=x.device)
    if workspace.dtype != torch.float32 or workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 tensor on x's device")
    check(lib().conv_tp_bwd_bwd_vec(ctypes.byref(prob), _p(grad_out), _p(x), _p(vec), _p(w), _p(a_x), _p(a_w),
                                    _p(a_vec), _p(dY), _p(graph.row_ptr), _p(graph.senders), _p(send_ptr),
                                    _p(send_perm), _p(send_recv), _p(g_x), _p(g_w), _p(g_vec), _p(g_grad),
                                    _p(workspace), workspace.numel() * 4, _stream(x)))
    return g_x, g_w, g_vec, g_grad


class ConvTPFunction(torch.autograd.Function):
    """Autograd wrapper: forward = conv_tp_fwd (algo 0); backward =
    ConvTPBackward, itself differentiable once more, so that a loss on forces
    (gradients of an energy in the edge vectors) trains w and x through
    torch.autograd.grad(..., create_graph=True)."""

    @staticmethod
    def forward(ctx, x, y_or_vec, w, graph, lmax, y_mode, variant):
        ctx.save_for_backward(x, y_or_vec, w)
        ctx.graph, ctx.lmax, ctx.y_mode, ctx.variant = graph, lmax, y_mode, variant
        return conv_tp_fwd(x, y_or_vec, w, graph, lmax, y_mode, variant=variant)

    @staticmethod
    def backward(ctx, grad_out):
        x, y_or_vec, w = ctx.saved_tensors
        # grad mode is on here only under create_graph: then the second
        # backward follows, and the edge-vector path keeps its harmonic gradient
        dx, dy, dw = ConvTPBackward.apply(grad_out.contiguous(), x, y_or_vec, w, ctx.graph, ctx.lmax,
                                          ctx.y_mode, ctx.variant, torch.is_grad_enabled())
        return dx, dy, dw, None, None, None, None


class ConvTPBackward(torch.autograd.Function):
    """The VJP as a function of (grad_out, x, Y or vec, w), returning
    (dx, dY or dvec, dw): conv_tp_bwd (variant 0) or conv_tp_bwd_msg with a
    workspace from torch's allocator (variant 1, whose grad_out rows are much
    wider than x's).  With edge vectors and keep_dy it runs on Y = harmonics of
    vec and keeps dY, the harmonic gradient, for its own VJP (the VJP of the
    VJP): conv_tp_bwd_bwd, or conv_tp_bwd_bwd_vec for edge vectors."""

    @staticmethod
    def forward(ctx, grad_out, x, y_or_vec, w, graph, lmax, y_mode, variant, keep_dy=False):
        bwd = conv_tp_bwd_msg if variant == SLOTS else conv_tp_bwd
        dY = None
        if y_mode == VEC_GIVEN and keep_dy:
            l_sh = degrees(lmax)[1]
            Y = spherical_harmonics(y_or_vec, l_sh)
            dx, dw, dY = bwd(grad_out, x, Y, w, graph, lmax, Y_GIVEN, variant=variant)
            dy = spherical_harmonics_backward(y_or_vec, dY, l_sh)
        else:
            dx, dw, dy = bwd(grad_out, x, y_or_vec, w, graph, lmax, y_mode, variant=variant)
        ctx.save_for_backward(grad_out, x, y_or_vec, w, dY)
        ctx.graph, ctx.lmax, ctx.y_mode, ctx.variant = graph, lmax, y_mode, variant
        return dx, dy, dw

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, a_x, a_y, a_w):
        G, x, y_or_vec, w, dY = ctx.saved_tensors
        a_x, a_y, a_w = a_x.contiguous(), a_y.contiguous(), a_w.contiguous()
        if ctx.y_mode == Y_GIVEN:
            g_x, g_w, g_y, g_grad = conv_tp_bwd_bwd(G, x, y_or_vec, w, a_x, a_w, a_y, ctx.graph, ctx.lmax,
                                                    variant=ctx.variant)
        else:
            g_x, g_w, g_y, g_grad = conv_tp_bwd_bwd_vec(G, x, y_or_vec, w, a_x, a_w, a_y, ctx.graph, ctx.lmax,
                                                        variant=ctx.variant, dY=dY)
        return g_grad, g_x, g_y, g_w, None, None, None, None, None


def conv_tp(x, y_or_vec, w, graph: Graph, lmax, y_mode: int = Y_GIVEN, variant: int = SUMMED):
    """Differentiable fused convolution tensor product (twice differentiable in
    x, w and Y or vec)."""
    return ConvTPFunction.apply(x, y_or_vec, w, graph, lmax, y_mode, variant)

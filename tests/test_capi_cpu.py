"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, answers path/coupling queries like the oracle, and rejects
every invalid argument on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import cg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def capi():
    from tensor_product_message_amd import _capi
    if not os.path.exists(_capi.LIB_PATH):
        from tensor_product_message_amd.build import build
        build(verbose=False)
    return _capi


def _header_functions():
    src = open(os.path.join(ROOT, "include", "convtp.h")).read()
    return sorted(set(re.findall(r"\b(conv_tp_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(capi):
    L = capi.lib()
    declared = _header_functions()
    assert set(declared) == set(capi.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.conv_tp_version() == 110


def test_paths_match_oracle(capi):
    import tensor_product_message_amd as t
    for L in range(4):
        assert t.num_paths(L) == len(cg.paths(L, L, L))
        assert t.paths(L) == cg.paths(L, L, L)
    assert t.paths(0, 3, 3) == cg.paths(0, 3, 3)


def test_variant_layouts_match_oracle(capi):
    import tensor_product_message_amd as t
    from oracle import convtp as oc
    for L in range(4):
        for v in (0, 1):
            ps, d = t.layout(L, v)
            pr = oc.Problem(L, L, L, variant=v)
            assert ps == pr.paths and d == pr.D3
    L = capi.lib()
    n, d = ctypes.c_int32(0), ctypes.c_int32(0)
    assert L.conv_tp_layout(2, 1, 1, 1, ctypes.byref(n), ctypes.byref(d), None) == capi.CTP_EINVAL
    assert L.conv_tp_layout(1, 4, 4, 4, ctypes.byref(n), ctypes.byref(d), None) == capi.CTP_EUNSUPPORTED
    assert L.conv_tp_layout(1, 1, 1, 1, None, ctypes.byref(d), None) == capi.CTP_EINVAL
    assert _fwd(capi, _prob(capi, variant=3)) == capi.CTP_EINVAL


def test_coupling_tables_match_oracle(capi):
    import tensor_product_message_amd as t
    for p in cg.paths(3, 3, 3):
        np.testing.assert_allclose(t.coupling(*p), cg.real_cg(*p), atol=1e-14, rtol=0)
        # identical structural zeros
        assert np.array_equal(t.coupling(*p) != 0, cg.real_cg(*p) != 0)


def _prob(capi, **kw):
    d = dict(n_nodes=4, n_edges=8, channels=16, l_in=1, l_sh=1, l_out=1, y_mode=0, algo=0)
    d.update(kw)
    return capi.Problem(**d)


A = ctypes.c_void_p(0x10000)          # aligned fake addresses: validation must fail first
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)        # 4-byte aligned only
NUL = ctypes.c_void_p(0)


def _fwd(capi, prob, x=A, y=A, w=A, rp=A, s=A, out=A2):
    return capi.lib().conv_tp_fwd(ctypes.byref(prob) if prob is not None else None, x, y, w, rp, s, out, NUL)


def _bwd(capi, prob, g=A, x=A, y=A, w=A, rp=A, s=A, sp=A, pe=A, sr=A, dx=A2, dw=A2, dy=A2):
    return capi.lib().conv_tp_bwd(ctypes.byref(prob), g, x, y, w, rp, s, sp, pe, sr, dx, dw, dy, NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(n_nodes=-1), 1), (dict(n_edges=-3), 1), (dict(channels=0), 1),
    (dict(channels=1025), 2), (dict(l_in=4, l_sh=4, l_out=4), 2), (dict(l_in=-1), 2),
    (dict(l_sh=4), 2), (dict(l_out=4), 2), (dict(l_in=4), 2), (dict(y_mode=2), 1), (dict(algo=7), 1),
    (dict(n_nodes=0, n_edges=5), 5),
])
def test_fwd_rejects_bad_problem(capi, kw, code):
    assert _fwd(capi, _prob(capi, **kw)) == code
    assert capi.lib().conv_tp_last_error().decode()


def test_fwd_rejects_bad_pointers(capi):
    p = _prob(capi)
    assert _fwd(capi, None) == capi.CTP_EINVAL
    assert _fwd(capi, p, x=NUL) == capi.CTP_EINVAL
    assert _fwd(capi, p, y=NUL) == capi.CTP_EINVAL
    assert _fwd(capi, p, w=NUL) == capi.CTP_EINVAL
    assert _fwd(capi, p, rp=NUL) == capi.CTP_EINVAL
    assert _fwd(capi, p, s=NUL) == capi.CTP_EINVAL
    assert _fwd(capi, p, out=NUL) == capi.CTP_EINVAL
    assert _fwd(capi, p, x=MIS) == capi.CTP_EALIGN
    assert _fwd(capi, p, w=MIS) == capi.CTP_EALIGN
    assert _fwd(capi, p, out=MIS) == capi.CTP_EALIGN
    assert _fwd(capi, p, rp=ctypes.c_void_p(0x10002)) == capi.CTP_EALIGN
    assert "aligned" in capi.lib().conv_tp_last_error().decode()


def test_frame_forward_rejections(capi):
    # the edge-frame forward (algo 2) needs edge vectors and the summed variant
    assert _fwd(capi, _prob(capi, algo=2, y_mode=0)) == capi.CTP_EUNSUPPORTED
    assert _fwd(capi, _prob(capi, algo=2, y_mode=1, variant=1)) == capi.CTP_EUNSUPPORTED
    assert "edge frame" in capi.lib().conv_tp_last_error().decode()
    assert _fwd(capi, _prob(capi, algo=3, y_mode=1)) == capi.CTP_EINVAL
    assert _fwd(capi, _prob(capi, algo=2, y_mode=1), x=NUL) == capi.CTP_EINVAL
    # the edge-frame backward (algo 2) likewise; the message backwards have no frame form
    assert _bwd(capi, _prob(capi, algo=2, y_mode=0)) == capi.CTP_EUNSUPPORTED
    assert _bwd(capi, _prob(capi, algo=2, y_mode=1, variant=1)) == capi.CTP_EUNSUPPORTED
    assert _bwd(capi, _empty(capi, algo=2, y_mode=1), g=NUL, x=NUL, y=NUL, w=NUL, s=NUL, pe=NUL, sr=NUL,
                dx=NUL, dw=NUL, dy=NUL) == capi.CTP_OK
    assert _bwd_msg(capi, _prob(capi, algo=2, y_mode=1)) == capi.CTP_EUNSUPPORTED
    assert capi.lib().conv_tp_bwd_msg_noalloc(ctypes.byref(_prob(capi, algo=2, y_mode=1)), *([A] * 9),
                                              A2, A2, A2, NUL) == capi.CTP_EUNSUPPORTED


def _empty(capi, **kw):
    # N = E = 0: validation runs in full, then nothing is launched (safe without a GPU)
    return _prob(capi, n_nodes=0, n_edges=0, **kw)


@pytest.mark.parametrize("deg", [(0, 3, 3), (1, 3, 2), (3, 2, 1), (2, 2, 2), (0, 0, 3), (3, 0, 0)])
@pytest.mark.parametrize("channels", [1, 513, 1024])
def test_every_degree_triple_and_channel_count_is_accepted(capi, deg, channels):
    a, b, c = deg
    for variant in (0, 1):
        for y_mode in (0, 1):
            p = _empty(capi, channels=channels, l_in=a, l_sh=b, l_out=c, y_mode=y_mode, variant=variant)
            assert _fwd(capi, p, x=NUL, y=NUL, w=NUL, s=NUL, out=NUL) == capi.CTP_OK
            assert _bwd(capi, p, g=NUL, x=NUL, y=NUL, w=NUL, s=NUL, pe=NUL, sr=NUL, dx=NUL, dw=NUL,
                        dy=NUL) == capi.CTP_OK, capi.lib().conv_tp_last_error()
            assert _bwd_msg(capi, p, ws=NUL, nbytes=0, g=NUL, x=NUL, y=NUL, w=NUL, s=NUL, pe=NUL, sr=NUL,
                            dx=NUL, dw=NUL, dy=NUL) == capi.CTP_OK
        p = _empty(capi, channels=channels, l_in=a, l_sh=b, l_out=c, variant=variant)
        dd = [NUL] * 16
        dd[7] = dd[9] = A
        assert _bwd_bwd(capi, p, dd) == capi.CTP_OK
        assert capi.lib().conv_tp_bwd_dy(ctypes.byref(p), NUL, NUL, NUL, A, NUL, NUL, NUL) == capi.CTP_OK


def test_bwd_rejections(capi):
    assert _bwd(capi, _prob(capi, channels=1025)) == capi.CTP_EUNSUPPORTED
    assert _bwd(capi, _prob(capi, algo=1, channels=1025)) == capi.CTP_EUNSUPPORTED
    assert _bwd(capi, _prob(capi, algo=3)) == capi.CTP_EINVAL
    for algo in (0, 1):
        p = _prob(capi, algo=algo)
        for k in ("g", "x", "y", "w", "rp", "s", "sp", "pe", "sr", "dx", "dw", "dy"):
            assert _bwd(capi, p, **{k: NUL}) == capi.CTP_EINVAL, (algo, k)
    p = _prob(capi)
    assert _bwd(capi, p, dw=MIS) == capi.CTP_EALIGN
    assert _bwd(capi, p, g=MIS) == capi.CTP_EALIGN


def _bwd_msg(capi, prob, ws=A2, nbytes=1 << 40, **kw):
    a = dict(g=A, x=A, y=A, w=A, rp=A, s=A, sp=A, pe=A, sr=A, dx=A2, dw=A2, dy=A2)
    a.update(kw)
    return capi.lib().conv_tp_bwd_msg(ctypes.byref(prob), *a.values(), ws, nbytes, NUL)


def test_bwd_msg_rejections(capi):
    L = capi.lib()
    nb = ctypes.c_int64(-1)
    p = _prob(capi, n_nodes=4, n_edges=8, channels=16, l_in=2, l_sh=2, l_out=2)
    assert L.conv_tp_bwd_msg_workspace(ctypes.byref(p), ctypes.byref(nb)) == capi.CTP_OK
    assert nb.value == 8 * 9 * 16 * 4
    assert L.conv_tp_bwd_msg_workspace(ctypes.byref(p), None) == capi.CTP_EINVAL
    assert L.conv_tp_bwd_msg_workspace(ctypes.byref(_prob(capi, variant=3)), ctypes.byref(nb)) == capi.CTP_EINVAL
    assert len(L.conv_tp_bwd_msg.argtypes) == 16   # problem, 12 arrays, workspace, its size, stream
    assert _bwd_msg(capi, _prob(capi, algo=1)) == capi.CTP_EUNSUPPORTED
    assert _bwd_msg(capi, _prob(capi, channels=1025)) == capi.CTP_EUNSUPPORTED
    for k in ("g", "x", "y", "w", "rp", "s", "sp", "pe", "sr", "dx", "dw", "dy"):
        assert _bwd_msg(capi, p, **{k: NUL}) == capi.CTP_EINVAL, k
    assert _bwd_msg(capi, p, nbytes=nb.value - 4) == capi.CTP_EINVAL
    assert "workspace" in L.conv_tp_last_error().decode()
    assert _bwd_msg(capi, p, ws=NUL, nbytes=nb.value) == capi.CTP_EINVAL
    assert _bwd_msg(capi, p, ws=MIS, nbytes=nb.value) == capi.CTP_EALIGN


def test_bwd_msg_noalloc_rejections(capi):
    # same argument checks as conv_tp_bwd_msg, then a size check against the
    # fixed scratch, all before any HIP call
    L = capi.lib()
    f = lambda p, **kw: L.conv_tp_bwd_msg_noalloc(ctypes.byref(p), *dict(  # noqa: E731
        dict(g=A, x=A, y=A, w=A, rp=A, s=A, sp=A, pe=A, sr=A, dx=A2, dw=A2, dy=A2), **kw).values(), NUL)
    assert len(L.conv_tp_bwd_msg_noalloc.argtypes) == 14
    assert f(_prob(capi, algo=1)) == capi.CTP_EUNSUPPORTED
    assert f(_prob(capi, channels=1025)) == capi.CTP_EUNSUPPORTED
    for k in ("g", "x", "y", "w", "rp", "s", "sp", "pe", "sr", "dx", "dw", "dy"):
        assert f(_prob(capi), **{k: NUL}) == capi.CTP_EINVAL, k
    # E * (l_in+1)^2 * C * 4 = 32769 * 16 * 128 * 4 > 256 MiB
    big = _prob(capi, n_nodes=100, n_edges=32769, channels=128, l_in=3, l_sh=3, l_out=3)
    assert f(big) == capi.CTP_EUNSUPPORTED
    assert "scratch" in L.conv_tp_last_error().decode()
    assert f(_empty(capi, channels=1024, l_in=3, l_sh=3, l_out=3), g=NUL, x=NUL, y=NUL, w=NUL, s=NUL, pe=NUL,
             sr=NUL, dx=NUL, dw=NUL, dy=NUL) == capi.CTP_OK


def test_bwd_dy_rejections(capi):
    L = capi.lib()
    f = lambda p, a: L.conv_tp_bwd_dy(ctypes.byref(p), *a, NUL)  # noqa: E731
    args = [A, A, A, A, A, A2]          # grad_out, x, w, row_ptr, senders, dy
    assert len(L.conv_tp_bwd_dy.argtypes) == 8
    assert f(_prob(capi, y_mode=1), args) == capi.CTP_EUNSUPPORTED
    assert f(_prob(capi, algo=1), args) == capi.CTP_EUNSUPPORTED
    assert f(_prob(capi, channels=1025), args) == capi.CTP_EUNSUPPORTED
    for k in range(6):
        a = list(args)
        a[k] = NUL
        assert f(_prob(capi), a) == capi.CTP_EINVAL, k
    a = list(args)
    a[1] = MIS
    assert f(_prob(capi), a) == capi.CTP_EALIGN


def test_node_entry_points_validate(capi):
    L = capi.lib()
    nb = lambda **kw: capi.NodeProblem(**{**dict(n_nodes=4, channels=16, l_x=2, l_y=2, l_out=2), **kw})  # noqa: E731
    fwd = lambda p, x=A, y=A, w=A, o=A2: L.conv_tp_node_fwd(ctypes.byref(p), x, y, w, o, NUL)  # noqa: E731
    assert L.conv_tp_node_fwd(None, A, A, A, A2, NUL) == capi.CTP_EINVAL
    assert fwd(nb(n_nodes=-1)) == capi.CTP_EINVAL
    assert fwd(nb(channels=0)) == capi.CTP_EINVAL
    assert fwd(nb(channels=(1 << 20) + 1)) == capi.CTP_EUNSUPPORTED
    assert fwd(nb(l_x=4, l_y=4, l_out=4)) == capi.CTP_EUNSUPPORTED
    assert fwd(nb(l_y=1)) == capi.CTP_EUNSUPPORTED
    for k in ("x", "y", "w", "o"):
        assert fwd(nb(), **{k: NUL}) == capi.CTP_EINVAL, k
    assert fwd(nb(), y=MIS) == capi.CTP_EALIGN
    assert fwd(nb(n_nodes=0), x=NUL, y=NUL, w=NUL, o=NUL) == capi.CTP_OK
    p = nb()
    args = [A, A, A, A, A2, A2, A2]
    for i in range(7):
        a = list(args)
        a[i] = NUL
        assert L.conv_tp_node_bwd(ctypes.byref(p), *a, NUL) == capi.CTP_EINVAL, i
    a = list(args)
    a[6] = MIS
    assert L.conv_tp_node_bwd(ctypes.byref(p), *a, NUL) == capi.CTP_EALIGN


def _bwd_bwd(capi, prob, args):
    return capi.lib().conv_tp_bwd_bwd(ctypes.byref(prob), *args, NUL)


def test_bwd_bwd_rejections(capi):
    args = [A] * 12 + [A2] * 4      # 12 inputs (grad_out .. send_recv), 4 outputs
    assert _bwd_bwd(capi, _prob(capi, y_mode=1), args) == capi.CTP_EUNSUPPORTED
    assert _bwd_bwd(capi, _prob(capi, algo=1), args) == capi.CTP_EUNSUPPORTED
    assert _bwd_bwd(capi, _prob(capi, channels=1025), args) == capi.CTP_EUNSUPPORTED
    assert len(args) == len(capi.lib().conv_tp_bwd_bwd.argtypes) - 2
    for k in range(16):
        a = list(args)
        a[k] = NUL
        assert _bwd_bwd(capi, _prob(capi), a) == capi.CTP_EINVAL, k
    a = list(args)
    a[5] = MIS          # a_w
    assert _bwd_bwd(capi, _prob(capi), a) == capi.CTP_EALIGN
    a = [NUL] * 16
    a[7] = a[9] = A     # empty graph: only row_ptr and send_ptr (N+1 = 1 entry); nothing is launched
    assert _bwd_bwd(capi, _prob(capi, n_nodes=0, n_edges=0), a) == capi.CTP_OK


def _bwd_bwd_vec(capi, prob, args, ws_bytes):
    return capi.lib().conv_tp_bwd_bwd_vec(ctypes.byref(prob), *args, ws_bytes, NUL)


def test_bwd_bwd_vec_rejections_and_workspace(capi):
    L = capi.lib()
    nb = ctypes.c_int64(-1)
    p = _prob(capi, y_mode=1, l_sh=2)   # E = 8, D_sh = 9
    assert L.conv_tp_bwd_bwd_vec_workspace(ctypes.byref(p), 1, ctypes.byref(nb)) == capi.CTP_OK
    assert nb.value == 3 * 8 * 9 * 4
    assert L.conv_tp_bwd_bwd_vec_workspace(ctypes.byref(p), 0, ctypes.byref(nb)) == capi.CTP_OK
    assert nb.value == 4 * 8 * 9 * 4
    assert L.conv_tp_bwd_bwd_vec_workspace(ctypes.byref(p), 0, None) == capi.CTP_EINVAL
    # grad_out x vec w a_x a_w a_vec dY row_ptr senders send_ptr send_perm send_recv | 4 outputs | workspace
    args = [A] * 13 + [A2] * 4 + [A]
    big = 1 << 20
    assert len(args) + 3 == len(L.conv_tp_bwd_bwd_vec.argtypes)
    assert _bwd_bwd_vec(capi, _prob(capi, y_mode=0), args, big) == capi.CTP_EUNSUPPORTED
    assert _bwd_bwd_vec(capi, _prob(capi, y_mode=1, algo=2), args, big) == capi.CTP_EUNSUPPORTED
    assert _bwd_bwd_vec(capi, _prob(capi, y_mode=1, channels=1025), args, big) == capi.CTP_EUNSUPPORTED
    for k in range(18):
        if k == 7:
            continue    # dY is optional
        a = list(args)
        a[k] = NUL
        assert _bwd_bwd_vec(capi, p, a, big) == capi.CTP_EINVAL, k
    assert _bwd_bwd_vec(capi, p, args, 3 * 8 * 9 * 4 - 4) == capi.CTP_EINVAL       # dY given: 3 arrays
    a = list(args)
    a[7] = NUL
    assert _bwd_bwd_vec(capi, p, a, 3 * 8 * 9 * 4) == capi.CTP_EINVAL              # dY computed: 4 arrays
    a = list(args)
    a[17] = MIS
    assert _bwd_bwd_vec(capi, p, a, big) == capi.CTP_EALIGN
    a = [NUL] * 18
    a[8] = a[10] = A    # empty graph: only row_ptr and send_ptr; nothing is launched
    assert _bwd_bwd_vec(capi, _prob(capi, y_mode=1, n_nodes=0, n_edges=0), a, 0) == capi.CTP_OK


def test_empty_arrays_may_be_null(capi):
    # N = 0, E = 0: only row_ptr (one element) is required; the call then
    # succeeds without any kernel, so it is safe without a GPU only if it
    # returns before touching the device -- it does: nothing to launch.
    L = capi.lib()
    p = _prob(capi, n_nodes=0, n_edges=0)
    assert _fwd(capi, p, x=NUL, y=NUL, w=NUL, s=NUL, out=NUL) == capi.CTP_OK
    assert _fwd(capi, p, rp=NUL) == capi.CTP_EINVAL
    assert L.conv_tp_sh(0, 2, NUL, NUL, NUL) == capi.CTP_OK


def test_other_entry_points_validate(capi):
    L = capi.lib()
    assert L.conv_tp_num_paths(4, 1, 1) == -1
    assert L.conv_tp_num_paths(2, 2, 2) == 15 and L.conv_tp_last_error().decode() == ""
    assert L.conv_tp_paths(1, 1, 1, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_coupling(0, 1, 2, A) == capi.CTP_EINVAL
    assert L.conv_tp_coupling(4, 1, 3, A) == capi.CTP_EUNSUPPORTED
    assert L.conv_tp_sh(-1, 2, A, A, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_sh(5, 4, A, A, NUL) == capi.CTP_EUNSUPPORTED
    assert L.conv_tp_sh(5, 2, NUL, A, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_sh_bwd(5, 2, A, A, NUL, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_sh_jvp(5, 2, A, NUL, A2, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_sh_jvp(5, 4, A, A, A2, NUL) == capi.CTP_EUNSUPPORTED
    assert L.conv_tp_sh_jvp(-5, 2, A, A, A2, NUL) == capi.CTP_EINVAL
    for k in range(5):
        a = [A, A, A, A, A2]
        a[k] = NUL
        assert L.conv_tp_sh_bwd_bwd(5, 2, *a, NUL) == capi.CTP_EINVAL, k
    assert L.conv_tp_sh_bwd_bwd(0, 3, NUL, NUL, NUL, NUL, NUL, NUL) == capi.CTP_OK
    assert L.conv_tp_build_transpose(-1, 0, A, A, A, A, A, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_build_transpose(0, 3, A, A, A, A, A, NUL) == capi.CTP_EGRAPH
    assert L.conv_tp_build_transpose(4, 3, A, A, NUL, A, A, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_build_transpose(4, 3, A, MIS, A, A, ctypes.c_void_p(0x10001), NUL) == capi.CTP_EALIGN
    assert L.conv_tp_check_graph(4, 3, A, A, None, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_check_graph(4, -3, A, A, None, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_stream_probe(6, A, A2, 16, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_stream_probe(-1, A, A2, 16, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_stream_probe(5, NUL, A2, 16, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_stream_probe(4, NUL, MIS, 16, NUL) == capi.CTP_EALIGN
    assert L.conv_tp_stream_probe(3, A, A2, 0, NUL) == capi.CTP_OK
    assert L.conv_tp_stream_probe(2, A, A2, 18, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_stream_probe(2, NUL, A2, 16, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_stream_probe(1, NUL, NUL, 16, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_stream_probe(0, MIS, A2, 16, NUL) == capi.CTP_EALIGN
    assert L.conv_tp_stream_probe(2, A, A2, 0, NUL) == capi.CTP_OK
    fm = ctypes.c_int64(-1)
    assert L.conv_tp_valu_probe(-1, A, ctypes.byref(fm), NUL) == capi.CTP_EINVAL
    assert L.conv_tp_valu_probe(5, A, None, NUL) == capi.CTP_EINVAL
    assert L.conv_tp_valu_probe(5, NUL, ctypes.byref(fm), NUL) == capi.CTP_EINVAL
    assert L.conv_tp_valu_probe(0, A, ctypes.byref(fm), NUL) == capi.CTP_OK and fm.value == 0


def test_header_is_plain_c99(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "convtp.h"\nint f(void) { return CTP_OK + (int)sizeof(conv_tp_problem); }\n')
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_consumer_builds_and_reports_bad_input(capi, tmp_path):
    """The C99 consumer of the ABI compiles warning-free (built here into a
    temporary directory) and fails cleanly, before any device work, on input
    it cannot read."""
    exe = tmp_path / "roundtrip"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib_dir = os.path.dirname(capi.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
                        os.path.join(ROOT, "tests", "c_abi", "roundtrip.c"), "-o", str(exe),
                        "-L", lib_dir, "-lconvtp", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                        "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + os.path.join(rocm, "lib")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe), str(tmp_path / "missing.bin"), str(tmp_path / "o.bin")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "cannot open input" in r.stderr


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from tensor_product_message_amd import _capi
    monkeypatch.setattr(_capi, "_lib", None)
    monkeypatch.setattr(_capi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _capi.lib()

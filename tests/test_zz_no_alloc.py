"""The allocation-free message backward (conv_tp_bwd_msg_noalloc) against
conv_tp_bwd_msg with a caller workspace, through the C ABI.

The two share their kernels; only the workspace differs (the library's fixed
per-device scratch here), so the outputs are compared both to the parity bar
(max |a - b| <= 1e-4 * max |b|) and bitwise.  Two calls in a row, the second
on a smaller problem, check that the scratch's previous contents do not leak
into a result.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import convtp as oc
from oracle import sh as osh
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_product_message_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch.device("cuda:0")


def _case(ctp, dev, deg, n, c, variant, y_mode, seed):
    prob = oc.Problem(*deg, variant=variant)
    d = gen.poisson_degrees(n, c, deg[0], deg[1], prob.P, prob.D3, mean_deg=10.0, seed=seed)
    Y = osh.real_sh(deg[1], d["vec"].astype(np.float64)).astype(np.float32)
    t = lambda a: torch.as_tensor(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    g = ctp.Graph(n, t(d["row_ptr"]), t(d["senders"]))
    return g, t(d["grad_out"]), t(d["x"]), t(Y if y_mode == 0 else d["vec"]), t(d["w"])


def _noalloc_via_c_abi(ctp, G, x, yv, w, g, deg, y_mode, variant):
    from tensor_product_message_amd import _capi
    n, e, c = x.shape[0], w.shape[0], x.shape[2]
    prob = _capi.Problem(n, e, c, *deg, y_mode, 0, variant)
    sp, pe, sr = g.transpose
    dx, dw, dy = torch.full_like(x, np.nan), torch.full_like(w, np.nan), torch.full_like(yv, np.nan)
    p = lambda t: ctypes.c_void_p(t.data_ptr() if t.numel() else 0)  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)
    rc = _capi.lib().conv_tp_bwd_msg_noalloc(ctypes.byref(prob), p(G), p(x), p(yv), p(w), p(g.row_ptr),
                                             p(g.senders), p(sp), p(pe), p(sr), p(dx), p(dw), p(dy), st)
    assert rc == 0, _capi.lib().conv_tp_last_error().decode()
    return dx, dw, dy


def _agree(name, got, ref):
    got, ref = got.double().cpu().numpy(), ref.double().cpu().numpy()
    assert np.isfinite(got).all(), name
    scale = float(np.abs(ref).max())
    assert float(np.abs(got - ref).max()) <= 1e-4 * scale, name
    assert np.array_equal(got, ref), f"{name}: not bitwise equal to conv_tp_bwd_msg"


@pytest.mark.parametrize("variant,y_mode", [(1, 0), (0, 1)])
def test_noalloc_matches_workspace_backward_twice(dev, variant, y_mode):
    import tensor_product_message_amd as ctp
    cases = [((3, 3, 3), 400, 128, 7), ((1, 2, 2), 90, 64, 8)]   # the second call is smaller
    for deg, n, c, seed in cases:
        print(f"[noalloc] deg={deg} n={n} c={c} variant={variant} y_mode={y_mode}", flush=True)
        g, G, x, yv, w = _case(ctp, dev, deg, n, c, variant, y_mode, seed)
        got = _noalloc_via_c_abi(ctp, G, x, yv, w, g, deg, y_mode, variant)
        ref = ctp.conv_tp_bwd_msg(G, x, yv, w, g, deg, y_mode, variant=variant)
        torch.cuda.synchronize()
        for name, a, b in zip(("dx", "dw", "dy"), got, ref):
            _agree(name, a, b)

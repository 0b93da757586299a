"""The library driven from plain C: tests/c_abi/roundtrip (a C99 program
built by the repository build entry point or `python tests/c_abi/build.py`) allocates
device memory with the HIP runtime, builds the transpose and runs the
forward and a backward (each algorithm) through include/convtp.h; its outputs
are compared with the oracle (transpose arrays bit-exact)."""
import os
import subprocess

import numpy as np
import pytest

from oracle import convtp as oc
from oracle import graph as og
from oracle import sh as osh
from workloads import gen

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "roundtrip")


def _close(name, got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.abs(got.astype(np.float64) - ref).max())
    scale = float(np.abs(ref).max())
    assert scale > 0.0 and err <= 1e-4 * scale, f"{name}: max err {err:.3e} vs scale {scale:.3e}"


@pytest.mark.parametrize("L,c,variant,y_mode,use_msg,algo", [
    (2, 48, 0, 0, 0, 0), (3, 128, 0, 1, 0, 0), (3, 96, 1, 0, 1, 0), (1, 16, 1, 1, 0, 0), (2, 70, 0, 0, 1, 0),
    (3, 128, 0, 1, 0, 2),      # edge frame, forward and backward
    (3, 96, 1, 0, 0, 1),       # atomics: edge-parallel forward, receiver-major backward
])
def test_c_program_roundtrip(tmp_path, L, c, variant, y_mode, use_msg, algo):
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: build it with `python tests/c_abi/build.py`")
    d = gen.poisson_small(70, c, L, mean_deg=9.0, seed=L + c)
    pr = oc.Problem(L, L, L, variant=variant)
    rng = np.random.default_rng(c)
    n, e = d["n_nodes"], d["n_edges"]
    w = rng.standard_normal((e, pr.P, c)).astype(np.float32)
    G = rng.standard_normal((n, pr.D3, c)).astype(np.float32)
    vec = d["vec"].astype(np.float32)
    Y = osh.real_sh(L, vec.astype(np.float64)).astype(np.float32)
    yin = Y if y_mode == 0 else vec
    head = np.array([n, e, c, L, y_mode, variant, use_msg, algo], dtype=np.int32)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for a in (head, d["x"].astype(np.float32), yin, w, G, d["row_ptr"].astype(np.int32),
                  d["senders"].astype(np.int32)):
            f.write(np.ascontiguousarray(a).tobytes())
    print(f"roundtrip L={L} c={c} variant={variant} y_mode={y_mode} msg={use_msg} algo={algo}", flush=True)
    r = subprocess.run([BIN, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(dst, dtype=np.uint8)
    sizes = [(np.float32, n * pr.D3 * c), (np.float32, n * pr.D1 * c), (np.float32, e * pr.P * c),
             (np.float32, e * yin.shape[1]), (np.int32, n + 1), (np.int32, e), (np.int32, e)]
    parts, off = [], 0
    for dt, k in sizes:
        parts.append(raw[off:off + 4 * k].view(dt))
        off += 4 * k
    assert off == raw.size
    out, dx, dw, dy, sp, pe, sr = parts
    Yref = Y.astype(np.float64) if y_mode == 0 else osh.real_sh(L, vec.astype(np.float64))
    rp, s = d["row_ptr"], d["senders"]
    sp0, pe0, sr0 = og.transpose(n, rp, s)
    assert np.array_equal(sp, sp0) and np.array_equal(pe, pe0) and np.array_equal(sr, sr0)
    _close("out", out.reshape(n, pr.D3, c), oc.fwd(pr, d["x"], Yref, w, rp, s))
    _close("dx", dx.reshape(n, pr.D1, c), oc.bwd_dx(pr, Yref, w, G, sp0, pe0, sr0))
    dw_ref, dY_ref = oc.bwd_edges(pr, d["x"], Yref, w, G, rp, s)
    _close("dw", dw.reshape(e, pr.P, c), dw_ref)
    if y_mode == 0:
        _close("dY", dy.reshape(e, pr.D2), dY_ref)
    else:
        _close("dvec", dy.reshape(e, 3), osh.vec_grad_from_sh_grad(L, vec.astype(np.float64), dY_ref))

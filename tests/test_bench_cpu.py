"""Host-side logic of bench.py (no GPU): the byte model and FMA counts behind
the reported GB/s and roofline figures, the traffic-record lookup, and the
one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.fixture(scope="module")
def ctp():
    from tensor_product_message_amd import _capi
    if not os.path.exists(_capi.LIB_PATH):
        from tensor_product_message_amd.build import build
        build(verbose=False)
    import tensor_product_message_amd as t
    return t


def test_byte_model_at_the_lmax3_step():
    # N=16384, E=737,156, C=128, D=16, P=34, Y given: each array once
    shp = (16384, 737156, 128, 16, 16, 16, 34, 16)
    assert bench.fwd_bytes(*shp) == 13151039252
    assert bench.bwd_bytes(*shp) == 26167795236
    # per edge at C=128 the edge streams dominate: w (and dw) are P*C*4 bytes
    assert bench.fwd_bytes(*shp) / shp[1] == pytest.approx(17840, abs=1)


def test_fma_counts(ctp):
    assert bench.fma_per_edge_channel(ctp, 3) == (665, 1876)
    assert bench.fma_per_edge_channel(ctp, 2)[0] == 170
    assert bench.fma_per_edge_channel(ctp, 3, ctp.SLOTS) == (386, 1400)
    assert bench.node_fma_per_node_channel(ctp, 3) == (1023, 3069)
    assert bench.dd_fma_per_edge_channel(ctp, 3) == 5302


def test_traffic_records_follow_the_sources(tmp_path, monkeypatch):
    for wl, kern in (("l3fb", "bwd"), ("l3fb", "fwd"), ("l3mace", "bwd"), ("l3dd", "dd"), ("node3", "bwd")):
        path = os.path.join(ROOT, "profiles", f"traffic_{wl}_{kern}.json")
        rec = json.load(open(path))
        got = bench.committed_traffic(wl, kern)
        if rec["source_sha"] == bench.kernel_sources_sha(wl):
            assert got == rec["bytes_per_launch"] > 0
        else:
            assert got is None
    # a record taken on other sources is not used
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda workload="l3fb": "0" * 16)
    assert bench.committed_traffic("l3fb", "bwd") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

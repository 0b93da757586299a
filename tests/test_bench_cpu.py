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
    for path in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not (path.startswith("traffic_") and path.endswith(".json")):
            continue
        rec = json.load(open(os.path.join(ROOT, "profiles", path)))
        tag, kern = rec.get("tag", rec["workload"]), rec["kernel"]
        assert path == f"traffic_{tag}_{kern}.json"
        got = bench.committed_traffic(tag, kern)
        if rec["source_sha"] == bench.kernel_sources_sha(tag):
            assert got == rec["bytes_per_launch"] > 0
        else:
            assert got is None
    # a record taken on other sources is not used
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda workload="l3fb": "0" * 16)
    assert bench.committed_traffic("l3fb", "bwd") is None


def test_run_tags_keep_modes_apart(tmp_path, monkeypatch):
    import argparse
    A = lambda **kw: argparse.Namespace(**{**dict(workload="l3fb", vec=False, frame=False, bwd="msg",  # noqa: E731
                                                  direct=False), **kw})
    assert bench.run_tag(A()) == "l3fb"
    assert bench.run_tag(A(vec=True)) == "l3fb-vec"
    assert bench.run_tag(A(vec=True, frame=True)) == "l3fb-vec-frame"
    assert bench.run_tag(A(workload="l3mace", bwd="sender")) == "l3mace-sender"
    assert bench.run_tag(A(workload="l3mace", bwd="atomic")) == "l3mace-atomic"
    assert bench.run_tag(A(workload="water")) == bench.run_tag(A(workload="water", frame=True)) == "water"
    assert bench.run_tag(A(workload="water", direct=True)) == "water-direct"
    # a record of the Y-given run is never reported for the edge-vector run
    rec = dict(workload="l3fb", tag="l3fb", kernel="bwd", source_sha=bench.kernel_sources_sha("l3fb"),
               bytes_per_launch=123)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_l3fb_bwd.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda tag="l3fb": rec["source_sha"])
    assert bench.committed_traffic("l3fb", "bwd") == 123
    assert bench.committed_traffic("l3fb-vec", "bwd") is None
    assert bench.committed_traffic("l3fb-vec-frame", "bwd") is None


def test_every_kernel_source_is_hashed():
    csrc = os.path.join(ROOT, "tensor_product_message_amd", "csrc")
    hashed = set(bench.CONV_SOURCES + bench.COMMON_SOURCES)
    for f in os.listdir(csrc):
        if f.startswith(("conv", "device_common", "tables", "kernels")):
            assert f in hashed, f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

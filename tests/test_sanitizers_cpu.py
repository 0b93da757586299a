"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two builds, each exercised by the CPU suites that drive it, in a child
Python process with the sanitizer runtime preloaded:

* the C ABI front (csrc/convtp_api.hip: argument validation, path and
  coupling queries, error reporting), compiled by hipcc with host-only
  sanitizer flags and linked against stubs of the kernel launchers
  (tests/sanitize/launch_stubs.hip), run under tests/test_capi_cpu.py's
  validation tests (every rejection, every accepted-but-empty call);
* the oracle's C edge loop (oracle/convtp_oracle.c, OpenMP), compiled by gcc,
  run under tests/test_oracle_convtp.py.

Any sanitizer report aborts the child (halt_on_error, no recovery), so the
child's exit status is the verdict.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "tensor_product_message_amd", "csrc")

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1:verify_asan_link_order=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    "OMP_NUM_THREADS": "4",
}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
                  + glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"))
    return hits[-1] if hits else None


def _child_pytest(env_extra, preload, args):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    env["LD_PRELOAD"] = ":".join(preload + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + args,
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_c_abi_front_under_asan_and_ubsan(tmp_path):
    runtime = _clang_asan_runtime()
    if runtime is None:
        pytest.skip("clang AddressSanitizer runtime not found under /opt/rocm/llvm")
    # host-only sanitizer flags: each -fsanitize= goes to the host compilation
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++20", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off"]
    api_o, stub_o = str(tmp_path / "api.o"), str(tmp_path / "stubs.o")
    _run([HIPCC, *common, *san, "-c", os.path.join(CSRC, "convtp_api.hip"), "-o", api_o])
    _run([HIPCC, *common, "-c", os.path.join(ROOT, "tests", "sanitize", "launch_stubs.hip"), "-o", stub_o])
    lib = str(tmp_path / "libconvtp_asan.so")
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", lib, api_o, stub_o])
    out = _child_pytest({"CONVTP_LIB": lib}, [runtime], [
        os.path.join("tests", "test_capi_cpu.py"),
        "-k", "rejects or rejections or accepted or validate or empty or exports or paths or layouts or coupling"])
    assert " passed" in out


def test_oracle_c_loop_under_asan_and_ubsan(tmp_path):
    asan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    ubsan = _run(["gcc", "-print-file-name=libubsan.so"]).stdout.strip()
    if not (os.path.isabs(asan) and os.path.exists(asan) and os.path.exists(ubsan)):
        pytest.skip("gcc sanitizer runtimes not found")
    lib = str(tmp_path / "liboracle_asan.so")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", lib,
          os.path.join(ROOT, "oracle", "convtp_oracle.c"), "-lm"])
    out = _child_pytest({"ORACLE_LIB": lib}, [asan, ubsan], [os.path.join("tests", "test_oracle_convtp.py")])
    assert " passed" in out

"""Build the plain-C consumer of the library's C ABI (test infrastructure).

    python tests/c_abi/build.py

gcc, C99, against include/convtp.h and the HIP runtime headers; links the
in-tree libconvtp.so (found at run time relative to the binary).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "roundtrip")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    lib_dir = os.path.join(ROOT, "tensor_product_message_amd")
    tmp = BIN + ".tmp"
    subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror",
                    "-D__HIP_PLATFORM_AMD__",   # selects the AMD runtime in the HIP headers
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(HERE, "roundtrip.c"), "-o", tmp,
                    "-L", lib_dir, "-lconvtp", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath,$ORIGIN/../../tensor_product_message_amd",
                    "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())

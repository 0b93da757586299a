"""ctypes declarations of libconvtp.so (include/convtp.h), nothing else.

Loading fails loudly if the HIP library has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; CONVTP_LIB names another build of the same library (the
# sanitizer test loads an AddressSanitizer build of the C ABI front this way)
LIB_PATH = os.environ.get("CONVTP_LIB") or os.path.join(HERE, "libconvtp.so")

CTP_OK, CTP_EINVAL, CTP_EUNSUPPORTED, CTP_EALIGN, CTP_EHIP, CTP_EGRAPH = range(6)
STATUS_NAMES = {0: "CTP_OK", 1: "CTP_EINVAL", 2: "CTP_EUNSUPPORTED", 3: "CTP_EALIGN",
                4: "CTP_EHIP", 5: "CTP_EGRAPH"}

# Every symbol include/convtp.h declares.
EXPORTS = ("conv_tp_num_paths", "conv_tp_paths", "conv_tp_layout", "conv_tp_coupling", "conv_tp_fwd", "conv_tp_bwd",
           "conv_tp_bwd_msg_workspace", "conv_tp_bwd_msg", "conv_tp_bwd_msg_noalloc", "conv_tp_bwd_dy", "conv_tp_bwd_bwd",
           "conv_tp_bwd_bwd_vec", "conv_tp_bwd_bwd_vec_workspace",
           "conv_tp_sh", "conv_tp_sh_bwd", "conv_tp_build_transpose", "conv_tp_check_graph",
           "conv_tp_sh_jvp", "conv_tp_sh_bwd_bwd", "conv_tp_node_fwd", "conv_tp_node_bwd", "conv_tp_stream_probe", "conv_tp_valu_probe", "conv_tp_last_error",
           "conv_tp_version")


class Problem(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("n_edges", ctypes.c_int32),
                ("channels", ctypes.c_int32), ("l_in", ctypes.c_int32),
                ("l_sh", ctypes.c_int32), ("l_out", ctypes.c_int32),
                ("y_mode", ctypes.c_int32), ("algo", ctypes.c_int32), ("variant", ctypes.c_int32)]


class NodeProblem(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("channels", ctypes.c_int32), ("l_x", ctypes.c_int32),
                ("l_y", ctypes.c_int32), ("l_out", ctypes.c_int32)]


class ConvTPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m tensor_product_message_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)
    pp = ctypes.POINTER(Problem)
    npp = ctypes.POINTER(NodeProblem)
    sig = {
        "conv_tp_num_paths": ([i32, i32, i32], i32),
        "conv_tp_paths": ([i32, i32, i32, vp], i32),
        "conv_tp_coupling": ([i32, i32, i32, vp], i32),
        "conv_tp_layout": ([i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), vp], i32),
        "conv_tp_fwd": ([pp, vp, vp, vp, vp, vp, vp, vp], i32),
        "conv_tp_bwd": ([pp] + [vp] * 13, i32),
        "conv_tp_bwd_msg_workspace": ([pp, i64p], i32),
        "conv_tp_bwd_dy": ([pp] + [vp] * 7, i32),
        "conv_tp_bwd_msg": ([pp] + [vp] * 13 + [ctypes.c_int64, vp], i32),
        "conv_tp_bwd_msg_noalloc": ([pp] + [vp] * 13, i32),
        "conv_tp_bwd_bwd": ([pp] + [vp] * 17, i32),
        "conv_tp_bwd_bwd_vec": ([pp] + [vp] * 18 + [ctypes.c_int64, vp], i32),
        "conv_tp_bwd_bwd_vec_workspace": ([pp, i32, i64p], i32),
        "conv_tp_sh": ([i32, i32, vp, vp, vp], i32),
        "conv_tp_sh_bwd": ([i32, i32, vp, vp, vp, vp], i32),
        "conv_tp_sh_jvp": ([i32, i32, vp, vp, vp, vp], i32),
        "conv_tp_sh_bwd_bwd": ([i32, i32, vp, vp, vp, vp, vp, vp], i32),
        "conv_tp_build_transpose": ([i32, i32, vp, vp, vp, vp, vp, vp], i32),
        "conv_tp_check_graph": ([i32, i32, vp, vp, i64p, vp], i32),
        "conv_tp_stream_probe": ([i32, vp, vp, ctypes.c_int64, vp], i32),
        "conv_tp_valu_probe": ([ctypes.c_int64, vp, i64p, vp], i32),
        "conv_tp_node_fwd": ([npp, vp, vp, vp, vp, vp], i32),
        "conv_tp_node_bwd": ([npp] + [vp] * 8, i32),
        "conv_tp_last_error": ([], ctypes.c_char_p),
        "conv_tp_version": ([], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def check(status: int) -> None:
    if status != CTP_OK:
        raise ConvTPError(status, lib().conv_tp_last_error().decode())

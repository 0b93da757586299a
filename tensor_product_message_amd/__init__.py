"""Fused equivariant convolution tensor product for MI355X (gfx950).

The HIP library libconvtp.so (C ABI in include/convtp.h) does all the work;
`ops` marshals torch tensors into it.  Import fails loudly at first use if the
library has not been built (`python -m tensor_product_message_amd.build`).
"""
from .ops import (SLOTS, SUMMED, layout, out_dim, degrees, ConvTPBackward, ConvTPFunction, ALGO_ATOMIC, ALGO_CSR, ALGO_FRAME, STREAM_COPY, STREAM_DWORD, STREAM_READ, STREAM_WRITE, VEC_GIVEN,  # noqa: F401
                  Y_GIVEN, ConvTPError, Graph, build_transpose, check_graph, conv_tp, conv_tp_bwd, conv_tp_bwd_msg, conv_tp_bwd_msg_noalloc, conv_tp_bwd_msg_workspace, conv_tp_bwd_dy, conv_tp_bwd_bwd,
                  conv_tp_bwd_bwd_vec, spherical_harmonics_jvp, spherical_harmonics_bwd_bwd,
                  conv_tp_fwd, coupling, dim, node_tp_bwd, node_tp_fwd, num_paths, paths,
                  spherical_harmonics,
                  spherical_harmonics_backward, stream_probe, valu_probe)

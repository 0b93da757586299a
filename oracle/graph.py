"""Graph bookkeeping by plain numpy sorts (exact integer results).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The convolution is organised CSR-by-receiver: row_ptr[N+1] and senders[E],
edges stable by receiver (FlashCart, arXiv 2610.06409, receiver-sorted
convolution).  The backward pass accumulates sender gradients per sender, so
it reads the same edges grouped by sender, stable in CSR edge id (FlashCart's
note on sender-ordered edges for deterministic gradients):
send_ptr[N+1], send_perm[E] (CSR edge ids) and send_recv[E] (their receivers).
"""
from __future__ import annotations

import numpy as np


def row_ptr_from_receivers(receivers, n_nodes: int) -> np.ndarray:
    """Exclusive cumulative sum of bincount(receivers)."""
    cnt = np.bincount(np.asarray(receivers, dtype=np.int64), minlength=n_nodes)
    rp = np.zeros(n_nodes + 1, dtype=np.int64)
    rp[1:] = np.cumsum(cnt)
    return rp.astype(np.int32)


def receivers_of(row_ptr) -> np.ndarray:
    rp = np.asarray(row_ptr, dtype=np.int64)
    return np.repeat(np.arange(rp.size - 1, dtype=np.int64), np.diff(rp)).astype(np.int32)


def csr_order(receivers) -> np.ndarray:
    """Edge permutation that sorts an edge list stably by receiver."""
    return np.argsort(np.asarray(receivers), kind="stable")


def transpose(n_nodes: int, row_ptr, senders):
    """(send_ptr, send_perm, send_recv): stable argsort of senders in CSR order."""
    s = np.asarray(senders, dtype=np.int64)
    perm = np.argsort(s, kind="stable")
    send_ptr = row_ptr_from_receivers(s, n_nodes)
    recv = receivers_of(row_ptr)
    return send_ptr, perm.astype(np.int32), recv[perm].astype(np.int32)


def check_graph(n_nodes: int, row_ptr, senders) -> int:
    """Number of defects: row_ptr[0] != 0, decreasing steps, row_ptr[N] != E,
    and senders outside [0, N)."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    s = np.asarray(senders, dtype=np.int64)
    bad = int(rp[0] != 0) + int((np.diff(rp) < 0).sum()) + int(rp[-1] != s.size)
    bad += int(((s < 0) | (s >= n_nodes)).sum())
    return bad

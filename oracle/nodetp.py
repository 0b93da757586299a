"""The node-local channelwise tensor product and its VJP, plain fp64 numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The same couplings as the convolution, applied at each node to two of its
own features instead of a neighbour's feature and an edge harmonic: the
tensor-product operations the e3j paper (arXiv 2609.35099, abstract) measures
against HBM bandwidth, and the node-local products FlashCart (arXiv
2610.06409, section 4) runs beside its edge convolutions.  Reading taken:
both inputs carry the C channels (channelwise, "uvu"), the weights are per
node, path and channel, and all paths with the same l3 are summed into one
output block, exactly as in the convolution:

  out[i, l3 m3, c] = sum_{p = (l1,l2,l3)} w[i,p,c]
                     sum_{m1,m2} C_p[m1][m2][m3] x[i, l1 m1, c] y[i, l2 m2, c]

x[N][D1][C], y[N][D2][C], w[N][P][C], out[N][D3][C]; paths and couplings from
oracle.cg (lexicographic triangle paths, no parity filter).  The backward is
the exact VJP of this trilinear map for upstream gradient G[N][D3][C].
"""
from __future__ import annotations

import numpy as np

from . import cg as _cg


class NodeProblem:
    """Paths and dense coupling blocks for (l1max, l2max, l3max)."""

    def __init__(self, l_in: int, l_sh: int, l_out: int):
        self.paths = _cg.paths(l_in, l_sh, l_out)
        self.P = len(self.paths)
        self.D1, self.D2, self.D3 = _cg.dim(l_in), _cg.dim(l_sh), _cg.dim(l_out)
        self.blocks = [_cg.real_cg(*p) for p in self.paths]


def _blk(l):
    return slice(l * l, (l + 1) * (l + 1))


def fwd(prob: NodeProblem, x, y, w):
    """out[N][D3][C] by the definition, one path at a time (einsum only
    chooses the pairwise contraction order of each path's product)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n, _, c = x.shape
    out = np.zeros((n, prob.D3, c))
    for p, (l1, l2, l3) in enumerate(prob.paths):
        out[:, _blk(l3), :] += w[:, p, None, :] * np.einsum(
            "abk,nac,nbc->nkc", prob.blocks[p], x[:, _blk(l1), :], y[:, _blk(l2), :], optimize=True)
    return out


def bwd(prob: NodeProblem, x, y, w, G):
    """(dx, dy, dw): derivatives of <G, fwd(x, y, w)> with respect to x, y, w."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    dx, dy, dw = np.zeros_like(x), np.zeros_like(y), np.zeros_like(w)
    for p, (l1, l2, l3) in enumerate(prob.paths):
        Cp = prob.blocks[p]
        xs, ys, gs = x[:, _blk(l1), :], y[:, _blk(l2), :], G[:, _blk(l3), :]
        wp = w[:, p, None, :]
        dx[:, _blk(l1), :] += wp * np.einsum("abk,nbc,nkc->nac", Cp, ys, gs, optimize=True)
        dy[:, _blk(l2), :] += wp * np.einsum("abk,nac,nkc->nbc", Cp, xs, gs, optimize=True)
        dw[:, p, :] = np.einsum("abk,nac,nbc,nkc->nc", Cp, xs, ys, gs, optimize=True)
    return dx, dy, dw

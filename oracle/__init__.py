"""fp64 CPU oracle for the fused equivariant convolution tensor product.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or helpers with
the HIP library under `tensor_product_message_amd/`.

What it computes is the plain definition of the operation that the e3j paper
(arXiv 2609.35099, abstract and Table 1 caption) accelerates: for every edge
j -> i, build the message sum_p w_e,p (.) CG_p(x_j, Y(r_ij)) and sum the
messages into the receiver.  e3nn's implementation materialises exactly these
messages; the fused kernels compute the same sum without writing them.  The
backward pass is the exact vector-Jacobian product of that multilinear map
(FlashCart, arXiv 2610.06409, section on symbolic VJPs).

Modules
-------
cg      complex Clebsch-Gordan from Racah's closed form, the real basis, real
        coupling tensors and the path list
sh      real spherical harmonics (Legendre closed form) and their gradient
wigner  real Wigner-D matrices from Wigner's small-d formula (tests only)
convtp  the convolution: numpy materialise-then-scatter definition, and a
        ctypes front to the naive C edge loop in convtp_oracle.c
nodetp  the node-local channelwise tensor product (same couplings, two node
        features, per-node weights) and its VJP, numpy
graph   CSR bookkeeping (row pointers, stable transpose) by numpy sorts

Readings of points the pages leave open (all follow the plainest reading):
paths with the same l3 are summed into one output block; no parity filter;
orthonormal CG and orthonormal Y (no e3nn normalisation constants); odd-parity
real couplings take the imaginary part of the transformed complex CG; the
component order is m = -l..l with l=1 <-> (y, z, x); a zero edge vector has
Y_00 = 1/sqrt(4 pi), every other Y = 0 and zero vector gradient.

Every function here is pinned by the tests in tests/test_oracle_*.py against
values fixed by the mathematics (sympy's exact CG, scipy's spherical
harmonics, quadrature, closed forms, invariants, brute force and finite
differences).  The e3j paper prints no numerical values of the operation
itself, so agreement with e3j's own numbers is parity unpinned.
"""

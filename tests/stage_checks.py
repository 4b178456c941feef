"""Element-by-element checks of the GPU's stage results (h, h_shared, Y, out) against the fp64
oracle's stages, with error bounds derived from the arithmetic. Test infrastructure only.

Bounds
------
u = 2^-24 (binary32 unit roundoff). A GEMM element is a chain of matrix-core instructions,
each adding STEP products of the K dimension (32 for bf16 operands, 4 for fp32) to the fp32
accumulator, in ascending K. A probe of v_mfma_f32_16x16x32_bf16 shows each instruction
aligns its addends (the accumulator and the products) to about 24 bits below the largest of
them: small addends next to a large one lose their low bits, and exact cancellations inside
one instruction are kept. So one instruction errs by at most about one unit 2^-24 * M_s per
addend, M_s the largest addend's magnitude, plus the rounding of its result; with STEP + 1
addends that is below (STEP + 8) u M_s, and M_s <= |A_(s-1)| + B_s, where A_(s-1) is the exact
partial sum before the instruction and B_s the sum of its |products|. The bound of an element
is therefore

    delta = (STEP + 8) u sum_s (|A_(s-1)| + B_s),

computed per element from the exact partial sums.

For h = silu(G) * U (the GPU evaluates silu with the hardware exp2 and reciprocal, good to
about 2 ulp each, and the rounding of -G log2(e) adds |G| u relative), the bound is
    |silu'(G)| |U| dG + |silu(G)| dU + |h| (2 |G| + 24) u   (+ second-order terms),
and the GPU's bf16 h must be the round-to-nearest-even value of the exact h wherever that
rounding is decided inside the bound (`rounding_check`); elsewhere it may be either
neighbour. The fraction of decided elements is reported and required to stay high, so that
a kernel that truncates h, or rounds twice, fails on most elements.

Y is fp32 and unrounded: |Y_gpu - W_down h_gpu| <= delta over K = I.

The combine is a binary32 fma chain in ascending expert order plus the shared output
(oracle.combine_fp32): where the shared output is known exactly, the GPU's out must equal
the oracle's rounding of that chain bit for bit; with a Gaussian shared expert, out must be
the rounding of the exact fp64 combine wherever the rounding is decided inside the bound
of the chain (k + 1 binary32 roundings of the running sum) plus the shared GEMM's bound.
"""
from __future__ import annotations

import numpy as np

import oracle.moe_oracle as orc

U = 2.0 ** -24
STEP = {"bf16": 32, "f32": 4}


def gemm_exact_and_bound(X, W, step):
    """(exact X W^T in fp64, per-element bound of the fp32 matrix-core chain)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    n, K = X.shape
    aX, aW = np.abs(X), np.abs(W)
    A = np.zeros((n, W.shape[0]))
    acc = np.zeros_like(A)
    for s0 in range(0, K, step):
        acc += np.abs(A)
        acc += aX[:, s0:s0 + step] @ aW[:, s0:s0 + step].T
        A += X[:, s0:s0 + step] @ W[:, s0:s0 + step].T
    return A, (step + 8) * U * acc


def _sigmoid(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def hidden_exact_and_bound(xr, w_gu, step):
    """exact h = silu(gate) * up (oracle) and its bound for the GPU's fp32 evaluation."""
    w_gu = orc.as_f64(w_gu)
    inter = w_gu.shape[0] // 2
    xr = orc.as_f64(xr)
    _, dg = gemm_exact_and_bound(xr, w_gu[:inter], step)
    _, du = gemm_exact_and_bound(xr, w_gu[inter:], step)
    g, u, h = orc.expert_hidden(xr, w_gu)
    sg = _sigmoid(g)
    dsilu = np.abs(sg * (1.0 + g * (1.0 - sg))) + 0.5 * dg      # |silu'| over [g - dg, g + dg]
    s = np.abs(g * sg)
    bound = (dsilu * np.abs(u) * dg + (s + 1.1 * dg) * du + dsilu * dg * du
             + np.abs(h) * (2.0 * np.abs(g) + 24.0) * U)
    return h, bound


def rounding_check(gpu, exact, delta, rne=orc.bf16_rne):
    """gpu must be rne(exact) wherever rne(exact - delta) == rne(exact + delta) ("decided"),
    and lie between those two roundings elsewhere. Returns (n, decided, failures)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    lo = rne(exact - delta)
    hi = rne(exact + delta)
    decided = lo == hi
    bad = np.where(decided, gpu != lo, (gpu < lo) | (gpu > hi))
    return int(gpu.size), int(decided.sum()), int(bad.sum())


def abs_check(gpu, exact, delta):
    """|gpu - exact| <= delta elementwise. Returns (n, worst |err| / delta, failures)."""
    err = np.abs(np.asarray(gpu, dtype=np.float64) - exact)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(delta > 0, err / delta, np.where(err > 0, np.inf, 0.0))
    return int(err.size), float(ratio.max(initial=0.0)), int((err > delta).sum())


def chain_exact_and_bound(weights, y, shared=None, shared_bound=None):
    """(exact fp64 combine, bound of the GPU's binary32 chain against it): the chain
    acc = fma(w_j, y_j, acc), then acc + S, rounds each running sum once (u |run| each, taken
    twice for margin); S itself carries the shared GEMM's bound."""
    w = np.asarray(weights, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    run = np.zeros((y.shape[0], y.shape[2]))
    tot = np.zeros_like(run)
    for j in range(w.shape[1]):
        run = run + w[:, j, None] * y[:, j, :]
        tot += np.abs(run)
    if shared is not None:
        run = run + shared
        tot += np.abs(run)
    b = 2.0 * U * tot
    if shared_bound is not None:
        b = b + shared_bound
    return run, b

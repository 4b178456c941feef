"""CPU pins of the GEMM error bound the stage and routing checks use
(tests/stage_checks.gemm_exact_and_bound): binary32 evaluations of a matrix-core chain of
bf16 products must lie inside it, and plausible mistakes (a dropped K step, a bf16
accumulator) must fall outside it."""
import numpy as np
import pytest

from tests import stage_checks as sc


def _bf16(a):
    """Round fp32 values to bf16 (nearest even), returned as fp64."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _operands(seed, n, m, K):
    rng = np.random.default_rng(seed)
    X = _bf16(rng.standard_normal((n, K)) / np.sqrt(K))
    W = _bf16(rng.standard_normal((m, K)) * 0.02)
    return X, W


def _chain_sequential(X, W):
    """Every product (exact in binary32 for bf16 operands) added one at a time in fp32."""
    acc = np.zeros((X.shape[0], W.shape[0]), dtype=np.float32)
    for k in range(X.shape[1]):
        acc = (acc + np.outer(X[:, k], W[:, k]).astype(np.float32)).astype(np.float32)
    return acc.astype(np.float64)


def _chain_per_step(X, W, step):
    """Each step's products summed exactly, then one binary32 rounding of acc + that sum."""
    acc = np.zeros((X.shape[0], W.shape[0]), dtype=np.float64)
    for s0 in range(0, X.shape[1], step):
        part = X[:, s0:s0 + step] @ W[:, s0:s0 + step].T
        acc = (acc + part).astype(np.float32).astype(np.float64)
    return acc


@pytest.mark.parametrize("K", [64, 2048, 16384])
def test_fp32_chains_inside_the_bound(K):
    X, W = _operands(K, 6, 5, K)
    exact, bound = sc.gemm_exact_and_bound(X, W, sc.STEP["bf16"])
    assert np.allclose(exact, X @ W.T, rtol=1e-12, atol=1e-15)
    for got in (_chain_per_step(X, W, sc.STEP["bf16"]), _chain_sequential(X, W)):
        assert np.all(np.abs(got - exact) <= bound)


def test_mistakes_fall_outside_the_bound():
    X, W = _operands(7, 8, 8, 2048)
    exact, bound = sc.gemm_exact_and_bound(X, W, sc.STEP["bf16"])
    dropped = _chain_per_step(X[:, 32:], W[:, 32:], sc.STEP["bf16"])       # one K step lost
    assert np.mean(np.abs(dropped - exact) > bound) > 0.9
    acc = np.zeros_like(exact)                                                # bf16 accumulator
    for s0 in range(0, X.shape[1], 32):
        acc = _bf16(acc + X[:, s0:s0 + 32] @ W[:, s0:s0 + 32].T)
    assert np.mean(np.abs(acc - exact) > bound) > 0.9

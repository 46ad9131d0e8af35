"""Pins for the oracle's batch-reduce GEMM (no GPU).

The single-building-block page defines the kernel in words (a batch of
block products reduced into one output block); the oracle writes that sum
out.  It is checked against numpy's matmul summed over the batch (a library
primitive, a different code path), against the pinned convolution oracle
(a fully-connected layer is a 1x1 convolution on a 1x1 map, and a 1x1
convolution of a whole image is one block product per image row), for
batch splitting (a batch of K-slices equals one product over all of K),
strided views and alpha/beta.
"""
import numpy as np
import pytest

import gen
import oracle


def _rand(seed, shape):
    return gen.uniform(seed, shape, -1.0, 1.0)


@pytest.mark.parametrize("batch,M,N,K", [(1, 5, 7, 3), (3, 4, 6, 5), (4, 17, 9, 33), (2, 1, 1, 1)])
def test_matches_numpy_matmul_sum(batch, M, N, K):
    a = _rand(1400 + M, (batch, M, K))
    b = _rand(1500 + N, (batch, K, N))
    c, bound = oracle.brgemm(a, b)
    want = sum(a[i] @ b[i] for i in range(batch))
    np.testing.assert_allclose(c, want, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(bound, sum(np.abs(a[i]) @ np.abs(b[i]) for i in range(batch)), rtol=1e-13)


def test_fully_connected_is_a_one_by_one_convolution():
    Nb, C, K = 6, 37, 11
    x = _rand(1601, (Nb, C))
    w = _rand(1602, (K, C))
    y, _ = oracle.conv2d_fprop(x.reshape(Nb, C, 1, 1), w.reshape(K, C, 1, 1))
    c, _ = oracle.brgemm(x[None], w.T[None])           # B[c, k] = W[k, c]: a strided view
    np.testing.assert_allclose(c, y.reshape(Nb, K), rtol=1e-13, atol=1e-14)


def test_batch_of_k_slices_equals_one_product():
    M, N, K, parts = 9, 8, 24, 4
    a = _rand(1701, (M, K))
    b = _rand(1702, (K, N))
    whole, _ = oracle.brgemm(a[None], b[None])
    kb = K // parts
    a_parts = np.stack([a[:, i * kb:(i + 1) * kb] for i in range(parts)])
    b_parts = np.stack([b[i * kb:(i + 1) * kb] for i in range(parts)])
    split, _ = oracle.brgemm(a_parts, b_parts)
    np.testing.assert_allclose(split, whole, rtol=1e-14, atol=1e-14)


def test_pointwise_convolution_rows_are_block_products():
    # y[n, k, p, q] = sum_c w[k, c] x[n, c, p, q]: for image n, the (P*Q x K) block is x_n^T @ w^T
    N, C, H, W, K = 2, 5, 3, 4, 6
    x = _rand(1801, (N, C, H, W))
    w = _rand(1802, (K, C))
    y, _ = oracle.conv2d_fprop(x, w.reshape(K, C, 1, 1))
    for n in range(N):
        a = x[n].reshape(C, H * W).T[None]                 # (1, HW, C), a transposed view
        c, _ = oracle.brgemm(a, w.T[None])
        np.testing.assert_allclose(c, y[n].reshape(K, H * W).T, rtol=1e-13, atol=1e-14)


def test_alpha_beta():
    a = _rand(1901, (2, 4, 5))
    b = _rand(1902, (2, 5, 3))
    base, _ = oracle.brgemm(a, b)
    old = _rand(1903, (4, 3))
    c, _ = oracle.brgemm(a, b, alpha=-0.5, beta=2.0, c_old=old)
    np.testing.assert_allclose(c, -0.5 * base + 2.0 * old, rtol=0, atol=1e-15)

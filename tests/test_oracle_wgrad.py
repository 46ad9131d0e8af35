"""Pins for the oracle's filter gradient (backward pass with respect to F).

The pages print no formula; the reading taken is the adjoint of the forward
sum in F.  Each test checks it against something other than itself: the
adjoint identity <conv(x, dF), dy> = <dF, wgrad(x, dy)> with the (already
pinned) forward oracle, the product of dy with an im2col matrix built from
the definition in numpy, an integer closed form for all-ones inputs, a plain
matmul for 1x1 filters, and a shifted copy of dy for a one-hot input.
test_oracle_mutants.py plants slips in the filter-gradient code and checks
that these tests catch them.
"""
import numpy as np
import pytest

import gen
import oracle


def _rand(seed, shape):
    return gen.uniform(seed, shape, -1.0, 1.0)


def _fwd_dims(H, W, R, S, stride, pads):
    pt, pb, pl, pr = pads
    return (H + pt + pb - R) // stride[0] + 1, (W + pl + pr - S) // stride[1] + 1


FUZZ = [
    (2, 3, 7, 6, 4, 3, 2, (2, 1), (1, 0, 0, 1)),
    (1, 2, 9, 9, 3, 3, 3, (1, 1), (1, 1, 1, 1)),
    (2, 4, 8, 11, 5, 5, 3, (3, 2), (2, 1, 0, 2)),
    (3, 1, 5, 5, 2, 1, 1, (2, 2), (0, 0, 0, 0)),
    (1, 5, 12, 7, 3, 4, 4, (1, 3), (3, 0, 2, 1)),
    (2, 2, 6, 10, 6, 2, 5, (2, 1), (0, 1, 4, 0)),
]


@pytest.mark.parametrize("case", FUZZ, ids=[str(i) for i in range(len(FUZZ))])
def test_adjoint_identity(case):
    N, C, H, W, K, R, S, stride, pads = case
    seed = 700 + 7 * FUZZ.index(case)
    x = _rand(seed, (N, C, H, W))
    dF = _rand(seed + 1, (K, C, R, S))
    y, _ = oracle.conv2d_fprop(x, dF, stride, pads)
    dy = _rand(seed + 2, y.shape)
    dw, bound = oracle.conv2d_bwd_filter(x, dy, dF.shape, stride, pads)
    lhs = float(np.sum(y * dy))
    rhs = float(np.sum(dF * dw))
    scale = float(np.sum(np.abs(dF) * bound))
    assert abs(lhs - rhs) <= 1e-13 * max(scale, 1.0), (lhs, rhs)


def _im2col(x, R, S, stride, pads):
    """Xcol[n, (p,q), (c,r,s)] = x[n, c, p*u + r - pt, q*v + s - pl] inside the plane, else 0."""
    N, C, H, W = x.shape
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    xp = np.zeros((N, C, H + pads[0] + pads[1] + R, W + pads[2] + pads[3] + S))
    xp[:, :, pads[0]:pads[0] + H, pads[2]:pads[2] + W] = x
    cols = np.empty((N, P, Q, C, R, S))
    for r in range(R):
        for s in range(S):
            rows = np.arange(P) * stride[0] + r
            cs = np.arange(Q) * stride[1] + s
            cols[:, :, :, :, r, s] = xp[:, :, rows][:, :, :, cs].transpose(0, 2, 3, 1)
    return cols.reshape(N, P * Q, C * R * S), P, Q


@pytest.mark.parametrize("case", FUZZ, ids=[str(i) for i in range(len(FUZZ))])
def test_im2col_product(case):
    N, C, H, W, K, R, S, stride, pads = case
    seed = 800 + 7 * FUZZ.index(case)
    x = _rand(seed, (N, C, H, W))
    cols, P, Q = _im2col(x, R, S, stride, pads)
    dy = _rand(seed + 1, (N, K, P, Q))
    want = sum(dy[n].reshape(K, P * Q) @ cols[n] for n in range(N)).reshape(K, C, R, S)
    dw, _ = oracle.conv2d_bwd_filter(x, dy, (K, C, R, S), stride, pads)
    np.testing.assert_allclose(dw, want, rtol=1e-13, atol=1e-13)


def _in_count(n_out, n_in, f, stride, pad):
    """#{p < n_out: 0 <= p*stride + r - pad < n_in} for each tap r < f."""
    return np.array([sum(1 for p in range(n_out) if 0 <= p * stride + r - pad < n_in) for r in range(f)])


@pytest.mark.parametrize("case", FUZZ + [(2, 1, 81, 35, 3, 21, 11, (2, 1), (10, 10, 0, 10))],
                         ids=[str(i) for i in range(len(FUZZ) + 1)])
def test_all_ones_closed_form(case):
    N, C, H, W, K, R, S, stride, pads = case
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    x = np.ones((N, C, H, W))
    dy = np.ones((N, K, P, Q))
    cr = _in_count(P, H, R, stride[0], pads[0])
    cs = _in_count(Q, W, S, stride[1], pads[2])
    want = np.broadcast_to((N * cr[:, None] * cs[None, :]).astype(np.float64), (K, C, R, S))
    dw, _ = oracle.conv2d_bwd_filter(x, dy, (K, C, R, S), stride, pads)
    assert np.array_equal(dw, want)


def test_one_by_one_filter_is_a_matmul():
    N, C, H, W, K = 3, 5, 6, 7, 4
    stride = (2, 1)
    x = _rand(901, (N, C, H, W))
    P, Q = _fwd_dims(H, W, 1, 1, stride, (0, 0, 0, 0))
    dy = _rand(902, (N, K, P, Q))
    xs = x[:, :, ::stride[0], ::stride[1]][:, :, :P, :Q]
    want = np.zeros((K, C))
    for n in range(N):
        want += dy[n].reshape(K, -1) @ xs[n].reshape(C, -1).T
    dw, _ = oracle.conv2d_bwd_filter(x, dy, (K, C, 1, 1), stride, (0, 0, 0, 0))
    np.testing.assert_allclose(dw[:, :, 0, 0], want, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("n0,c0,h0,w0", [(0, 0, 0, 0), (1, 2, 4, 3), (1, 1, 6, 0)])
def test_one_hot_input_is_a_shifted_copy(n0, c0, h0, w0):
    N, C, H, W, K, R, S = 2, 3, 7, 5, 4, 3, 2
    stride, pads = (2, 1), (1, 1, 1, 0)
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    x = np.zeros((N, C, H, W))
    x[n0, c0, h0, w0] = 1.0
    dy = _rand(903, (N, K, P, Q))
    want = np.zeros((K, C, R, S))
    for r in range(R):
        for s in range(S):
            hh, ww = h0 + pads[0] - r, w0 + pads[2] - s
            if hh >= 0 and ww >= 0 and hh % stride[0] == 0 and ww % stride[1] == 0:
                p, q = hh // stride[0], ww // stride[1]
                if p < P and q < Q:
                    want[:, c0, r, s] = dy[n0, :, p, q]
    dw, _ = oracle.conv2d_bwd_filter(x, dy, (K, C, R, S), stride, pads)
    assert np.array_equal(dw, want)


def test_layouts_and_alpha_beta():
    N, C, H, W, K, R, S = 2, 3, 9, 7, 4, 3, 3
    stride, pads = (1, 2), (1, 1, 0, 2)
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    x = _rand(951, (N, C, H, W))
    dy = _rand(952, (N, K, P, Q))
    base, bound = oracle.conv2d_bwd_filter(x, dy, (K, C, R, S), stride, pads)
    xn = np.ascontiguousarray(x.transpose(0, 2, 3, 1)).transpose(0, 3, 1, 2)
    dyn = np.ascontiguousarray(dy.transpose(0, 2, 3, 1)).transpose(0, 3, 1, 2)
    dw, _ = oracle.conv2d_bwd_filter(xn, dyn, (K, C, R, S), stride, pads)
    assert np.array_equal(dw, base)
    old = _rand(953, (K, C, R, S))
    dw, _ = oracle.conv2d_bwd_filter(x, dy, (K, C, R, S), stride, pads, alpha=0.5, beta=-2.0, dw_old=old)
    np.testing.assert_allclose(dw, 0.5 * base - 2.0 * old, rtol=0, atol=1e-15)
    assert np.all(bound >= np.abs(base))
    idx = np.array([[0, 0, 0, 0], [3, 2, 2, 2], [1, 1, 0, 2], [2, 0, 1, 1]], dtype=np.int64)
    vals, bnd = oracle.conv2d_bwd_filter_at(x, dy, (K, C, R, S), idx, stride, pads, alpha=0.5, beta=-2.0,
                                            dw_old_vals=old[tuple(idx.T)])
    assert np.array_equal(vals, dw[tuple(idx.T)])
    assert np.array_equal(bnd, bound[tuple(idx.T)])

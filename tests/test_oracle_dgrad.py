"""Pins for the oracle's data gradient (backward pass with respect to x).

The pages print no formula for it; the reading taken is the adjoint of the
forward sum in x.  Each test checks it against something other than itself:
the adjoint identity <conv(x, F), dy> = <x, dgrad(dy, F)> with the (already
pinned) forward oracle, the transpose of the dense Toeplitz matrix built the
other way round, an integer closed form for all-ones inputs, a shifted copy
for delta filters, and, at stride 1, the forward pass of the flipped and
transposed filter.  test_oracle_mutants.py plants slips in the data-gradient
code and checks that these tests catch them.
"""
import itertools

import numpy as np
import pytest

import gen
import oracle
from test_oracle import toeplitz


def _rand(seed, shape):
    return gen.uniform(seed, shape, -1.0, 1.0)


def _fwd_dims(H, W, R, S, stride, pads):
    pt, pb, pl, pr = pads
    return (H + pt + pb - R) // stride[0] + 1, (W + pl + pr - S) // stride[1] + 1


# (N, C, H, W, K, R, S, stride, pads): square and non-square, strides 1-3,
# asymmetric padding, filters wider than tall, a stride that skips rows
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
    seed = 100 + 7 * FUZZ.index(case)
    x = _rand(seed, (N, C, H, W))
    w = _rand(seed + 1, (K, C, R, S))
    y, _ = oracle.conv2d_fprop(x, w, stride, pads)
    dy = _rand(seed + 2, y.shape)
    dx, bound = oracle.conv2d_bwd_data(dy, w, x.shape, stride, pads)
    lhs = float(np.sum(y * dy))
    rhs = float(np.sum(x * dx))
    scale = float(np.sum(np.abs(x) * bound))
    assert abs(lhs - rhs) <= 1e-13 * max(scale, 1.0), (lhs, rhs)


@pytest.mark.parametrize("case", FUZZ, ids=[str(i) for i in range(len(FUZZ))])
def test_toeplitz_transpose(case):
    N, C, H, W, K, R, S, stride, pads = case
    seed = 200 + 7 * FUZZ.index(case)
    w = _rand(seed, (K, C, R, S))
    T, P, Q = toeplitz(w, H, W, stride, pads)
    dy = _rand(seed + 1, (N, K, P, Q))
    want = np.stack([T.T @ dy[n].reshape(-1) for n in range(N)]).reshape(N, C, H, W)
    dx, _ = oracle.conv2d_bwd_data(dy, w, (N, C, H, W), stride, pads)
    np.testing.assert_allclose(dx, want, rtol=1e-13, atol=1e-13)


def _tap_count(n_out, n_in, f, stride, pad):
    """#{(r, p): p*stride + r - pad == i, 0 <= r < f, 0 <= p < n_out} for each input i."""
    cnt = np.zeros(n_in, dtype=np.int64)
    for i in range(n_in):
        for r in range(f):
            hh = i + pad - r
            if hh >= 0 and hh % stride == 0 and hh // stride < n_out:
                cnt[i] += 1
    return cnt


@pytest.mark.parametrize("case", FUZZ + [(2, 3, 81, 35, 4, 21, 11, (2, 1), (10, 10, 0, 10))],
                         ids=[str(i) for i in range(len(FUZZ) + 1)])
def test_all_ones_closed_form(case):
    N, C, H, W, K, R, S, stride, pads = case
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    dy = np.ones((N, K, P, Q))
    w = np.ones((K, C, R, S))
    ch = _tap_count(P, H, R, stride[0], pads[0])
    cw = _tap_count(Q, W, S, stride[1], pads[2])
    want = np.broadcast_to((K * ch[:, None] * cw[None, :]).astype(np.float64), (N, C, H, W))
    dx, _ = oracle.conv2d_bwd_data(dy, w, (N, C, H, W), stride, pads)
    assert np.array_equal(dx, want)


@pytest.mark.parametrize("r0,s0", [(0, 0), (2, 1), (1, 3)])
def test_delta_filter_is_a_shifted_copy(r0, s0):
    N, C, H, W, R, S = 2, 3, 11, 9, 3, 4
    stride, pads = (2, 1), (1, 2, 2, 0)
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    w = np.zeros((C, C, R, S))
    for c in range(C):
        w[c, c, r0, s0] = 1.0
    dy = _rand(301, (N, C, P, Q))
    want = np.zeros((N, C, H, W))
    for h, x in itertools.product(range(H), range(W)):
        hh, ww = h + pads[0] - r0, x + pads[2] - s0
        if hh >= 0 and ww >= 0 and hh % stride[0] == 0 and ww % stride[1] == 0:
            p, q = hh // stride[0], ww // stride[1]
            if p < P and q < Q:
                want[:, :, h, x] = dy[:, :, p, q]
    dx, _ = oracle.conv2d_bwd_data(dy, w, (N, C, H, W), stride, pads)
    assert np.array_equal(dx, want)


@pytest.mark.parametrize("R,S,pads", [(3, 3, (1, 1, 1, 1)), (5, 5, (2, 2, 2, 2)), (3, 2, (0, 2, 1, 0))])
def test_stride1_is_forward_of_flipped_transposed_filter(R, S, pads):
    N, C, H, W, K = 2, 4, 9, 8, 5
    P, Q = _fwd_dims(H, W, R, S, (1, 1), pads)
    w = _rand(401, (K, C, R, S))
    dy = _rand(402, (N, K, P, Q))
    wt = np.ascontiguousarray(w.transpose(1, 0, 2, 3)[:, :, ::-1, ::-1])
    pads_t = (R - 1 - pads[0], H - P + pads[0], S - 1 - pads[2], W - Q + pads[2])
    want, _ = oracle.conv2d_fprop(dy, wt, (1, 1), pads_t)
    assert want.shape == (N, C, H, W)
    dx, _ = oracle.conv2d_bwd_data(dy, w, (N, C, H, W), (1, 1), pads)
    np.testing.assert_allclose(dx, want, rtol=1e-13, atol=1e-14)


def test_strided_dy_layouts_agree():
    N, C, H, W, K, R, S = 2, 3, 9, 7, 4, 3, 3
    stride, pads = (2, 1), (1, 1, 0, 2)
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    w = _rand(501, (K, C, R, S))
    dy = _rand(502, (N, K, P, Q))
    base, _ = oracle.conv2d_bwd_data(dy, w, (N, C, H, W), stride, pads)
    nhwc = np.ascontiguousarray(dy.transpose(0, 2, 3, 1)).transpose(0, 3, 1, 2)
    padded = np.zeros((N, K, P, 16))
    padded[..., :Q] = dy
    for view in (nhwc, padded[..., :Q]):
        dx, _ = oracle.conv2d_bwd_data(view, w, (N, C, H, W), stride, pads)
        assert np.array_equal(dx, base)


def test_alpha_beta_and_sampled_values():
    N, C, H, W, K, R, S = 2, 3, 8, 8, 4, 3, 3
    stride, pads = (1, 2), (1, 1, 1, 0)
    P, Q = _fwd_dims(H, W, R, S, stride, pads)
    w = _rand(601, (K, C, R, S))
    dy = _rand(602, (N, K, P, Q))
    old = _rand(603, (N, C, H, W))
    base, bound = oracle.conv2d_bwd_data(dy, w, (N, C, H, W), stride, pads)
    dx, _ = oracle.conv2d_bwd_data(dy, w, (N, C, H, W), stride, pads, alpha=0.5, beta=-2.0, dx_old=old)
    np.testing.assert_allclose(dx, 0.5 * base - 2.0 * old, rtol=0, atol=1e-15)
    idx = np.array([[0, 0, 0, 0], [1, 2, 7, 7], [0, 1, 3, 5], [1, 0, 6, 1]], dtype=np.int64)
    vals, bnd = oracle.conv2d_bwd_data_at(dy, w, (N, C, H, W), idx, stride, pads, alpha=0.5, beta=-2.0,
                                          dx_old_vals=old[tuple(idx.T)])
    assert np.array_equal(vals, dx[tuple(idx.T)])
    assert np.array_equal(bnd, bound[tuple(idx.T)])


def test_shape_mismatch_rejected():
    w = np.ones((4, 3, 3, 3))
    with pytest.raises(ValueError):
        oracle.conv2d_bwd_data(np.ones((2, 4, 5, 5)), w, (2, 3, 9, 9), (1, 1), (1, 1, 1, 1))

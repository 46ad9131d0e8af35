"""Pins for the oracle's pooling forward pass (no GPU).

The pages print no formula (cuDNN page, "Proposed Method", lists pooling
among the library's routines); the reading taken is max / average over the
window positions inside the input plane.  Each test checks the oracle
against something other than itself: a numpy sliding-window computation over
an explicitly padded array, closed forms for all-ones inputs, identity for a
1x1 window, and layout independence.  test_oracle_mutants.py plants slips in
the pooling code and checks these tests catch them.
"""
import numpy as np
import pytest

import gen
import oracle

MODES = ["max", "avg_include_pad", "avg_exclude_pad"]


def _dims(H, W, R, S, stride, pads):
    pt, pb, pl, pr = pads
    return (H + pt + pb - R) // stride[0] + 1, (W + pl + pr - S) // stride[1] + 1


def _numpy_pool(x, R, S, stride, pads, mode):
    """Sliding windows over x padded with a marker; the marker decides what padding counts as."""
    N, C, H, W = x.shape
    pt, pb, pl, pr = pads
    P, Q = _dims(H, W, R, S, stride, pads)
    fill = -np.inf if mode == "max" else 0.0
    xp = np.full((N, C, H + pt + pb, W + pl + pr), fill)
    xp[:, :, pt:pt + H, pl:pl + W] = x
    inside = np.zeros((H + pt + pb, W + pl + pr))
    inside[pt:pt + H, pl:pl + W] = 1.0
    win = np.lib.stride_tricks.sliding_window_view(xp, (R, S), axis=(2, 3))
    win = win[:, :, ::stride[0], ::stride[1]][:, :, :P, :Q]
    cnt = np.lib.stride_tricks.sliding_window_view(inside, (R, S))[::stride[0], ::stride[1]][:P, :Q].sum(axis=(2, 3))
    if mode == "max":
        out = win.max(axis=(4, 5))
        return np.where(cnt[None, None] > 0, out, 0.0)
    total = win.sum(axis=(4, 5))
    if mode == "avg_include_pad":
        return total / (R * S)
    return np.where(cnt[None, None] > 0, total / np.maximum(cnt, 1)[None, None], 0.0)


CASES = [
    (2, 3, 7, 6, 3, 3, (2, 2), (0, 0, 0, 0)),
    (1, 2, 9, 9, 3, 3, (2, 2), (1, 1, 1, 1)),
    (2, 4, 8, 11, 2, 3, (1, 2), (1, 0, 2, 1)),
    (3, 1, 5, 5, 5, 5, (1, 1), (2, 2, 2, 2)),
    (1, 5, 27, 27, 3, 3, (2, 2), (0, 0, 0, 0)),
    (2, 2, 6, 10, 4, 2, (3, 1), (3, 3, 1, 1)),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_matches_numpy_sliding_windows(case, mode):
    N, C, H, W, R, S, stride, pads = case
    x = gen.uniform(1000 + 17 * CASES.index(case), (N, C, H, W), -1.0, 1.0)
    want = _numpy_pool(x, R, S, stride, pads, mode)
    got = oracle.pool2d_forward(x, (R, S), stride, pads, mode)
    if mode == "max":
        assert np.array_equal(got, want)
    else:
        np.testing.assert_allclose(got, want, rtol=1e-15, atol=1e-16)


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_all_ones_closed_forms(case):
    N, C, H, W, R, S, stride, pads = case
    x = np.ones((N, C, H, W))
    P, Q = _dims(H, W, R, S, stride, pads)
    ch = np.array([sum(1 for r in range(R) if 0 <= p * stride[0] + r - pads[0] < H) for p in range(P)])
    cw = np.array([sum(1 for s in range(S) if 0 <= q * stride[1] + s - pads[2] < W) for q in range(Q)])
    cnt = ch[:, None] * cw[None, :]
    assert np.array_equal(oracle.pool2d_forward(x, (R, S), stride, pads, "max"),
                          np.broadcast_to((cnt > 0).astype(float), (N, C, P, Q)))
    assert np.array_equal(oracle.pool2d_forward(x, (R, S), stride, pads, "avg_include_pad"),
                          np.broadcast_to(cnt / (R * S), (N, C, P, Q)))
    assert np.array_equal(oracle.pool2d_forward(x, (R, S), stride, pads, "avg_exclude_pad"),
                          np.broadcast_to((cnt > 0).astype(float), (N, C, P, Q)))


def test_negative_plane_max_ignores_padding():
    x = -1.0 - gen.uniform(1101, (1, 2, 4, 4), 0.0, 1.0)     # all below -1
    got = oracle.pool2d_forward(x, (3, 3), (1, 1), (1, 1, 1, 1), "max")
    assert np.all(got < -1.0)


@pytest.mark.parametrize("mode", MODES)
def test_one_by_one_window_is_a_copy(mode):
    x = gen.uniform(1102, (2, 3, 5, 7), -1.0, 1.0)
    assert np.array_equal(oracle.pool2d_forward(x, (1, 1), (1, 1), (0, 0, 0, 0), mode), x)


def test_layouts_and_alpha_beta():
    x = gen.uniform(1103, (2, 3, 9, 8), -1.0, 1.0)
    base = oracle.pool2d_forward(x, (3, 2), (2, 1), (1, 0, 0, 1), "avg_exclude_pad")
    xn = np.ascontiguousarray(x.transpose(0, 2, 3, 1)).transpose(0, 3, 1, 2)
    assert np.array_equal(oracle.pool2d_forward(xn, (3, 2), (2, 1), (1, 0, 0, 1), "avg_exclude_pad"), base)
    old = gen.uniform(1104, base.shape, -1.0, 1.0)
    got = oracle.pool2d_forward(x, (3, 2), (2, 1), (1, 0, 0, 1), "avg_exclude_pad", alpha=2.0, beta=-0.5,
                                y_old=old)
    np.testing.assert_allclose(got, 2.0 * base - 0.5 * old, rtol=0, atol=1e-15)

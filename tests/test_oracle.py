"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: hand-worked
values, a dense Toeplitz-matrix product built the other way round (output x
input position pairs, tap derived from the pair), a plain channel matmul, a
shifted copy, an integer closed form, linearity, and layout independence.
A dropped term, a wrong sign or index, a flipped filter or swapped k/c
operands each break at least one of them (see test_oracle_mutants.py).
"""
import itertools
import json
import os

import numpy as np
import pytest

import gen
import oracle
from gen import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _dims(H, W, R, S, u, v, pads):
    pt, pb, pl, pr = pads
    return (H + pt + pb - R) // u + 1, (W + pl + pr - S) // v + 1


def toeplitz(w, H, W, stride, pads):
    """Dense T with T[(k,p,q),(c,h,w)] = F[k,c,h-p*u+pt, w-q*v+pl] inside the filter, else 0."""
    K, C, R, S = w.shape
    u, v = stride
    pt, pb, pl, pr = pads
    P, Q = _dims(H, W, R, S, u, v, pads)
    r = np.arange(H)[None, :] - np.arange(P)[:, None] * u + pt        # (P, H)
    s = np.arange(W)[None, :] - np.arange(Q)[:, None] * v + pl        # (Q, W)
    vr = (r >= 0) & (r < R)
    vs = (s >= 0) & (s < S)
    rc = np.clip(r, 0, R - 1)
    sc = np.clip(s, 0, S - 1)
    # T6[k, c, p, h, q, w]
    T6 = w[:, :, rc[:, :, None, None], sc[None, None, :, :]]
    T6 = T6 * (vr[:, :, None, None] & vs[None, None, :, :])
    T = T6.transpose(0, 2, 4, 1, 3, 5).reshape(K * P * Q, C * H * W)
    return T, P, Q


def toeplitz_conv(x, w, stride, pads):
    N, C, H, W = x.shape
    T, P, Q = toeplitz(w, H, W, stride, pads)
    y = np.stack([T @ x[n].reshape(-1) for n in range(N)])
    return y.reshape(N, w.shape[0], P, Q)


def _rand(seed, shape):
    return gen.uniform(seed, shape, -1.0, 1.0)


# ---------------------------------------------------------------- hand examples

def test_hand_examples():
    with open(GOLDEN) as fh:
        data = json.load(fh)
    assert len(data["examples"]) >= 2
    for ex in data["examples"]:
        x = np.array(ex["x"], dtype=np.float64)
        w = np.array(ex["w"], dtype=np.float64)
        want = np.array(ex["y"], dtype=np.float64)
        y, _ = oracle.conv2d_fprop(x, w, tuple(ex["stride"]),
                                   tuple(ex["padding_top_bottom_left_right"]))
        assert y.shape == want.shape, ex["name"]
        assert np.array_equal(y, want), ex["name"]


# ---------------------------------------------------------------- Toeplitz

def test_toeplitz_tiny_workload():
    lay = workloads.TINY[0]
    x = gen.round_to(_rand(11, lay.x_shape), "f32")
    w = gen.round_to(_rand(12, lay.w_shape), "f32")
    y, bound = oracle.conv2d_fprop(x, w, lay.stride, lay.padding)
    yt = toeplitz_conv(x, w, lay.stride, lay.padding)
    assert y.shape == (2, 16, 12, 12)
    assert np.all(np.abs(y - yt) <= 1e-14 * bound + 1e-300)


@pytest.mark.parametrize("case", range(40))
def test_toeplitz_fuzz(case):
    rng = np.random.default_rng(1000 + case)
    N = int(rng.integers(1, 3))
    C = int(rng.integers(1, 5))
    K = int(rng.integers(1, 6))
    R = int(rng.integers(1, 6))
    S = int(rng.integers(1, 6))
    u = int(rng.integers(1, 5))
    v = int(rng.integers(1, 5))
    pads = tuple(int(t) for t in rng.integers(0, 4, size=4))
    H = int(rng.integers(max(1, R - pads[0] - pads[1]), 12))
    W = int(rng.integers(max(1, S - pads[2] - pads[3]), 12))
    x = _rand(2000 + case, (N, C, H, W))
    w = _rand(3000 + case, (K, C, R, S))
    y, bound = oracle.conv2d_fprop(x, w, (u, v), pads)
    yt = toeplitz_conv(x, w, (u, v), pads)
    assert y.shape == yt.shape
    assert np.all(np.abs(y - yt) <= 1e-14 * bound + 1e-300), (N, C, H, W, K, R, S, u, v, pads)


# ---------------------------------------------------------------- 1x1 filter

@pytest.mark.parametrize("stride", [(1, 1), (2, 3)])
def test_one_by_one_is_channel_matmul(stride):
    N, C, H, W, K = 2, 7, 9, 10, 5
    x = _rand(21, (N, C, H, W))
    w = _rand(22, (K, C, 1, 1))
    y, bound = oracle.conv2d_fprop(x, w, stride, (0, 0, 0, 0))
    u, v = stride
    P, Q = (H - 1) // u + 1, (W - 1) // v + 1
    assert y.shape == (N, K, P, Q)
    F = w[:, :, 0, 0]
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                want = np.zeros(K)
                for k in range(K):
                    for c in range(C):
                        want[k] += F[k, c] * x[n, c, p * u, q * v]
                assert np.allclose(y[n, :, p, q], want, rtol=0, atol=1e-14 * (1 + bound[n, :, p, q].max()))


# ---------------------------------------------------------------- delta filter

@pytest.mark.parametrize("r0,s0,stride,pads", [
    (0, 0, (1, 1), (0, 0, 0, 0)),
    (2, 1, (1, 1), (1, 1, 1, 1)),
    (1, 3, (2, 1), (3, 0, 0, 2)),
    (3, 0, (1, 3), (0, 2, 3, 1)),
])
def test_delta_filter_is_shifted_copy(r0, s0, stride, pads):
    N, C, H, W = 2, 3, 8, 9
    R, S = 4, 4
    x = _rand(31, (N, C, H, W))
    w = np.zeros((C, C, R, S))
    for c in range(C):
        w[c, c, r0, s0] = 1.0
    y, _ = oracle.conv2d_fprop(x, w, stride, pads)
    u, v = stride
    pt, pb, pl, pr = pads
    P, Q = _dims(H, W, R, S, u, v, pads)
    assert y.shape == (N, C, P, Q)
    want = np.zeros_like(y)
    for p in range(P):
        for q in range(Q):
            h = p * u + r0 - pt
            ww = q * v + s0 - pl
            if 0 <= h < H and 0 <= ww < W:
                want[:, :, p, q] = x[:, :, h, ww]
    assert np.array_equal(y, want)


# ---------------------------------------------------------------- all-ones closed form

def _ones_count(P, Q, C, H, W, R, S, u, v, pads):
    pt, pb, pl, pr = pads
    ch = np.array([sum(1 for r in range(R) if 0 <= p * u + r - pt < H) for p in range(P)])
    cw = np.array([sum(1 for s in range(S) if 0 <= q * v + s - pl < W) for q in range(Q)])
    return C * ch[:, None] * cw[None, :]


@pytest.mark.parametrize("pads,stride", [((1, 1, 1, 1), (1, 1)), ((20, 20, 0, 10), (2, 2)),
                                         ((0, 3, 2, 0), (3, 2))])
def test_all_ones_closed_form_small(pads, stride):
    N, C, H, W, K, R, S = 2, 3, 17, 23, 2, 5, 4
    x = np.ones((N, C, H, W))
    w = np.ones((K, C, R, S))
    y, bound = oracle.conv2d_fprop(x, w, stride, pads)
    P, Q = _dims(H, W, R, S, *stride, pads)
    want = _ones_count(P, Q, C, H, W, R, S, *stride, pads)
    assert y.shape == (N, K, P, Q)
    assert np.array_equal(y, np.broadcast_to(want, y.shape))
    assert np.array_equal(bound, y)


def _sample_coords(rng, N, K, P, Q, count):
    """Random coordinates plus every corner and edge midpoint."""
    pts = [(n, k, p, q) for n in (0, N - 1) for k in (0, K - 1)
           for p in (0, P // 2, P - 1) for q in (0, Q // 2, Q - 1)]
    rnd = np.stack([rng.integers(0, N, count), rng.integers(0, K, count),
                    rng.integers(0, P, count), rng.integers(0, Q, count)], axis=1)
    return np.concatenate([np.array(pts, dtype=np.int64), rnd.astype(np.int64)])


@pytest.mark.parametrize("lay", workloads.ALL_LAYERS, ids=lambda l: l.name)
def test_all_ones_closed_form_workload_shapes(lay):
    """At every workload's real shape, on sampled outputs (integer, exact)."""
    x = np.ones((1, lay.C, lay.H, lay.W))     # one image: the count does not depend on n
    w = np.ones((1, lay.C, lay.R, lay.S))
    pb = oracle.make_problem(x.shape, [s // 8 for s in x.strides], w.shape, lay.stride, lay.padding)
    P, Q = oracle.output_dims(pb)
    assert (P, Q) == _dims(lay.H, lay.W, lay.R, lay.S, *lay.stride, lay.padding)
    rng = np.random.default_rng(lay.config * 100 + lay.layer)
    idx = _sample_coords(rng, 1, 1, P, Q, 64)
    y, bound = oracle.conv2d_fprop_at(x, w, idx, lay.stride, lay.padding)
    want = _ones_count(P, Q, lay.C, lay.H, lay.W, lay.R, lay.S, *lay.stride, lay.padding)
    assert np.array_equal(y, want[idx[:, 2], idx[:, 3]].astype(np.float64))


def test_output_dims_floor_and_errors():
    # speech layer 1: (700 + 0 + 10 - 11) / 2 = 349.5 -> Q = 350; (161 + 40 - 41)/2 + 1 = 81
    lay = workloads.by_name("speech_l1")
    pb = oracle.make_problem(lay.x_shape, (1, 1, 1, 1), lay.w_shape, lay.stride, lay.padding)
    assert oracle.output_dims(pb) == (81, 350)
    lay = workloads.by_name("speech_l2")
    pb = oracle.make_problem(lay.x_shape, (1, 1, 1, 1), lay.w_shape, lay.stride, lay.padding)
    assert oracle.output_dims(pb) == (41, 350)
    lay = workloads.by_name("overfeat_l1")
    pb = oracle.make_problem(lay.x_shape, (1, 1, 1, 1), lay.w_shape, lay.stride, lay.padding)
    assert oracle.output_dims(pb) == (56, 56)
    # filter larger than the padded input: no output
    pb = oracle.make_problem((1, 1, 3, 3), (9, 9, 3, 1), (1, 1, 5, 1), (1, 1), (0, 1, 0, 0))
    with pytest.raises(ValueError):
        oracle.output_dims(pb)
    with pytest.raises(ValueError):
        oracle.make_problem((1, 2, 3, 3), (18, 9, 3, 1), (1, 3, 1, 1))


# ---------------------------------------------------------------- linearity

def test_linearity_in_filter_and_input():
    N, C, H, W, K, R, S = 2, 4, 11, 9, 3, 3, 5
    stride, pads = (2, 1), (1, 2, 0, 3)
    x1, x2 = _rand(41, (N, C, H, W)), _rand(42, (N, C, H, W))
    f1, f2 = _rand(43, (K, C, R, S)), _rand(44, (K, C, R, S))
    a, b = 0.75, -1.5
    y_mix, bnd = oracle.conv2d_fprop(x1, a * f1 + b * f2, stride, pads)
    y1, b1 = oracle.conv2d_fprop(x1, f1, stride, pads)
    y2, b2 = oracle.conv2d_fprop(x1, f2, stride, pads)
    scale = abs(a) * b1 + abs(b) * b2
    assert np.all(np.abs(y_mix - (a * y1 + b * y2)) <= 1e-13 * scale)
    y_mix, _ = oracle.conv2d_fprop(a * x1 + b * x2, f1, stride, pads)
    y2, b2 = oracle.conv2d_fprop(x2, f1, stride, pads)
    scale = abs(a) * b1 + abs(b) * b2
    assert np.all(np.abs(y_mix - (a * y1 + b * y2)) <= 1e-13 * scale)


# ---------------------------------------------------------------- layouts and strides

def _relayout(x, layout, pitch):
    N, C, H, W = x.shape
    st = workloads.padded_strides(N, C, H, W, layout, pitch)
    buf = np.full(workloads.storage_elems(N, C, H, W, st), np.nan)
    view = np.lib.stride_tricks.as_strided(buf, shape=x.shape, strides=[s * 8 for s in st])
    view[...] = x
    return view


def test_layout_and_stride_independence():
    N, C, H, W, K, R, S = 3, 5, 13, 13, 4, 3, 3
    x = _rand(51, (N, C, H, W))
    w = _rand(52, (K, C, R, S))
    ref, _ = oracle.conv2d_fprop(x, w, (1, 1), (1, 1, 1, 1))
    for layout, pitch in [("nchw", 0), ("nhwc", 0), ("nchw", 16), ("nhwc", 16)]:
        xv = _relayout(x, layout, pitch)
        y, _ = oracle.conv2d_fprop(xv, w, (1, 1), (1, 1, 1, 1))
        assert np.array_equal(y, ref), (layout, pitch)
    # a channel sub-range view reads only its own channels
    y_sub, _ = oracle.conv2d_fprop(x[:, 1:4], w[:, 1:4], (1, 1), (1, 1, 1, 1))
    y_cut, _ = oracle.conv2d_fprop(np.ascontiguousarray(x[:, 1:4]), w[:, 1:4], (1, 1), (1, 1, 1, 1))
    assert np.array_equal(y_sub, y_cut)


# ---------------------------------------------------------------- alpha, beta, bound

def test_alpha_beta_and_bound():
    N, C, H, W, K, R, S = 2, 3, 7, 6, 4, 3, 2
    x = gen.integers(61, (N, C, H, W))
    w = gen.integers(62, (K, C, R, S))
    y1, bound = oracle.conv2d_fprop(x, w, (1, 2), (1, 0, 1, 1))
    y_old = gen.integers(63, y1.shape)
    y, _ = oracle.conv2d_fprop(x, w, (1, 2), (1, 0, 1, 1), alpha=0.5, beta=0.25, y_old=y_old)
    assert np.array_equal(y, 0.5 * y1 + 0.25 * y_old)        # all values exact in fp64
    y, _ = oracle.conv2d_fprop(x, w, (1, 2), (1, 0, 1, 1), alpha=0.0, beta=-2.0, y_old=y_old)
    assert np.array_equal(y, -2.0 * y_old)
    # beta == 0: y_old is not read, so NaN there cannot leak
    idx = np.array([[0, 0, 0, 0], [1, 3, 2, 1]], dtype=np.int64)
    yv, _ = oracle.conv2d_fprop_at(x, w, idx, (1, 2), (1, 0, 1, 1), beta=0.0,
                                   y_old_vals=np.array([np.nan, np.nan]))
    assert np.all(np.isfinite(yv))
    # bound: |acc| <= B, with equality for non-negative operands
    assert np.all(np.abs(y1) <= bound)
    xa, wa = np.abs(x), np.abs(w)
    ya, ba = oracle.conv2d_fprop(xa, wa, (1, 2), (1, 0, 1, 1))
    assert np.array_equal(ya, ba)
    ym, _ = oracle.conv2d_fprop(xa, wa, (1, 2), (1, 0, 1, 1))
    assert np.array_equal(ba, ym)


def test_bound_is_sum_of_abs_products():
    x = np.array([[[[1.0, -2.0], [3.0, -4.0]]]])
    w = np.array([[[[1.0, 1.0], [-1.0, 1.0]]]])
    y, b = oracle.conv2d_fprop(x, w)
    # 1*1 + (-2)*1 + 3*(-1) + (-4)*1 = -8 ; |1| + |-2| + |-3| + |-4| = 10
    assert y.item() == -8.0 and b.item() == 10.0


def test_sampled_equals_full():
    N, C, H, W, K, R, S = 2, 6, 10, 12, 5, 3, 4
    stride, pads = (2, 1), (2, 0, 1, 2)
    x = _rand(71, (N, C, H, W))
    w = _rand(72, (K, C, R, S))
    y, b = oracle.conv2d_fprop(x, w, stride, pads)
    idx = np.array(list(itertools.product(range(N), range(K), range(y.shape[2]), range(y.shape[3]))),
                   dtype=np.int64)
    ys, bs = oracle.conv2d_fprop_at(x, w, idx, stride, pads)
    assert np.array_equal(ys, y.reshape(-1))
    assert np.array_equal(bs, b.reshape(-1))
    with pytest.raises(ValueError):
        oracle.conv2d_fprop_at(x, w, np.array([[0, K, 0, 0]]), stride, pads)


def test_thread_count_does_not_change_results():
    x = _rand(81, (3, 4, 9, 9))
    w = _rand(82, (6, 4, 3, 3))
    y1, b1 = oracle.conv2d_fprop(x, w, (1, 1), (1, 1, 1, 1), nthreads=1)
    y4, b4 = oracle.conv2d_fprop(x, w, (1, 1), (1, 1, 1, 1), nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(b1, b4)

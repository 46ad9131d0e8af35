"""GPU parity of the pooling forward pass (mic_pool_forward) against the oracle.

Every mode on small shapes (padding, strides, non-square windows, NCHW,
NHWC and padded rows) and the AlexNet pooling layers at full size are
compared in full.  Max pooling selects one input value, so it must match
bit-exactly; averages are held to the fp32 bound |err| <= 2e-6 * B with
B the same average of |x| (the oracle run on |x|), and the f64 and bf16
relative-L2 gates.
"""
import numpy as np
import pytest
import torch

import convolution_forward_conv2d_amd as mic
import gen
import oracle
from gen import workloads

import gpu_harness as H

pytestmark = pytest.mark.gpu

MODES = ["max", "avg_include_pad", "avg_exclude_pad"]

SHAPES = [
    dict(name="s2_3x3", N=2, C=5, Hh=27, Ww=27, R=3, S=3, stride=(2, 2), pads=(0, 0, 0, 0)),
    dict(name="padded", N=3, C=4, Hh=13, Ww=11, R=3, S=3, stride=(2, 2), pads=(1, 1, 1, 1)),
    dict(name="asym", N=2, C=3, Hh=9, Ww=14, R=2, S=4, stride=(1, 3), pads=(1, 0, 2, 1)),
    dict(name="overlap5", N=1, C=7, Hh=12, Ww=12, R=5, S=5, stride=(1, 1), pads=(2, 2, 2, 2)),
]


def _x(seed, shape, dtype):
    return gen.round_to(gen.uniform(seed, shape, -1.0, 1.0), dtype)


def _check_pool(dtype, mode, got, ref, bref, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), what
    if mode == "max":
        assert np.array_equal(got, ref), "%s: %d mismatches" % (what, int((got != ref).sum()))
    else:
        H.check(dtype, got, ref, bref, what=what)


def _run(x, y, window, stride, pads, mode, alpha=1.0, beta=0.0):
    plan = mic.PoolPlan(x, y, window, stride, pads, mode)
    try:
        plan(alpha, beta)
        torch.cuda.synchronize()
    finally:
        plan.close()
    return y


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("layout,pitch", [("nchw", 0), ("nhwc", 0), ("nchw", 16)])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s["name"])
def test_small_full_parity(dtype, layout, pitch, shape):
    N, C, Hh, Ww = shape["N"], shape["C"], shape["Hh"], shape["Ww"]
    if pitch and Ww > pitch:
        pytest.skip("row pitch narrower than the row")
    x64 = _x(1200 + SHAPES.index(shape), (N, C, Hh, Ww), dtype)
    x = H.to_device(x64, dtype, layout, pitch)
    window, stride, pads = (shape["R"], shape["S"]), shape["stride"], shape["pads"]
    for mode in MODES:
        ref = oracle.pool2d_forward(x64, window, stride, pads, mode)
        bref = oracle.pool2d_forward(np.abs(x64), window, stride, pads, mode)
        st = workloads.padded_strides(*ref.shape, layout, pitch)
        y = H.strided_empty(ref.shape, st, H.OUT_DT[dtype], H.dev())
        _run(x, y, window, stride, pads, mode)
        _check_pool(dtype, mode, y.double().cpu().numpy(), ref, bref,
                    "%s/%s/%s/%s" % (shape["name"], dtype, layout, mode))


@pytest.mark.parametrize("lay", workloads.POOLING, ids=lambda l: l.name)
@pytest.mark.parametrize("mode", MODES)
def test_workload_layers_full(lay, mode):
    print("layer", lay.name, mode, flush=True)
    x64 = _x(gen.derive_seed(lay.config, lay.layer, 0), lay.x_shape, lay.dtype)
    x = H.to_device(x64, lay.dtype)
    window = (lay.R, lay.S)
    ref = oracle.pool2d_forward(x64, window, lay.stride, lay.padding, mode)
    bref = oracle.pool2d_forward(np.abs(x64), window, lay.stride, lay.padding, mode)
    y = H.strided_empty(ref.shape, workloads.padded_strides(*ref.shape, "nchw", 0), torch.float32, H.dev())
    _run(x, y, window, lay.stride, lay.padding, mode)
    _check_pool(lay.dtype, mode, y.double().cpu().numpy(), ref, bref, lay.name)
    y2 = torch.zeros_like(y)
    _run(x, y2, window, lay.stride, lay.padding, mode)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_alpha_beta(dtype):
    x64 = gen.integers(1300, (2, 3, 9, 9), -4, 4)
    ref = oracle.pool2d_forward(x64, (3, 3), (2, 2), (1, 1, 1, 1), "avg_include_pad")
    old = gen.integers(1301, ref.shape, -4, 4)
    x = H.to_device(x64, dtype)
    y = torch.from_numpy(old).to(H.OUT_DT[dtype]).to(H.dev())
    _run(x, y, (3, 3), (2, 2), (1, 1, 1, 1), "max", alpha=0.5, beta=0.25)
    want = 0.5 * oracle.pool2d_forward(x64, (3, 3), (2, 2), (1, 1, 1, 1), "max") + 0.25 * old
    assert np.array_equal(y.double().cpu().numpy(), want)


def test_pool_error_statuses_on_device():
    x = torch.zeros((2, 3, 9, 9), device=H.dev())
    y = torch.zeros((2, 3, 4, 5), device=H.dev())                 # output is 4 x 4
    with pytest.raises(mic.MicError) as e:
        mic.pool2d_forward(x, (3, 3), (2, 2), (0, 0, 0, 0), "max", y=y)
    assert e.value.status == mic.MIC_STATUS_BAD_PARAM

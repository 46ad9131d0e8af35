"""GPU parity of the filter gradient (mic_conv_backward_filter) against the oracle.

Small shapes spanning several dw tiles with ragged edges are compared in
full for every kernel variant, also with the tiles run in reverse order (bit
for bit the same result); every workload layer's filter gradient is run at
full size and its whole dw compared with the whole oracle output (canary
cells around dw untouched, reruns bit-identical), and integer-valued inputs
are bit-exact on sampled (k, c, r, s) coordinates in every layout.  The halo kernel's
reduction in two parts (added atomically into a zeroed dw) is compared with one part, in
reversed tile order and on reruns (bit-identical: two terms added onto zero commute).  x is the layer's
seeded input, dy seeded uniform [-1, 1] (tensor id 3), both rounded to the
layer's storage type.

The fp32 per-element tolerance is the forward pass's, |err| <= 2e-6 * B
with B = sum |dy * x| over the reduction.  The reduction here runs over
N*P*Q positions (up to 907200, speech L1) instead of at most 9216 terms:
the relative-L2 gate (1e-5 fp32, 1e-2 bf16) is scaled by sqrt(L / 9216),
the growth of an fp32 sum's relative rounding error with its length when
the terms have mixed signs (gpu_harness.rel_l2_scale).  Measured without
the scaling, Overfeat L1 (L = 401408) gives 1.1e-5.
"""
import time

import numpy as np
import pytest
import torch

import convolution_forward_conv2d_amd as mic
import gen
import oracle
from gen import workloads
from gen.workloads import Layer

import gpu_harness as H
from test_parity_gpu import SMALL_SHAPES, U

pytestmark = pytest.mark.gpu

WG_VARIANTS = {
    "f32": ["wg_f32_128x128", "wg_f32_64x128", "wg_f32_128x64", "wg_f32_64x64", "wgh_f32_3x3_64x64",
            "wgh_f32_5x5_w24_64x64", "wgh_f32_5x5_w36_64x64", "wgh_f32_3x3_64x96", "wgh_f32x16_3x3_64x64",
            "wgh_f32x16_5x5_w24_64x64", "wgs_f32_32x32", "wgs_f32_16x16", "wgs_f32_8x16"],
    "f64": ["wg_f64_128x64", "wg_f64_64x64", "wgh_f64_3x3_64x64", "wgs_f64_32x32", "wgs_f64_16x16",
            "wgh_f64_3x3_64x64_ks4", "wgh_f64_3x3_64x96"],
    "bf16": ["wg_bf16_128x128", "wg_bf16_64x64", "wgs_bf16_32x32"],
}
# the 3x3 halo kernel that steps along output rows of exactly 12 columns (no padding positions)
WG_VARIANTS["f32"] += ["wgh_f32_3x3_q12_64x96", "wgh_f32_3x3_q13_64x64", "wgh_f32x16_5x5_q20_64x64",
                       "wgh_f32x16_5x5_q27_64x64", "wgh_f32x16_5x5_q20_64x48", "wgh_f32x16_5x5_q27_64x48",
                       "wgh_f32_3x3_q13_64x64_ks4", "wgh_f32_3x3_64x96_ks4", "wgh_f32_3x3_q12_64x96_ks4",
                       "wgh_f32x16_5x5_q20_64x48_ks4", "wgh_f32x16_5x5_q27_64x48_ks4",
                       "wgh_f32x16_pairs_s11_32x32", "wgh_f32x16_pairs_s11_32x32_ks4",
                       "wgh_f32x16_pairs_s11_32x64"]
# the first-layer kernels on the vector ALU (wgr_): 11-wide filter rows at column stride 2 or 4
WG_VARIANTS["f32"] += ["wgr_f32_s11_v2", "wgr_f32_s11_v4"]
# the halo variants (wgh_) take stride-1 layers of their filter size whose rows fit their pitch, the
# wgr_ variants their stride and filter width; the library answers NOT_SUPPORTED for other shapes,
# and every variant must run on at least one shape
# the channels-last bf16 kernel (wgc_) takes x and dy with channel stride 1 and
# 8-aligned strides and channel counts
WG_VARIANTS["bf16"] += ["wgc_bf16_64x64", "wgc_bf16_64x64_ks2", "wgc_bf16_64x64_ks3"]
# the halo kernel on bf16 x and dy, widened to fp32 as they are staged (fp32 MFMA)
WG_VARIANTS["bf16"] += ["wgh_bf16_3x3_64x64", "wgh_bf16_3x3_q13_64x64", "wgh_bf16_3x3_64x96_ks4"]
_MAY_REFUSE = ("wgh_", "wgr_", "wgc_")
_ran = set()


def _small(name, N, C, Hh, Ww, K, R, S, stride, pads, dtype, layout="nchw", pitch=0):
    return Layer(name, 9, 3, N, C, Hh, Ww, K, R, S, stride, pads, dtype, U, U,
                 layout=layout, row_pitch=pitch)


def _dy(lay, shape, integer=False):
    seed = gen.derive_seed(lay.config, lay.layer, 3)
    d = gen.integers(seed, shape, -4, 4) if integer else gen.uniform(seed, shape, -1.0, 1.0)
    return gen.round_to(d, lay.dtype)


def _run(lay, x, dy, dw, alpha=1.0, beta=0.0):
    plan = mic.WgradPlan(x, dy, dw, lay.stride, lay.padding)
    try:
        plan(alpha, beta)
        torch.cuda.synchronize()
    finally:
        plan.close()
    return dw


def _out(lay, fill=float("nan")):
    return torch.full(lay.w_shape, fill, dtype=H.OUT_DT[lay.dtype], device=H.dev())


# a speech-like layer: one channel, 21x11 filters, stride (2, 1), asymmetric padding; its
# N*P*Q = 2520 positions run through ten chunks of the split-reduction kernels, and dw
# (32 x 231) is ragged against their 16- and 32-column tiles
WG_SHAPES = SMALL_SHAPES + [
    dict(name="speech_like", N=2, C=1, Hh=41, Ww=60, K=32, R=21, S=11, stride=(2, 1), pads=(10, 10, 0, 10)),
    # first layers at column stride 2 and 4 (11-wide filter rows): filter counts ragged against the
    # 3- and 7-filter tiles, rows whose input row falls in the padding, a 367-wide output row
    # spanning six 64-position groups
    dict(name="wgr_s2", N=2, C=1, Hh=30, Ww=150, K=7, R=7, S=11, stride=(2, 2), pads=(3, 3, 0, 10)),
    dict(name="wgr_s4_c3", N=2, C=3, Hh=31, Ww=70, K=10, R=5, S=11, stride=(4, 4), pads=(0, 1, 2, 0)),
    dict(name="wgr_s2_wide", N=1, C=1, Hh=21, Ww=740, K=5, R=9, S=11, stride=(2, 2), pads=(4, 4, 1, 3)),
    # 12-column output rows, 17 of them (a second, short row chunk per image), tiles ragged in k and in
    # (c, r, s), for the 12-column halo instance
    dict(name="wgh_q12_p17", N=2, C=20, Hh=17, Ww=12, K=70, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
    # 13-column rows (14-row chunks: one row past P), and 5x5 filters on 20-column rows (4-row chunks)
    dict(name="wgh_q13", N=2, C=12, Hh=13, Ww=13, K=70, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
    dict(name="wgh_q20_5x5", N=2, C=7, Hh=22, Ww=24, K=40, R=5, S=5, stride=(1, 1), pads=(1, 1, 0, 0)),
    dict(name="wgh_q27_5x5", N=2, C=5, Hh=10, Ww=27, K=70, R=5, S=5, stride=(1, 1), pads=(2, 2, 2, 2)),
    # (channel, filter row) pairs staged: 21x11 at stride (2, 1) onto 3 channels (693 columns, a
    # ragged last 32-column tile; filter count 20 ragged against 32), row stride 3 with rows in the
    # padding, and stride 1 with a 358-wide output row (the staged row is 368)
    dict(name="pairs_21x11_s2", N=2, C=3, Hh=41, Ww=120, K=20, R=21, S=11, stride=(2, 1), pads=(10, 10, 0, 10)),
    dict(name="pairs_7x11_s3", N=3, C=2, Hh=25, Ww=50, K=36, R=7, S=11, stride=(3, 1), pads=(4, 1, 3, 2)),
    dict(name="pairs_3x11_wide", N=1, C=2, Hh=6, Ww=360, K=8, R=3, S=11, stride=(1, 1), pads=(1, 1, 4, 4)),
]


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("shape", WG_SHAPES, ids=lambda s: s["name"])
def test_small_full_parity_every_variant(dtype, shape, monkeypatch):
    lay = _small(dtype=dtype, **{k: v for k, v in shape.items()})
    x64, _ = H.inputs(lay)
    N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
    dy64 = _dy(lay, (N, K, P, Q))
    ref, bound = oracle.conv2d_bwd_filter(x64, dy64, lay.w_shape, lay.stride, lay.padding)
    x = H.to_device(x64, dtype, lay.layout, lay.row_pitch)
    dy = H.to_device(dy64, dtype, lay.layout, lay.row_pitch)
    for var in WG_VARIANTS[dtype]:
        monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", var)
        print("case", shape["name"], dtype, var, flush=True)
        dw = _out(lay)
        try:
            _run(lay, x, dy, dw)
        except mic.MicError as e:
            if var.startswith(_MAY_REFUSE) and e.status == mic.MIC_STATUS_NOT_SUPPORTED:
                continue
            raise
        H.check(dtype, dw.double().cpu().numpy(), ref, bound, what="%s/%s/%s" % (shape["name"], dtype, var),
                rel_scale=H.rel_l2_scale(N * P * Q))
        monkeypatch.setenv("MIC_TILE_ORDER", "reverse")
        dw_rev = _out(lay)
        _run(lay, x, dy, dw_rev)
        monkeypatch.delenv("MIC_TILE_ORDER")
        assert torch.equal(dw, dw_rev), "%s/%s/%s: reversed tile order changed the result" % (
            shape["name"], dtype, var)
        _ran.add(var)


def test_every_wgrad_variant_was_exercised():
    want = {v for vs in WG_VARIANTS.values() for v in vs}
    assert want <= _ran, "filter-gradient variants never run: %s" % sorted(want - _ran)


def _sample(rng, w_shape, count):
    K, C, R, S = w_shape
    pts = {(k, c, r, s) for k in (0, K - 1) for c in (0, C - 1) for r in (0, R - 1) for s in (0, S - 1)}
    rnd = np.stack([rng.integers(0, K, count), rng.integers(0, C, count),
                    rng.integers(0, R, count), rng.integers(0, S, count)], axis=1)
    return np.concatenate([np.array(sorted(pts), dtype=np.int64), rnd.astype(np.int64)])


_cache = {}


def _layer_case(lay):
    """x, dy and the whole-tensor oracle dw (and bound); layouts of one logical layer share them."""
    key = (lay.config, lay.layer, lay.dtype)
    if key not in _cache:
        _cache.clear()
        x64, _ = H.inputs(lay)
        N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
        dy64 = _dy(lay, (N, K, P, Q))
        t0 = time.perf_counter()
        ref, bound = oracle.conv2d_bwd_filter(x64, dy64, lay.w_shape, lay.stride, lay.padding)
        print("  oracle %.1f s" % (time.perf_counter() - t0), flush=True)
        _cache[key] = (x64, dy64, ref, bound)
    return _cache[key]


@pytest.mark.parametrize("lay", H.full_order(workloads.ALL_LAYERS), ids=lambda l: l.name)
def test_workload_layer_full(lay):
    """Full-size filter gradient, default variant: the whole dw against the whole
    oracle output, NaN-safe beta = 0, canaries around dw, rerun bit-identity.
    The relative-L2 error without the sqrt(L / 9216) scaling of the gate is
    printed beside the scaled gate."""
    print("layer", lay.name, flush=True)
    x64, dy64, ref, bound = _layer_case(lay)
    N, K, P, Q = dy64.shape
    x = H.to_device(x64, lay.dtype, lay.layout, lay.row_pitch)
    dy = H.to_device(dy64, lay.dtype, lay.layout, lay.row_pitch)
    dw, base = H.guarded_empty(lay.w_shape, workloads.padded_strides(*lay.w_shape, "nchw", 0),
                               H.OUT_DT[lay.dtype])
    _run(lay, x, dy, dw)
    H.assert_only_tensor_written(dw, base, lay.name)
    scale = H.rel_l2_scale(N * P * Q)
    rel, worst = H.check(lay.dtype, H.to_host(dw), ref, bound, what=lay.name, rel_scale=scale)
    print("  whole tensor (%d outputs): rel-L2 %.3e (gate %.2e = %.0e x %.2f), worst |err|/B %.3e"
          % (ref.size, rel, H.RELL2[lay.dtype] * (scale if lay.dtype != "f64" else 1.0), H.RELL2[lay.dtype],
             scale if lay.dtype != "f64" else 1.0, worst), flush=True)
    dw2 = _out(lay, fill=0.0)
    _run(lay, x, dy, dw2)
    assert torch.equal(dw, dw2), "rerun not bit-identical"


@pytest.mark.parametrize("lay", workloads.ALL_LAYERS, ids=lambda l: l.name)
def test_workload_layer_integer_exact(lay):
    """Integer x and dy in [-4, 4]: |partial sums| <= 16 * N*P*Q < 2^24, all exact."""
    print("layer", lay.name, flush=True)
    x64, _ = H.inputs(lay, ("integers", -4, 4), ("integers", -4, 4))
    N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
    assert 16 * N * P * Q < 2 ** 24
    dy64 = _dy(lay, (N, K, P, Q), integer=True)
    x = H.to_device(x64, lay.dtype, lay.layout, lay.row_pitch)
    dy = H.to_device(dy64, lay.dtype, lay.layout, lay.row_pitch)
    dw = _out(lay)
    _run(lay, x, dy, dw)
    rng = np.random.default_rng(lay.config * 1000 + lay.layer + 53)
    idx = _sample(rng, lay.w_shape, 200)
    ref, _ = oracle.conv2d_bwd_filter_at(x64, dy64, lay.w_shape, idx, lay.stride, lay.padding)
    got = H.gather(dw, idx)
    assert np.array_equal(got, ref), "%s: %d mismatches" % (lay.name, int((got != ref).sum()))


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("geom", [((1, 2), (1, 1, 1, 0)), ((1, 1), (1, 1, 1, 1))], ids=["s12", "s11"])
def test_alpha_beta(dtype, geom, monkeypatch):
    lay = _small("wg_ab", 2, 20, 13, 11, 36, 3, 3, geom[0], geom[1], dtype)
    xi, _ = H.inputs(lay, ("integers", -4, 4), ("integers", -4, 4))
    N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
    dyi = _dy(lay, (N, K, P, Q), integer=True)
    acc, _ = oracle.conv2d_bwd_filter(xi, dyi, lay.w_shape, lay.stride, lay.padding)
    old = gen.integers(97, acc.shape)
    x = H.to_device(xi, dtype)
    dy = H.to_device(dyi, dtype)
    for var in WG_VARIANTS[dtype]:
        monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", var)
        dw = torch.from_numpy(old).to(H.OUT_DT[dtype]).to(H.dev())
        try:
            _run(lay, x, dy, dw, alpha=0.5, beta=0.25)
        except mic.MicError as e:
            if var.startswith(_MAY_REFUSE) and e.status == mic.MIC_STATUS_NOT_SUPPORTED:
                continue
            raise
        assert np.array_equal(dw.double().cpu().numpy(), 0.5 * acc + 0.25 * old), var


@pytest.mark.parametrize("stride", [(2, 2), (1, 4)], ids=["s2", "s14"])
def test_alpha_beta_first_layer_kernels(stride, monkeypatch):
    """The vector-ALU first-layer kernels: y = alpha * sum + beta * y exactly on integer data."""
    lay = _small("wgr_ab", 2, 2, 9, 80, 9, 3, 11, stride, (1, 1, 0, 3), "f32")
    xi, _ = H.inputs(lay, ("integers", -4, 4), ("integers", -4, 4))
    N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
    dyi = _dy(lay, (N, K, P, Q), integer=True)
    acc, _ = oracle.conv2d_bwd_filter(xi, dyi, lay.w_shape, lay.stride, lay.padding)
    old = gen.integers(97, acc.shape)
    var = "wgr_f32_s11_v2" if stride[1] == 2 else "wgr_f32_s11_v4"
    monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", var)
    dw = torch.from_numpy(old).to(torch.float32).to(H.dev())
    _run(lay, H.to_device(xi, "f32"), H.to_device(dyi, "f32"), dw, alpha=0.5, beta=0.25)
    assert np.array_equal(dw.double().cpu().numpy(), 0.5 * acc + 0.25 * old), var


# the halo kernel's reduction in two parts (beta = 0, tiles that leave compute units idle in one
# round): AlexNet conv2's geometry at N = 2 makes 200 tiles of 64 x 48 (long parts 4/5 of the 14
# chunks), 152 of 64 x 64 (2/3); the 3x3 layer 216 tiles of 64 x 64 (6/7)
SPLIT_CASES = [
    ("conv2_n2", dict(N=2, C=96, Hh=27, Ww=27, K=256, R=5, S=5, stride=(1, 1), pads=(2, 2, 2, 2)),
     ["auto", "wgh_f32x16_5x5_q27_64x48", "wgh_f32x16_5x5_q27_64x64", "wgh_f32x16_5x5_q27_64x48_ks4"]),
    ("conv3_n2", dict(N=2, C=256, Hh=13, Ww=13, K=384, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
     ["auto", "wgh_f32_3x3_q13_64x64", "wgh_f32_3x3_q13_64x64_ks4", "wgh_f32_3x3_64x96_ks4"]),
    ("conv3_n2_f64", dict(N=2, C=256, Hh=13, Ww=13, K=384, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
     ["auto", "wgh_f64_3x3_64x64_ks4", "wgh_f64_3x3_64x96"]),
    ("conv3_n2_bf16", dict(N=2, C=256, Hh=13, Ww=13, K=384, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
     ["auto", "wgh_bf16_3x3_q13_64x64", "wgh_bf16_3x3_64x96_ks4"]),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: c[0])
def test_split_reduction(case, monkeypatch):
    """Two reduction parts added atomically into a zeroed dw: the same tolerance against the
    oracle as one part, bit-identical with the tiles reversed and on a rerun (two terms onto zero
    commute), and exact on integer data with alpha = 0.5."""
    name, shape, variants = case
    dtype = name.rsplit("_", 1)[1] if name.endswith(("f64", "bf16")) else "f32"
    lay = _small(name, **shape, dtype=dtype)
    x64, _ = H.inputs(lay)
    N, K, P, Q = mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding)
    dy64 = _dy(lay, (N, K, P, Q))
    ref, bound = oracle.conv2d_bwd_filter(x64, dy64, lay.w_shape, lay.stride, lay.padding)
    x = H.to_device(x64, dtype)
    dy = H.to_device(dy64, dtype)
    xi64, _ = H.inputs(lay, ("integers", -4, 4), ("integers", -4, 4))
    dyi64 = _dy(lay, (N, K, P, Q), integer=True)
    acc_i, _ = oracle.conv2d_bwd_filter(xi64, dyi64, lay.w_shape, lay.stride, lay.padding)
    xi = H.to_device(xi64, dtype)
    dyi = H.to_device(dyi64, dtype)
    for var in variants:
        if var == "auto":
            monkeypatch.delenv("MIC_FORCE_WGRAD_VARIANT", raising=False)
        else:
            monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", var)
        print("case", name, var, flush=True)
        what = "%s/%s" % (name, var)
        monkeypatch.setenv("MIC_WGRAD_SPLIT", "off")
        one = _run(lay, x, dy, _out(lay))
        monkeypatch.delenv("MIC_WGRAD_SPLIT")
        two = _run(lay, x, dy, _out(lay))
        for got, how in ((one, "one part"), (two, "two parts")):
            H.check(dtype, got.double().cpu().numpy(), ref, bound, what=what + " " + how,
                    rel_scale=H.rel_l2_scale(N * P * Q))
        assert not torch.equal(one, two) or var == "auto", what + ": the split changed no bit (not taken?)"
        monkeypatch.setenv("MIC_TILE_ORDER", "reverse")
        rev = _run(lay, x, dy, _out(lay))
        monkeypatch.delenv("MIC_TILE_ORDER")
        assert torch.equal(two, rev), what + ": reversed tile order changed the two-part result"
        assert torch.equal(two, _run(lay, x, dy, _out(lay))), what + ": rerun not bit-identical"
        dw = _run(lay, xi, dyi, _out(lay), alpha=0.5)
        assert np.array_equal(dw.double().cpu().numpy(), 0.5 * acc_i), what + ": integer data not exact"


def test_wgrad_error_statuses_on_device():
    lay = workloads.TINY[0]
    x = torch.zeros(lay.x_shape, device=H.dev())
    dy = torch.zeros((2, 16, 12, 11), device=H.dev())          # forward output is 12 x 12
    dw = torch.zeros(lay.w_shape, device=H.dev())
    with pytest.raises(mic.MicError) as e:
        mic.conv2d_backward_filter(x, dy, lay.w_shape, lay.stride, lay.padding, dw=dw)
    assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    dy = torch.zeros((2, 16, 12, 12), device=H.dev())
    plan = mic.WgradPlan(x, dy, dw, lay.stride, lay.padding)
    try:
        with pytest.raises(mic.MicError) as e:                   # null dw pointer
            mic.mic_conv_backward_filter(plan.handle, 1.0, plan.xd, x.data_ptr(), plan.dyd, dy.data_ptr(),
                                         plan.cd, 0.0, plan.wd, 0)
        assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    finally:
        plan.close()

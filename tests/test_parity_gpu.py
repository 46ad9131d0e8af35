"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small shapes that span several tiles with ragged tails are compared element
by element in full, for every kernel variant, in the normal tile order and
with the tiles run in reverse (the result must not change by a bit); every
workload layer is run at its full size and its whole output is compared with
the whole oracle output (relative L2 over the tensor and the per-element
bound on every element), plus properties that hold at any size:
integer-valued inputs give bit-exact results over the whole tensor, reruns
are bit-identical, NaN in y never leaks when beta = 0, and nothing outside y
is written (canary cells directly before and after y, and the pad cells of
padded rows, stay untouched).
"""
import time
import os

import numpy as np
import pytest
import torch

import convolution_forward_conv2d_amd as mic
import gen
import oracle
from gen import workloads
from gen.workloads import Layer

import gpu_harness as H

pytestmark = pytest.mark.gpu

VARIANTS = {
    "f32": ["direct", "mfma_f32_128x128", "mfma_f32_128x64", "mfma_f32_64x128", "mfma_f32_256x32",
            "halo_f32_3x3_128x128", "halo_f32_3x3_128x64", "halo_f32_3x3_64x128", "halo_f32_3x3_96x128",
            "halo_f32_5x5_128x128", "halo_f32_5x5_128x128_c2", "halo_f32x16_3x3_176x128",
            "halo_f32x16_3x3_144x128", "halo_f32x16_5x5_128x96", "halo_f32_5x5_128x96_c2",
            "halo_f32x16_5x5_208x64",
            "halo_f32x16_3x3_176x128_ks2",
            "halo_f32_3x3_128x128_ks2"],
    "f64": ["direct", "mfma_f64_128x128", "mfma_f64_128x64", "mfma_f64_64x64",
            "halo_f64_3x3_128x128", "halo_f64_3x3_64x64", "halo_f64_3x3_128x64",
            "halo_f64_3x3_176x64_ks2"],
    "bf16": ["direct", "mfma_bf16_128x128", "mfma_bf16_128x64", "mfma_bf16_256x32",
             "halo_bf16_3x3_128x128", "halo_bf16_3x3_128x64", "halo_bf16_3x3_192x128"],
}
# the gather variants also run with the reduction in channel blocks per filter tap
for _dt in VARIANTS:
    VARIANTS[_dt] += [v + "_tap" for v in VARIANTS[_dt] if v.startswith("mfma_")]
# the reduction streamed by filter row: 11-wide filters, 8-channel blocks, Q >= 256
VARIANTS["f32"] += ["rows_f32_s11_256x32", "rows1_f32_s11_256x32", "rows1n6_f32_s11_256x32"]
_MAY_REFUSE = ("halo_", "rows_", "rows1_", "rows1n6_")
# halo variants only take the shapes they were built for (the library answers
# NOT_SUPPORTED otherwise); every one of them must run on at least one shape
_ran = set()

U = ("uniform", -1.0, 1.0)


def _small(name, N, C, Hh, Ww, K, R, S, stride, pads, dtype, layout="nchw", pitch=0):
    return Layer(name, 9, 1, N, C, Hh, Ww, K, R, S, stride, pads, dtype, U, U,
                 layout=layout, row_pitch=pitch)


SMALL_SHAPES = [
    # several 128-row tiles plus a ragged tail; K = 100 is ragged against every n-tile
    dict(name="ragged3x3", N=3, C=40, Hh=15, Ww=15, K=100, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
    # 11x11 / stride 4 / no padding, K = 96, C*R*S = 363 (odd)
    dict(name="big_filter", N=2, C=3, Hh=63, Ww=63, K=96, R=11, S=11, stride=(4, 4), pads=(0, 0, 0, 0)),
    # non-square filter, mixed stride, asymmetric padding
    dict(name="asym", N=2, C=5, Hh=33, Ww=70, K=33, R=7, S=5, stride=(2, 1), pads=(3, 2, 0, 4)),
    # channels-last storage
    dict(name="nhwc", N=2, C=64, Hh=13, Ww=13, K=64, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1),
         layout="nhwc"),
    # padded row pitch (16) on x and y
    dict(name="pitch16", N=2, C=24, Hh=13, Ww=13, K=40, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1),
         pitch=16),
    # one output element per image, one channel
    dict(name="degenerate", N=5, C=1, Hh=3, Ww=2, K=3, R=3, S=2, stride=(3, 3), pads=(0, 0, 0, 0)),
    # 3x3 on 13x13: several ragged m tiles (M = 507), images straddling tiles, K = 100
    dict(name="halo3", N=3, C=20, Hh=13, Ww=13, K=100, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
    # 3x3, stride 2 along H, asymmetric padding (only the 64-row tiles fit its slot span)
    dict(name="halo3_strided", N=2, C=8, Hh=12, Ww=11, K=40, R=3, S=3, stride=(2, 1), pads=(1, 0, 2, 1)),
    # one channel block only: with the reduction split in two, the second half has no work
    dict(name="halo3_c4", N=1, C=4, Hh=13, Ww=13, K=16, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
    # 5x5 / pad 2 on 20x20
    dict(name="halo5", N=2, C=8, Hh=20, Ww=20, K=70, R=5, S=5, stride=(1, 1), pads=(2, 2, 2, 2)),
    # whole 16-channel blocks (bf16 halo kernel): three blocks, ragged m and K tiles
    dict(name="halo3_c48", N=3, C=48, Hh=13, Ww=13, K=100, R=3, S=3, stride=(1, 1), pads=(1, 1, 1, 1)),
    # channels-last with a padded row pitch: 16-byte channel loads of x
    dict(name="halo3_nhwc_pitch", N=2, C=32, Hh=13, Ww=13, K=72, R=3, S=3, stride=(1, 1),
         pads=(1, 1, 1, 1), layout="nhwc", pitch=16),
    # one 16-channel block, stride 2, asymmetric padding, non-square input
    dict(name="halo3_c16_s2", N=2, C=16, Hh=14, Ww=12, K=40, R=3, S=3, stride=(2, 2), pads=(1, 0, 1, 1)),
    # NCHW rows on a 16-element pitch: bf16 rows loaded 8 pixels at a time (a whole and a
    # 5-pixel segment per row; the tensor's last row read pixel by pixel), two channel blocks
    dict(name="halo3_c32_pitch16", N=3, C=32, Hh=13, Ww=13, K=72, R=3, S=3, stride=(1, 1),
         pads=(1, 1, 1, 1), pitch=16),
    # ... 8-pixel rows (one whole segment) with asymmetric padding
    dict(name="halo3_w8_pitch16", N=2, C=16, Hh=9, Ww=8, K=40, R=3, S=3, stride=(1, 1),
         pads=(0, 2, 2, 0), pitch=16),
]


def _run(lay, x, w, y, alpha=1.0, beta=0.0):
    plan = mic.ConvPlan(x, w, y, lay.stride, lay.padding)
    try:
        plan(alpha, beta)
        torch.cuda.synchronize()
    finally:
        plan.close()
    return y


# forward-only shapes for the row-streamed kernel: a 5x11 filter bank with a ragged second
# filter tile (K = 40) and a ragged last position tile; a speech-like 21x11 bank, stride (2, 1),
# padding on three sides, output rows 260 wide (a tile straddles two of them)
FWD_SHAPES = SMALL_SHAPES + [
    dict(name="rows_5x11", N=2, C=16, Hh=25, Ww=270, K=40, R=5, S=11, stride=(2, 1), pads=(2, 2, 0, 10)),
    dict(name="rows_21x11", N=1, C=8, Hh=41, Ww=260, K=32, R=21, S=11, stride=(2, 1), pads=(10, 10, 0, 10)),
    # an odd row width and left pad: the halo loads one column at a time (rows_5x11 and
    # rows_21x11 load 2 and 4)
    dict(name="rows_5x11_odd", N=2, C=8, Hh=21, Ww=271, K=40, R=5, S=11, stride=(1, 1), pads=(2, 2, 1, 9)),
    # one input channel (adjacent taps paired): speech-like 41x11 / (2, 2) with padding on three
    # sides and K = 40 (a ragged filter tile); 7 filter rows (the last chunk of 4 half empty)
    dict(name="rows1_41x11", N=1, C=1, Hh=61, Ww=530, K=40, R=41, S=11, stride=(2, 2), pads=(20, 20, 0, 10)),
    dict(name="rows1_7x11", N=2, C=1, Hh=15, Ww=270, K=32, R=7, S=11, stride=(1, 1), pads=(3, 3, 5, 5)),
    # 1-4 channels, short output rows (six slots): Overfeat-like 11x11 / 4 on 3 channels with K = 96,
    # and 2 channels, 9 filter rows, padding on every side
    dict(name="rows1n6_c3_s4", N=2, C=3, Hh=71, Ww=231, K=96, R=11, S=11, stride=(4, 4), pads=(0, 0, 0, 0)),
    dict(name="rows1n6_c2", N=2, C=2, Hh=20, Ww=60, K=40, R=9, S=11, stride=(1, 1), pads=(2, 3, 4, 1)),
    # odd stride 3
    dict(name="rows1n6_c3_s3", N=2, C=3, Hh=40, Ww=160, K=20, R=5, S=11, stride=(3, 3), pads=(1, 1, 2, 2)),
    # stride 4 with padding on three sides, an odd output row width (Q = 53), a ragged last
    # tile and filter tile
    dict(name="rows1n6_s4_pad", N=3, C=2, Hh=45, Ww=217, K=40, R=11, S=11, stride=(4, 4), pads=(2, 0, 1, 2)),
]


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=lambda s: s["name"])
def test_small_full_parity_every_variant(dtype, shape, monkeypatch):
    lay = _small(dtype=dtype, **{k: v for k, v in shape.items()})
    x64, w64 = H.inputs(lay)
    ref, bound = oracle.conv2d_fprop(x64, w64, lay.stride, lay.padding)
    x = H.to_device(x64, dtype, lay.layout, lay.row_pitch)
    w = torch.from_numpy(w64).to(H.TORCH_DT[dtype]).to(H.dev())
    for var in VARIANTS[dtype]:
        monkeypatch.setenv("MIC_FORCE_VARIANT", var)
        print("case", shape["name"], dtype, var, flush=True)
        y = H.out_tensor(lay, ref.shape)
        try:
            _run(lay, x, w, y)
        except mic.MicError as e:
            if var.startswith(_MAY_REFUSE) and e.status == mic.MIC_STATUS_NOT_SUPPORTED:
                continue
            raise
        H.check(dtype, y.double().cpu().numpy(), ref, bound, what="%s/%s/%s" % (shape["name"], dtype, var))
        # the same tiles in reverse order: any dependence between workgroups
        # or race on LDS shows as a changed bit
        monkeypatch.setenv("MIC_TILE_ORDER", "reverse")
        y_rev = H.out_tensor(lay, ref.shape)
        _run(lay, x, w, y_rev)
        monkeypatch.delenv("MIC_TILE_ORDER")
        assert torch.equal(y, y_rev), "%s/%s/%s: reversed tile order changed the result" % (
            shape["name"], dtype, var)
        _ran.add(var)


def test_every_variant_was_exercised():
    want = {v for vs in VARIANTS.values() for v in vs}
    assert want <= _ran, "variants never run: %s" % sorted(want - _ran)


def test_tiny_workload_full_and_deterministic():
    lay = workloads.TINY[0]
    x64, w64 = H.inputs(lay)
    ref, bound = oracle.conv2d_fprop(x64, w64, lay.stride, lay.padding)
    x = H.to_device(x64, "f32")
    w = torch.from_numpy(w64).float().to(H.dev())
    y1 = _run(lay, x, w, H.out_tensor(lay, ref.shape))
    y2 = _run(lay, x, w, H.out_tensor(lay, ref.shape))
    H.check("f32", y1.double().cpu().numpy(), ref, bound, what="tiny")
    assert torch.equal(y1, y2)


_cache = {}


def _layer_case(lay, integer=False):
    """Inputs and the whole-tensor oracle output (y, bound) of a workload layer.
    The layouts of one logical layer share them (same generated values)."""
    key = (lay.config, lay.layer, lay.dtype, integer)
    if key not in _cache:
        _cache.clear()
        dist = ("integers", -4, 4) if integer else None
        x64, w64 = H.inputs(lay, dist, dist)
        t0 = time.perf_counter()
        ref, bound = oracle.conv2d_fprop(x64, w64, lay.stride, lay.padding)
        print("  oracle %.1f s" % (time.perf_counter() - t0), flush=True)
        _cache[key] = (x64, w64, ref, bound)
    return _cache[key]


FULL_LAYERS = H.full_order(workloads.ALL_LAYERS)


@pytest.mark.parametrize("lay", FULL_LAYERS, ids=lambda l: l.name)
def test_workload_layer_full(lay):
    """Full-size layer, default variant, whole output against the whole oracle
    output; NaN-prefilled y fully overwritten (beta = 0), canaries around y
    untouched, rerun bit-identical."""
    print("layer", lay.name, flush=True)
    x64, w64, ref, bound = _layer_case(lay)
    x = H.to_device(x64, lay.dtype, lay.layout, lay.row_pitch)
    w = torch.from_numpy(w64).to(H.TORCH_DT[lay.dtype]).to(H.dev())
    y, base = H.guarded_out(lay, ref.shape)
    _run(lay, x, w, y)
    H.assert_only_tensor_written(y, base, lay.name)
    rel, worst = H.check(lay.dtype, H.to_host(y), ref, bound, what=lay.name)
    print("  whole tensor (%d outputs): rel-L2 %.3e, worst |err|/B %.3e" % (ref.size, rel, worst), flush=True)
    y2 = H.out_tensor(lay, ref.shape, fill=0.0)
    _run(lay, x, w, y2)
    assert torch.equal(y, y2), "rerun not bit-identical"


@pytest.mark.parametrize("lay", FULL_LAYERS, ids=lambda l: l.name)
def test_workload_layer_integer_exact(lay):
    """Integer inputs in [-4, 4]: every partial sum is an exact integer below 2^24,
    so the whole output must equal the oracle's bit for bit, in every layout."""
    print("layer", lay.name, flush=True)
    x64, w64, ref, _ = _layer_case(lay, integer=True)
    x = H.to_device(x64, lay.dtype, lay.layout, lay.row_pitch)
    w = torch.from_numpy(w64).to(H.TORCH_DT[lay.dtype]).to(H.dev())
    y = H.out_tensor(lay, ref.shape)
    _run(lay, x, w, y)
    got = H.to_host(y)
    assert np.array_equal(got, ref), "%s: %d mismatches" % (lay.name, int((got != ref).sum()))


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("geom", [(11, 9, 3, 2, (1, 2), (1, 0, 2, 1)), (13, 13, 3, 3, (1, 1), (1, 1, 1, 1))],
                         ids=["3x2", "3x3"])
def test_alpha_beta(dtype, geom, monkeypatch):
    Hh, Ww, R, S, stride, pads = geom
    lay = _small("ab", 2, 20, Hh, Ww, 70, R, S, stride, pads, dtype)
    xi, wi = H.inputs(lay, ("integers", -4, 4), ("integers", -4, 4))
    acc, _ = oracle.conv2d_fprop(xi, wi, lay.stride, lay.padding)
    y_old = gen.integers(99, acc.shape)
    x = H.to_device(xi, dtype)
    w = torch.from_numpy(wi).to(H.TORCH_DT[dtype]).to(H.dev())
    for var in VARIANTS[dtype]:
        monkeypatch.setenv("MIC_FORCE_VARIANT", var)
        y = torch.from_numpy(y_old).to(H.OUT_DT[dtype]).to(H.dev())
        try:
            _run(lay, x, w, y, alpha=0.5, beta=0.25)
        except mic.MicError as e:
            if var.startswith(_MAY_REFUSE) and e.status == mic.MIC_STATUS_NOT_SUPPORTED:
                continue
            raise
        assert np.array_equal(y.double().cpu().numpy(), 0.5 * acc + 0.25 * y_old), var
        y = torch.from_numpy(y_old).to(H.OUT_DT[dtype]).to(H.dev())
        _run(lay, x, w, y, alpha=0.0, beta=-2.0)
        assert np.array_equal(y.double().cpu().numpy(), -2.0 * y_old), var
    # non-integer values with the tolerance of the type
    monkeypatch.delenv("MIC_FORCE_VARIANT")
    x64, w64 = H.inputs(lay)
    yo = gen.round_to(gen.uniform(98, acc.shape), "f32" if dtype != "f64" else "f64")
    ref, bound = oracle.conv2d_fprop(x64, w64, lay.stride, lay.padding, alpha=-2.0, beta=1.0, y_old=yo)
    y = torch.from_numpy(yo).to(H.OUT_DT[dtype]).to(H.dev())
    _run(lay, H.to_device(x64, dtype), torch.from_numpy(w64).to(H.TORCH_DT[dtype]).to(H.dev()), y,
         alpha=-2.0, beta=1.0)
    H.check(dtype, y.double().cpu().numpy(), ref, bound, alpha=-2.0, beta=1.0, y_old=yo, what="alpha-beta")


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
def test_subtensor_output_and_canaries(layout):
    """y is a channel slice of a larger tensor: neighbours and guard cells stay untouched."""
    lay = _small("sub", 3, 16, 14, 14, 50, 3, 3, (1, 1), (1, 1, 1, 1), "f32", layout=layout)
    x64, w64 = H.inputs(lay)
    ref, bound = oracle.conv2d_fprop(x64, w64, lay.stride, lay.padding)
    N, K, P, Q = ref.shape
    # the parent tensor (K + 9 channels) sits in one allocation between canary cells
    st = workloads.padded_strides(N, K + 9, P, Q, layout, 0)
    big, base = H.guarded_empty((N, K + 9, P, Q), st, torch.float32)
    big.fill_(7.25)
    y = big[:, 4:4 + K]
    x = H.to_device(x64, "f32", layout)
    w = torch.from_numpy(w64).float().to(H.dev())
    _run(lay, x, w, y)
    H.check("f32", y.double().cpu().numpy(), ref, bound, what="subtensor")
    assert bool((big[:, :4] == 7.25).all()) and bool((big[:, 4 + K:] == 7.25).all())
    assert bool(torch.isnan(base[:H.GUARD]).all()) and bool(torch.isnan(base[-H.GUARD:]).all())


def test_nondefault_stream():
    lay = _small("stream", 2, 32, 13, 13, 64, 3, 3, (1, 1), (1, 1, 1, 1), "f32")
    x64, w64 = H.inputs(lay)
    ref, bound = oracle.conv2d_fprop(x64, w64, lay.stride, lay.padding)
    s = torch.cuda.Stream()
    x = H.to_device(x64, "f32")
    w = torch.from_numpy(w64).float().to(H.dev())
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = mic.conv2d_forward(x, w, lay.stride, lay.padding)
    s.synchronize()
    H.check("f32", y.double().cpu().numpy(), ref, bound, what="stream")


def test_error_statuses_on_device():
    h = mic.handle_for()
    lay = workloads.TINY[0]
    x = torch.zeros(lay.x_shape, device=H.dev())
    w = torch.zeros(lay.w_shape, device=H.dev())
    y = torch.zeros((2, 16, 12, 12), device=H.dev())
    plan = mic.ConvPlan(x, w, y, lay.stride, lay.padding, handle=h)
    try:
        with pytest.raises(mic.MicError) as e:            # null input pointer
            mic.mic_conv_forward(h, 1.0, plan.xd, 0, plan.wd, w.data_ptr(), plan.cd, 0.0, plan.yd,
                                 y.data_ptr())
        assert e.value.status == mic.MIC_STATUS_BAD_PARAM
        with pytest.raises(mic.MicError) as e:            # misaligned output pointer
            mic.mic_conv_forward(h, 1.0, plan.xd, x.data_ptr(), plan.wd, w.data_ptr(), plan.cd, 0.0,
                                 plan.yd, y.data_ptr() + 2)
        assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    finally:
        plan.close()


def test_no_device_memory_allocated_by_calls():
    lay = workloads.by_name("alexnet_conv3")
    lay = Layer("nomem", 2, 3, 8, lay.C, lay.H, lay.W, lay.K, lay.R, lay.S, lay.stride, lay.padding,
                "f32", U, U)
    x = torch.randn(lay.x_shape, device=H.dev())
    w = torch.randn(lay.w_shape, device=H.dev())
    y = torch.empty((8, lay.K, 13, 13), device=H.dev())
    plan = mic.ConvPlan(x, w, y, lay.stride, lay.padding)
    plan()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(20):
        plan()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    plan.close()
    assert free1 == free0

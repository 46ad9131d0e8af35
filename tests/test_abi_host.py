"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function miconv.h declares, validates descriptors and computes output sizes
the same way the oracle does.  No kernel is launched here."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import convolution_forward_conv2d_amd as mic
import oracle
from gen import workloads
from gen.workloads import Layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "convolution_forward_conv2d_amd", "csrc")


def test_library_exports_every_declared_function():
    names = mic.header_functions()
    assert "mic_conv_forward" in names and len(names) >= 20
    lib = mic.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # every declared function has a Python wrapper of the same name
    assert not [n for n in names if not hasattr(mic, n)]


def test_status_strings_and_version():
    assert mic.status_string(0) == "success"
    assert mic.status_string(1) == "bad parameter"
    assert mic.status_string(2) == "not supported"
    assert mic.status_string(99) == "unknown status"
    assert mic.mic_get_version() == (0, 1, 0)


def test_tensor_descriptor_roundtrip_and_validation():
    d = mic.mic_tensor_desc_create()
    try:
        with pytest.raises(mic.MicError) as e:
            mic.mic_tensor_desc_get(d)            # never set
        assert e.value.status == mic.MIC_STATUS_BAD_PARAM
        mic.mic_tensor_desc_set(d, mic.MIC_DTYPE_F32, 2, 3, 4, 5, 60, 20, 5, 1)
        assert mic.mic_tensor_desc_get(d) == (0, (2, 3, 4, 5), (60, 20, 5, 1))
        mic.mic_tensor_desc_set_packed(d, mic.MIC_DTYPE_BF16, mic.MIC_LAYOUT_NHWC, 2, 3, 4, 5)
        assert mic.mic_tensor_desc_get(d) == (2, (2, 3, 4, 5), (60, 1, 15, 3))
        for bad in [(0, 3, 4, 5, 1, 1, 1, 1), (2, 3, 4, 5, 0, 1, 1, 1), (2, 3, 4, 5, 1, 1, -2, 1),
                    (2, -1, 4, 5, 1, 1, 1, 1)]:
            with pytest.raises(mic.MicError) as e:
                mic.mic_tensor_desc_set(d, mic.MIC_DTYPE_F32, *bad)
            assert e.value.status == mic.MIC_STATUS_BAD_PARAM
        with pytest.raises(mic.MicError):
            mic.mic_tensor_desc_set(d, 7, 1, 1, 1, 1, 1, 1, 1, 1)      # unknown dtype
    finally:
        mic.mic_tensor_desc_destroy(d)


def test_filter_and_conv_descriptor_validation():
    f = mic.mic_filter_desc_create()
    c = mic.mic_conv_desc_create()
    try:
        mic.mic_filter_desc_set(f, mic.MIC_DTYPE_F64, 4, 3, 2, 1)
        assert mic.mic_filter_desc_get(f) == (1, (4, 3, 2, 1))
        with pytest.raises(mic.MicError):
            mic.mic_filter_desc_set(f, mic.MIC_DTYPE_F32, 4, 0, 2, 1)
        mic.mic_conv_desc_set(c, 1, 2, 3, 4, 5, 6)
        assert mic.mic_conv_desc_get(c) == (1, 2, 3, 4, 5, 6)
        for bad in [(-1, 0, 0, 0, 1, 1), (0, 0, 0, -1, 1, 1), (0, 0, 0, 0, 0, 1), (0, 0, 0, 0, 1, -1)]:
            with pytest.raises(mic.MicError):
                mic.mic_conv_desc_set(c, *bad)
    finally:
        mic.mic_filter_desc_destroy(f)
        mic.mic_conv_desc_destroy(c)


def test_null_arguments_are_bad_param():
    l = mic.lib()
    assert l.mic_destroy(None) == mic.MIC_STATUS_BAD_PARAM
    assert l.mic_tensor_desc_destroy(None) == mic.MIC_STATUS_BAD_PARAM
    assert l.mic_set_stream(None, None) == mic.MIC_STATUS_BAD_PARAM
    assert l.mic_conv_forward(None, 1.0, None, None, None, None, None, 0.0, None, None) == \
        mic.MIC_STATUS_BAD_PARAM
    buf = ctypes.create_string_buffer(8)
    assert l.mic_conv_forward_kernel_name(None, None, None, None, None, buf, 8) == mic.MIC_STATUS_BAD_PARAM


@pytest.mark.parametrize("lay", workloads.ALL_LAYERS, ids=lambda l: l.name)
def test_output_dims_match_oracle(lay):
    pb = oracle.make_problem(lay.x_shape, (1, 1, 1, 1), lay.w_shape, lay.stride, lay.padding)
    P, Q = oracle.output_dims(pb)
    assert mic.output_shape(lay.x_shape, lay.w_shape, lay.stride, lay.padding) == (lay.N, lay.K, P, Q)


def test_output_dims_errors():
    with pytest.raises(mic.MicError) as e:        # channel mismatch
        mic.output_shape((1, 3, 8, 8), (2, 4, 3, 3))
    assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    with pytest.raises(mic.MicError):             # filter larger than padded input
        mic.output_shape((1, 1, 3, 3), (1, 1, 5, 1), (1, 1), (0, 1, 0, 0))
    # exactly fitting after padding is fine: one output row
    assert mic.output_shape((1, 1, 3, 3), (1, 1, 5, 1), (1, 1), (1, 1, 0, 0)) == (1, 1, 1, 3)


def _descs(lay, x_dt, w_dt, y_dt, y_dims=None):
    xd, wd, yd, cd = (mic.mic_tensor_desc_create(), mic.mic_filter_desc_create(),
                      mic.mic_tensor_desc_create(), mic.mic_conv_desc_create())
    xs = workloads.padded_strides(lay.N, lay.C, lay.H, lay.W, lay.layout, lay.row_pitch)
    mic.mic_tensor_desc_set(xd, x_dt, *lay.x_shape, *xs)
    mic.mic_filter_desc_set(wd, w_dt, *lay.w_shape)
    mic.mic_conv_desc_set(cd, *lay.padding, *lay.stride)
    N, K, P, Q = mic.mic_conv_forward_output_dim(cd, xd, wd) if y_dims is None else y_dims
    mic.mic_tensor_desc_set_packed(yd, y_dt, mic.MIC_LAYOUT_NCHW, N, K, P, Q)
    return xd, wd, cd, yd


def _free(xd, wd, cd, yd):
    mic.mic_tensor_desc_destroy(xd)
    mic.mic_filter_desc_destroy(wd)
    mic.mic_conv_desc_destroy(cd)
    mic.mic_tensor_desc_destroy(yd)


def test_kernel_choice_host_only():
    F32 = mic.MIC_DTYPE_F32
    names = {}
    for lay in workloads.ALL_LAYERS:
        dt = {"f32": (F32, F32, F32), "f64": (1, 1, 1), "bf16": (2, 2, F32)}[lay.dtype]
        d = _descs(lay, *dt)
        try:
            names[lay.name] = mic.mic_conv_forward_kernel_name(None, *d)
        finally:
            _free(*d)
    for name in ("alexnet_conv3", "alexnet_conv4", "alexnet_conv5", "overfeat_l3", "overfeat_l4",
                 "overfeat_l5"):
        assert names[name].startswith(("halo_f32_3x3_", "halo_f32x16_3x3_")), (name, names[name])
    assert names["alexnet_conv2"].startswith("halo_f32_5x5_")
    # 20x20 outputs, 256 filters: 208-row x 64-filter tiles on 16x16 blocks (988 tiles, about four per CU)
    assert names["overfeat_l2"] == "halo_f32x16_5x5_208x64"
    assert names["overfeat_l1"] == "rows1n6_f32_s11_256x32"      # 3 channels, 56-wide output rows
    # 21x11 filters, 32 filters, Q = 350 >= the 256-position tile: reduction streamed by filter row
    assert names["speech_l2"] == "rows_f32_s11_256x32"
    assert names["speech_l1"] == "rows1_f32_s11_256x32"         # one channel: adjacent taps paired
    assert names["prec_conv3_f64_nchw"].startswith("halo_f64_3x3_")
    assert names["prec_conv3_bf16_nhwc"].startswith("halo_bf16_3x3_")
    assert names["prec_conv5_bf16_nchw"].startswith("halo_bf16_3x3_")


def test_dtype_combinations_and_shape_mismatch():
    lay = workloads.TINY[0]
    for combo in [(0, 0, 1), (1, 1, 0), (2, 2, 2), (0, 2, 0)]:
        d = _descs(lay, *combo)
        try:
            with pytest.raises(mic.MicError) as e:
                mic.mic_conv_forward_kernel_name(None, *d)
            assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
        finally:
            _free(*d)
    d = _descs(lay, 0, 0, 0, y_dims=(2, 16, 12, 11))
    try:
        with pytest.raises(mic.MicError) as e:
            mic.mic_conv_forward_kernel_name(None, *d)
        assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    finally:
        _free(*d)


def test_forced_variant_must_match_dtype(monkeypatch):
    lay = workloads.TINY[0]
    monkeypatch.setenv("MIC_FORCE_VARIANT", "mfma_f64_64x64")
    d = _descs(lay, 0, 0, 0)
    try:
        with pytest.raises(mic.MicError) as e:
            mic.mic_conv_forward_kernel_name(None, *d)
        assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
        monkeypatch.setenv("MIC_FORCE_VARIANT", "direct")
        assert mic.mic_conv_forward_kernel_name(None, *d) == "direct"
    finally:
        _free(*d)


def test_size_limit_is_not_supported():
    d = mic.mic_tensor_desc_create()
    wd, cd, yd = mic.mic_filter_desc_create(), mic.mic_conv_desc_create(), mic.mic_tensor_desc_create()
    try:
        mic.mic_tensor_desc_set(d, 0, 1, 1, 1, 4, 1, 1, 1, 1 << 29)    # highest offset 3 * 2^29
        mic.mic_filter_desc_set(wd, 0, 1, 1, 1, 1)
        mic.mic_conv_desc_set(cd, 0, 0, 0, 0, 1, 1)
        mic.mic_tensor_desc_set_packed(yd, 0, 0, 1, 1, 1, 4)
        with pytest.raises(mic.MicError) as e:
            mic.mic_conv_forward_kernel_name(None, d, wd, cd, yd)
        assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    finally:
        _free(d, wd, cd, yd)


HOST_CHECK = r"""
#include <cstdio>
#include <cstdint>
#include <vector>
#include "conv_params.h"
#include "tile_map.h"
using namespace miconv;
int main() {
    // FastDiv: every divisor up to 70000 against plain division, on edge and spread numerators
    for (uint32_t d = 1; d <= 70000; ++d) {
        FastDiv f(d);
        const uint32_t probes[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 12345u * d + d - 1,
                                   0x7FFFFFFFu, 0x7FFFFFFEu, 0x40000000u, 0x3FFFFFFFu};
        for (uint32_t n : probes) {
            if (n > 0x7FFFFFFFu) continue;
            uint32_t q, r; f.divmod(n, q, r);
            if (q != n / d || r != n % d) { printf("fastdiv %u %u\n", d, n); return 1; }
        }
        for (uint64_t n = 0; n < 0x80000000ull; n += 0x7FFFFull + d) {
            uint32_t q, r; f.divmod((uint32_t)n, q, r);
            if (q != (uint32_t)n / d || r != (uint32_t)n % d) { printf("fastdiv %u %llu\n", d, (unsigned long long)n); return 1; }
        }
    }
    // XCD tile map: a bijection on [0, tiles) for every tile count up to 5000
    for (int tiles = 1; tiles <= 5000; ++tiles) {
        std::vector<int> seen(tiles, 0);
        for (int b = 0; b < tiles; ++b) {
            int t = xcd_logical_tile(b, tiles);
            if (t < 0 || t >= tiles || seen[t]++) { printf("map %d %d\n", tiles, b); return 1; }
            // ids on one XCD form one contiguous run
            if (b >= 8 && xcd_logical_tile(b - 8, tiles) != t - 1) { printf("run %d %d\n", tiles, b); return 1; }
            // the reversed order is the mirror image of the same bijection
            if (xcd_logical_tile(b, tiles, 1) != tiles - 1 - t) { printf("rev %d %d\n", tiles, b); return 1; }
        }
    }
    // grouped (m tile, n tile) order: a bijection onto the m_tiles x n_tiles grid for every group width
    for (int mt = 1; mt <= 40; ++mt)
        for (int nt = 1; nt <= 12; ++nt)
            for (int ng = 0; ng <= nt + 1; ++ng) {
                std::vector<int> seen(mt * nt, 0);
                for (int t = 0; t < mt * nt; ++t) {
                    TileRC rc = grouped_tile(t, mt, nt, ng);
                    if (rc.mt < 0 || rc.mt >= mt || rc.nt < 0 || rc.nt >= nt || seen[rc.mt * nt + rc.nt]++) {
                        printf("group %d %d %d %d\n", mt, nt, ng, t); return 1;
                    }
                    // within a group the n tiles of one m tile are consecutive
                    if (ng > 0 && ng < nt && rc.nt / ng != (t / (mt * ng))) { printf("grp %d %d %d %d\n", mt, nt, ng, t); return 1; }
                }
            }
    printf("ok\n");
    return 0;
}
"""


def test_fastdiv_and_tile_map_on_host():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "check.cpp")
        exe = os.path.join(tmp, "check")
        with open(src, "w") as fh:
            fh.write(HOST_CHECK)
        subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-I", CSRC, src, "-o", exe], check=True,
                       capture_output=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout


# ---------------------------------------------------------------- data gradient (host side)

def _dgrad_name(lay, dts=None):
    """Kernel the data gradient of a forward layer would use: (dy, w, dx) descriptors."""
    F32 = mic.MIC_DTYPE_F32
    dts = dts or {"f32": (F32, F32, F32), "f64": (1, 1, 1), "bf16": (2, 2, F32)}[lay.dtype]
    xd, wd, cd, yd = _descs(lay, dts[2], dts[1], dts[0])   # dx plays x, dy plays y
    try:
        return mic.mic_conv_backward_data_kernel_name(None, wd, yd, cd, xd)
    finally:
        _free(xd, wd, cd, yd)


def test_dgrad_kernel_choice_host_only():
    names = {lay.name: _dgrad_name(lay) for lay in workloads.ALL_LAYERS}
    for name in ("alexnet_conv2", "alexnet_conv3", "alexnet_conv4", "alexnet_conv5", "overfeat_l3",
                 "overfeat_l4", "overfeat_l5", "prec_conv3_f64_nchw", "prec_conv4_f64_nhwc"):
        assert names[name].startswith("dgrad_halo_f"), (name, names[name])
    # onto 96 channels: the 96-wide tiles
    assert names["alexnet_conv2"] == "dgrad_halo_f32_5x5_128x96_c2"
    # bf16 takes the halo kernel in data-gradient mode: 128 filters per tile onto NCHW dy
    # (the descriptors here), 64 onto channels-last dy; strided onto 3 channels at stride 4
    # (48 channel x phase columns) the stride-1 GEMM onto the stride phases, onto 1 channel
    # (4 columns) the stride-phase kernel's row-staged form
    for name in ("prec_conv3_bf16_nchw", "prec_conv4_bf16_nhwc", "prec_conv5_bf16_nhwc"):
        assert names[name] == "dgrad_halo_bf16_3x3_128x128", (name, names[name])
    lay = workloads.by_name("prec_conv4_bf16_nhwc")
    xd, wd, cd, yd = _descs(lay, mic.MIC_DTYPE_F32, 2, 2)
    try:
        mic.mic_tensor_desc_set_packed(yd, 2, mic.MIC_LAYOUT_NHWC, *mic.mic_conv_forward_output_dim(cd, xd, wd))
        assert mic.mic_conv_backward_data_kernel_name(None, wd, yd, cd, xd) == "dgrad_halo_bf16_3x3_128x64"
    finally:
        _free(xd, wd, cd, yd)
    # 21x11 / stride (2, 1) onto 32 channels: the row-streamed kernel per stride phase
    assert names["speech_l2"] == "dgrad_rows_mfma_f32_s11_256x32"
    assert names["overfeat_l1"] == "dgrad_subpixel"
    assert names["speech_l1"] == "dgrad_taps"


def test_dgrad_subpixel_kernel_limits(monkeypatch):
    """The stride-phase GEMM needs a stride above 1 and at least 32 (channel, row phase, column
    phase) columns, fp32/fp64; automatic choice below the row-streamed kernel."""
    def lay(C, u, v, dt="f32"):
        return Layer("sp", 9, 1, 2, C, 20, 24, 8, 5, 5, (u, v), (1, 1, 1, 1), dt,
                     workloads.U11, workloads.U11)
    assert _dgrad_name(lay(8, 2, 2)) == "dgrad_subpixel"          # 32 columns
    assert _dgrad_name(lay(3, 4, 4, "f64")) == "dgrad_subpixel"   # 48 columns
    assert _dgrad_name(lay(16, 2, 1)) == "dgrad_subpixel"
    assert _dgrad_name(lay(7, 2, 2)) != "dgrad_subpixel"          # 28 columns
    monkeypatch.setenv("MIC_FORCE_DGRAD_VARIANT", "subpixel")
    for bad in (lay(32, 1, 1), lay(7, 2, 2), lay(8, 2, 2, "bf16")):
        with pytest.raises(mic.MicError) as e:
            _dgrad_name(bad)
        assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED


def test_dgrad_taps_kernel_limits(monkeypatch):
    """The taps kernel takes 1-4 output channels at a stride above 1, fp32, filter rows of at
    most 16 taps, dy rows of at most 352 columns and at most 24 filter rows per row phase;
    chosen below the stride-phase GEMM (speech layer 1), NOT_SUPPORTED when forced elsewhere."""
    def lay(C, S, u, Ww=40, R=5, dt="f32", v=2):
        return Layer("tp", 9, 1, 2, C, R + 25, Ww, 8, R, S, (u, v), (1, 1, 1, 1), dt,
                     workloads.U11, workloads.U11)
    assert _dgrad_name(lay(1, 11, 2)) == "dgrad_taps"
    assert _dgrad_name(lay(8, 5, 2)) == "dgrad_subpixel"        # 32 columns
    monkeypatch.setenv("MIC_FORCE_DGRAD_VARIANT", "taps")
    for C in (1, 2, 3, 4):
        assert _dgrad_name(lay(C, 16, 2)) == "dgrad_taps"
    assert _dgrad_name(lay(1, 5, 2, Ww=703)) == "dgrad_taps"    # Q = 351
    assert _dgrad_name(lay(1, 5, 2, R=48)) == "dgrad_taps"      # 24 rows per phase
    assert _dgrad_name(lay(1, 5, 1)) == "dgrad_taps"            # stride (1, 2)
    for bad in (lay(5, 5, 2), lay(1, 17, 2), lay(1, 5, 1, v=1), lay(1, 5, 2, Ww=707),
                lay(1, 5, 2, R=49), lay(1, 5, 2, dt="f64")):
        with pytest.raises(mic.MicError) as e:
            _dgrad_name(bad)
        assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED


def test_dgrad_phase_kernel_limits(monkeypatch):
    """The stride-phase kernel takes 1-4 output channels and at most 6 column taps per phase,
    fp32/fp64: forced onto anything else it answers NOT_SUPPORTED."""
    def lay(C, S, v, dt="f32"):
        return Layer("ph", 9, 1, 2, C, 20, 24, 8, 5, S, (2, v), (1, 1, 1, 1), dt,
                     workloads.U11, workloads.U11)
    monkeypatch.setenv("MIC_FORCE_DGRAD_VARIANT", "phase")
    for C in (1, 2, 3, 4):
        assert _dgrad_name(lay(C, 5, 2)) == "dgrad_phase"
    assert _dgrad_name(lay(3, 12, 2)) == "dgrad_phase"        # 6 column taps
    assert _dgrad_name(lay(3, 3, 1, "f64")) == "dgrad_phase"
    for bad in (lay(5, 5, 2), lay(3, 13, 2), lay(3, 5, 2, "bf16")):
        with pytest.raises(mic.MicError) as e:
            _dgrad_name(bad)
        assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED


def test_dgrad_shape_and_type_errors():
    lay = workloads.TINY[0]
    F32 = mic.MIC_DTYPE_F32
    # dy dims that are not the forward output dims
    xd, wd, cd, yd = _descs(lay, F32, F32, F32, y_dims=(lay.N, lay.K, 11, 12))
    try:
        with pytest.raises(mic.MicError) as e:
            mic.mic_conv_backward_data_kernel_name(None, wd, yd, cd, xd)
        assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    finally:
        _free(xd, wd, cd, yd)
    for combo in [(0, 0, 1), (2, 2, 2), (1, 0, 1)]:
        xd, wd, cd, yd = _descs(lay, combo[2], combo[1], combo[0])
        try:
            with pytest.raises(mic.MicError) as e:
                mic.mic_conv_backward_data_kernel_name(None, wd, yd, cd, xd)
            assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
        finally:
            _free(xd, wd, cd, yd)
    l = mic.lib()
    assert l.mic_conv_backward_data(None, 1.0, None, None, None, None, None, 0.0, None, None) == \
        mic.MIC_STATUS_BAD_PARAM


def test_dgrad_forced_variant(monkeypatch):
    lay = workloads.by_name("alexnet_conv3")
    monkeypatch.setenv("MIC_FORCE_DGRAD_VARIANT", "direct")
    assert _dgrad_name(lay) == "dgrad_direct"
    monkeypatch.setenv("MIC_FORCE_DGRAD_VARIANT", "halo_f32_3x3_64x128")
    assert _dgrad_name(lay) == "dgrad_halo_f32_3x3_64x128"
    monkeypatch.setenv("MIC_FORCE_DGRAD_VARIANT", "halo_f32_5x5_128x128")    # wrong filter size
    with pytest.raises(mic.MicError) as e:
        _dgrad_name(lay)
    assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED


# ---------------------------------------------------------------- filter gradient (host side)

def _wgrad_name(lay, dts=None):
    """Kernel the filter gradient of a forward layer would use: (x, dy, dw) descriptors."""
    F32 = mic.MIC_DTYPE_F32
    dts = dts or {"f32": (F32, F32, F32), "f64": (1, 1, 1), "bf16": (2, 2, F32)}[lay.dtype]
    xd, wd, cd, yd = _descs(lay, dts[0], dts[2], dts[1])   # wd plays dw, yd plays dy
    try:
        return mic.mic_conv_backward_filter_kernel_name(None, xd, yd, cd, wd)
    finally:
        _free(xd, wd, cd, yd)


def _wgrad_name_same_layout(lay, k=None):
    """Like _wgrad_name, with dy in the layer's own layout (and row pitch)."""
    xd, wd, yd, cd = (mic.mic_tensor_desc_create(), mic.mic_filter_desc_create(),
                      mic.mic_tensor_desc_create(), mic.mic_conv_desc_create())
    try:
        dt = {"f32": 0, "f64": 1, "bf16": 2}[lay.dtype]
        K = lay.K if k is None else k
        xs = workloads.padded_strides(lay.N, lay.C, lay.H, lay.W, lay.layout, lay.row_pitch)
        mic.mic_tensor_desc_set(xd, dt, *lay.x_shape, *xs)
        mic.mic_filter_desc_set(wd, 1 if dt == 1 else 0, K, lay.C, lay.R, lay.S)
        mic.mic_conv_desc_set(cd, *lay.padding, *lay.stride)
        N, K, P, Q = mic.mic_conv_forward_output_dim(cd, xd, wd)
        ys = workloads.padded_strides(N, K, P, Q, lay.layout, lay.row_pitch)
        mic.mic_tensor_desc_set(yd, dt, N, K, P, Q, *ys)
        return mic.mic_conv_backward_filter_kernel_name(None, xd, yd, cd, wd)
    finally:
        _free(xd, wd, cd, yd)


def test_wgrad_channels_last_bf16_choice_host_only():
    """bf16 with channels-last x and dy goes to the transposing-read kernel: three wave groups
    where the tiles fit one per compute unit (conv3, conv5: 216 tiles), two where two workgroups
    share a unit (conv4: 324 tiles); channel counts that are not multiples of 8 cannot take it."""
    want = {"prec_conv3_bf16_nhwc": "wgc_bf16_64x64_ks3", "prec_conv4_bf16_nhwc": "wgc_bf16_64x64_ks2",
            "prec_conv5_bf16_nhwc": "wgc_bf16_64x64_ks3"}
    for lay in workloads.PRECISION:
        name = _wgrad_name_same_layout(lay)
        if lay.name in want:
            assert name == want[lay.name], (lay.name, name)
        else:
            assert not name.startswith("wgc_"), (lay.name, name)
    lay = workloads.by_name("prec_conv3_bf16_nhwc")
    assert not _wgrad_name_same_layout(lay, k=100).startswith("wgc_")      # K % 8 != 0


def test_wgrad_first_layer_kernel_limits(monkeypatch):
    """The vector-ALU first-layer kernels take 11-wide fp32 filters at their column stride (2 or 4),
    at most 384 (64) output columns, unit stride along w and q, left padding under 64; forced onto
    anything else they answer NOT_SUPPORTED."""
    def lay(S=11, v=2, W=150, layout="nchw", pl=0, dt="f32"):
        return Layer("wr", 9, 1, 2, 2, 20, W, 6, 5, S, (2, v), (1, 1, pl, 0), dt,
                     workloads.U11, workloads.U11, layout=layout)
    monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", "wgr_f32_s11_v2")
    assert _wgrad_name(lay()) == "wgr_f32_s11_v2"
    assert _wgrad_name(lay(W=700, pl=63)) == "wgr_f32_s11_v2"          # Q = 377, pad 63
    for bad in (lay(S=9), lay(v=4), lay(W=790), lay(layout="nhwc"), lay(pl=64), lay(dt="f64")):
        with pytest.raises(mic.MicError) as e:
            _wgrad_name(bad)
        assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", "wgr_f32_s11_v4")
    assert _wgrad_name(lay(v=4, W=260)) == "wgr_f32_s11_v4"            # Q = 63
    with pytest.raises(mic.MicError):
        _wgrad_name(lay(v=4, W=270))                                     # Q = 65


def test_wgrad_kernel_choice_host_only():
    """The plan's cost model (rounds of tiles x measured time per tile) on the workload layers:
    the halo kernel for the stride-1 3x3 and 5x5 (pitch 24) layers, with 64x96 tiles where they
    save a round (AlexNet conv4; Overfeat L3-L5 in the form that steps along their 12-column output
    rows only, as AlexNet conv2/conv3/conv5 and Overfeat L2 along 27, 13 and 20), the vector-ALU
    row-staged kernel for the strided
    11-wide first layers, the split-reduction kernel where dw has few tiles (the tiny layer), and
    for bf16 the halo kernel with x and dy widened to fp32 as they are staged (dy here in NCHW;
    with channels-last x and dy the channels-last kernel, tested below)."""
    want = {"tiny": "wgs_f32_8x16",
            "alexnet_conv2": "wgh_f32x16_5x5_q27_64x48", "alexnet_conv3": "wgh_f32_3x3_q13_64x64",
            "alexnet_conv4": "wgh_f32_3x3_64x96_ks4", "alexnet_conv5": "wgh_f32_3x3_q13_64x64",
            "overfeat_l1": "wgr_f32_s11_v4", "overfeat_l2": "wgh_f32x16_5x5_q20_64x48",
            "overfeat_l3": "wgh_f32_3x3_q12_64x96", "overfeat_l4": "wgh_f32_3x3_q12_64x96",
            "overfeat_l5": "wgh_f32_3x3_q12_64x96",
            "speech_l1": "wgr_f32_s11_v2", "speech_l2": "wgh_f32x16_pairs_s11_32x64"}
    for lay in workloads.ALL_LAYERS:
        name = _wgrad_name(lay)
        if lay.name in want:
            assert name == want[lay.name], (lay.name, name)
        elif lay.dtype == "f64":
            # 384 x 3456 (conv4): 64x96 tiles in one round; else 64x64 with four wave groups
            want64 = "wgh_f64_3x3_64x96" if "conv4" in lay.name else "wgh_f64_3x3_64x64_ks4"
            assert name == want64, (lay.name, name)
        else:
            # bf16: 64x96 tiles with four wave groups, the reduction in two parts (144 tiles on
            # conv3 / conv5, 216 on conv4)
            assert name == "wgh_bf16_3x3_64x96_ks4", (lay.name, name)


def test_wgrad_split_kernel_needs_small_tensors(monkeypatch):
    """The split-reduction kernel addresses x and dy with 32-bit byte offsets: forced onto a
    tensor of 2 GiB or more it answers NOT_SUPPORTED, and the plan never picks it there."""
    lay = workloads.TINY[0]
    monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", "wgs_f32_16x16")
    assert _wgrad_name(lay) == "wgs_f32_16x16"
    # dy: 4 filters x 16384 x 8192 fp32 = 2 GiB (x: 512 MiB)
    big = Layer("big", 9, 1, 1, 1, 1 << 14, 1 << 13, 4, 3, 3, (1, 1), (1, 1, 1, 1), "f32",
                workloads.U11, workloads.U11)
    with pytest.raises(mic.MicError) as e:
        _wgrad_name(big)
    assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    monkeypatch.delenv("MIC_FORCE_WGRAD_VARIANT")
    assert not _wgrad_name(big).startswith("wgs_")


def test_wgrad_shape_and_type_errors(monkeypatch):
    lay = workloads.TINY[0]
    F32 = mic.MIC_DTYPE_F32
    xd, wd, cd, yd = _descs(lay, F32, F32, F32, y_dims=(lay.N, lay.K, 12, 11))
    try:
        with pytest.raises(mic.MicError) as e:
            mic.mic_conv_backward_filter_kernel_name(None, xd, yd, cd, wd)
        assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    finally:
        _free(xd, wd, cd, yd)
    for combo in [(0, 0, 1), (2, 2, 2), (1, 0, 1)]:
        with pytest.raises(mic.MicError) as e:
            _wgrad_name(lay, combo)
        assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", "wg_f32_64x64")
    assert _wgrad_name(lay) == "wg_f32_64x64"
    monkeypatch.setenv("MIC_FORCE_WGRAD_VARIANT", "wg_f64_64x64")       # another element type
    with pytest.raises(mic.MicError) as e:
        _wgrad_name(lay)
    assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    l = mic.lib()
    assert l.mic_conv_backward_filter(None, 1.0, None, None, None, None, None, 0.0, None, None) == \
        mic.MIC_STATUS_BAD_PARAM


# ---------------------------------------------------------------- pooling (host side)

def test_pool_descriptor_and_output_dims():
    d = mic.mic_pool_desc_create()
    try:
        with pytest.raises(mic.MicError):
            mic.mic_pool_desc_get(d)                       # never set
        mic.mic_pool_desc_set(d, mic.MIC_POOL_AVG_EXCLUDE_PAD, 3, 2, 1, 0, 2, 1, 2, 1)
        assert mic.mic_pool_desc_get(d) == (2, 3, 2, 1, 0, 2, 1, 2, 1)
        for bad in [(3, 3, 3, 0, 0, 0, 0, 1, 1), (0, 0, 3, 0, 0, 0, 0, 1, 1), (0, 3, 3, -1, 0, 0, 0, 1, 1),
                    (0, 3, 3, 0, 0, 0, 0, 0, 1)]:
            with pytest.raises(mic.MicError) as e:
                mic.mic_pool_desc_set(d, *bad)
            assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    finally:
        mic.mic_pool_desc_destroy(d)
    for lay in workloads.POOLING:
        pb = oracle.make_problem(lay.x_shape, (1, 1, 1, 1), (1, lay.C, lay.R, lay.S), lay.stride, lay.padding)
        P, Q = oracle.output_dims(pb)
        assert mic.pool_output_shape(lay.x_shape, (lay.R, lay.S), lay.stride, lay.padding) == (lay.N, lay.C, P, Q)
    with pytest.raises(mic.MicError):                      # window larger than the padded input
        mic.pool_output_shape((1, 1, 3, 3), (5, 1), (1, 1), (0, 1, 0, 0))
    l = mic.lib()
    assert l.mic_pool_forward(None, 1.0, None, None, None, 0.0, None, None) == mic.MIC_STATUS_BAD_PARAM


def test_pool_size_limits_host_only():
    """Output sizes past INT32_MAX and windows of 2^30 positions or more are refused
    before anything is launched (the kernel indexes them with 32-bit ints)."""
    big = (1 << 31) - 1
    with pytest.raises(mic.MicError) as e:                 # P = 2^31 - 1 + 2^30 rows
        mic.pool_output_shape((1, 1, big, 1), (1, 1), (1, 1), (1 << 30, 0, 0, 0))
    assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    assert mic.pool_output_shape((1, 1, big, 1), (1, 1), (1, 1), (0, 0, 0, 0)) == (1, 1, big, 1)
    # a 32768 x 32768 window over a 1 x 1 input padded to the window: one output of
    # 2^30 window positions.  Fake non-null handle and pointers: the call must fail
    # in validation, before anything dereferences them.
    xd, yd, pd = mic.mic_tensor_desc_create(), mic.mic_tensor_desc_create(), mic.mic_pool_desc_create()
    try:
        mic.mic_tensor_desc_set_packed(xd, mic.MIC_DTYPE_F32, mic.MIC_LAYOUT_NCHW, 1, 1, 1, 1)
        mic.mic_tensor_desc_set_packed(yd, mic.MIC_DTYPE_F32, mic.MIC_LAYOUT_NCHW, 1, 1, 1, 1)
        l = mic.lib()
        for win, status in [(32768, mic.MIC_STATUS_NOT_SUPPORTED), (32767, None)]:
            pad = win - 1
            mic.mic_pool_desc_set(pd, mic.MIC_POOL_MAX, win, win, pad, 0, pad, 0, 1, 1)
            assert mic.mic_pool_forward_output_dim(pd, xd) == (1, 1, 1, 1)
            if status is not None:
                assert l.mic_pool_forward(1, 1.0, pd, xd, 16, 0.0, yd, 16) == status
    finally:
        mic.mic_tensor_desc_destroy(xd)
        mic.mic_tensor_desc_destroy(yd)
        mic.mic_pool_desc_destroy(pd)


def test_brgemm_kernel_choice_host_only():
    """Skinny products (the AlexNet fully-connected layers, weights contiguous along k) go to the
    wave-split kernel; large ones, or B not contiguous along k, to the shared-LDS tiles."""
    import torch
    tdt = {"f32": torch.float32, "f64": torch.float64, "bf16": torch.bfloat16}
    assert mic.brgemm_kernel_name(torch.float32, 128, 4096, 9216, b_strides=(0, 1, 9216)) == "ws_f32_32x64"
    assert mic.brgemm_kernel_name(torch.float32, 256, 4096, 9216, b_strides=(0, 1, 9216)) == "ws_f32_64x64"
    assert mic.brgemm_kernel_name(torch.float32, 128, 1000, 4096, b_strides=(0, 1, 4096)) == "ws_f32_16x32"
    assert mic.brgemm_kernel_name(torch.bfloat16, 128, 4096, 9216, b_strides=(0, 1, 9216)) == "ws_bf16_32x64"
    assert mic.brgemm_kernel_name(torch.float32, 128, 4096, 9216).startswith("br_f32_")      # B not k-contiguous
    assert mic.brgemm_kernel_name(torch.float32, 4096, 4096, 4096, b_strides=(0, 1, 4096)) == "br_f32_128x128"
    for lay in workloads.FC:
        F = lay.features
        name = mic.brgemm_kernel_name(tdt[lay.dtype], lay.m, lay.n, lay.k, lay.batch,
                                      a_strides=(lay.k, F, 1), b_strides=(lay.k, 1, F))
        assert name.startswith("ws_" + lay.dtype + "_"), (lay.name, name)


def test_brgemm_argument_errors(monkeypatch):
    import torch
    l = mic.lib()
    args = dict(m=4, n=4, k=4, batch=1)

    def call(dtype=mic.MIC_DTYPE_F32, handle=1, a=16, b=16, c=16, sa=(16, 4, 1), sb=(16, 4, 1), sc=(4, 1), **kw):
        d = dict(args, **kw)
        return l.mic_brgemm(handle, dtype, d["m"], d["n"], d["k"], d["batch"], 1.0, a, *sa, b, *sb, 0.0, c, *sc)

    # errors found before anything touches the device (handle 1 is never dereferenced on these paths)
    assert l.mic_brgemm(None, mic.MIC_DTYPE_F32, 4, 4, 4, 1, 1.0, 16, 16, 4, 1, 16, 16, 4, 1, 0.0, 16, 4, 1) \
        == mic.MIC_STATUS_BAD_PARAM
    assert call(m=-1) == mic.MIC_STATUS_BAD_PARAM
    assert call(batch=-1) == mic.MIC_STATUS_BAD_PARAM
    assert call(sa=(16, -4, 1)) == mic.MIC_STATUS_BAD_PARAM
    assert call(a=0) == mic.MIC_STATUS_BAD_PARAM                 # null A with work to do
    assert call(c=0) == mic.MIC_STATUS_BAD_PARAM
    assert call(a=18) == mic.MIC_STATUS_BAD_PARAM                # misaligned fp32 pointer
    assert call(sc=(0, 1)) == mic.MIC_STATUS_BAD_PARAM           # rows of C alias
    assert call(dtype=7) == mic.MIC_STATUS_NOT_SUPPORTED
    assert call(sa=(0, 1 << 30, 1)) == mic.MIC_STATUS_NOT_SUPPORTED
    assert call(k=1 << 16, batch=1 << 14, sa=(0, 0, 0), sb=(0, 0, 0)) == mic.MIC_STATUS_NOT_SUPPORTED
    buf = ctypes.create_string_buffer(4)
    assert l.mic_brgemm_kernel_name(None, mic.MIC_DTYPE_F32, 128, 128, 128, 1, 0, 128, 1, 0, 128, 1, 128, 1,
                                    buf, 4) == mic.MIC_STATUS_BAD_PARAM
    import torch
    monkeypatch.setenv("MIC_FORCE_BRGEMM_VARIANT", "br_f64_64x64")
    with pytest.raises(mic.MicError) as e:
        mic.brgemm_kernel_name(torch.float32, 128, 128, 128)
    assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    monkeypatch.setenv("MIC_FORCE_BRGEMM_VARIANT", "br_f32_64x64")
    assert mic.brgemm_kernel_name(torch.float32, 128, 128, 128) == "br_f32_64x64"
    # the wave-split kernel needs A and B contiguous along k
    monkeypatch.setenv("MIC_FORCE_BRGEMM_VARIANT", "ws_f32_32x64")
    with pytest.raises(mic.MicError) as e:
        mic.brgemm_kernel_name(torch.float32, 128, 128, 128)           # B packed (k, n): not contiguous in k
    assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    assert mic.brgemm_kernel_name(torch.float32, 128, 128, 128, b_strides=(0, 1, 128)) == "ws_f32_32x64"
    with pytest.raises(mic.MicError):
        mic.brgemm_kernel_name(torch.float32, 128, 128, 102, b_strides=(0, 1, 102))   # k % 4 != 0


def test_buffer_load_kernels_refuse_tensors_past_their_range():
    """The staging kernels read x (dy) and the filters through range-checked buffer
    descriptors whose record count is 32-bit: tensors of 2^31 bytes or more must go to
    another kernel (the gather kernel), just under it the fast kernels stay."""
    import dataclasses
    F32 = mic.MIC_DTYPE_F32

    def fwd(lay):
        d = _descs(lay, F32, F32, F32)
        try:
            return mic.mic_conv_forward_kernel_name(None, *d)
        finally:
            _free(*d)

    l1, l5, sp2 = (workloads.by_name(n) for n in ("overfeat_l1", "overfeat_l5", "speech_l2"))
    # Overfeat L1: x = N * 3 * 231 * 231 * 4 bytes (N = 3000: 1.92e9; 3400: 2.18e9)
    assert fwd(dataclasses.replace(l1, N=3000)) == "rows1n6_f32_s11_256x32"
    assert not fwd(dataclasses.replace(l1, N=3400)).startswith("rows")
    # Overfeat L5: x = N * 1024 * 144 * 4 bytes (N = 1024: 0.60e9; 4096: 2.42e9)
    assert fwd(dataclasses.replace(l5, N=1024)).startswith("halo_")
    big5 = dataclasses.replace(l5, N=4096)
    assert not fwd(big5).startswith("halo_")
    assert not _dgrad_name(big5).startswith("dgrad_halo")
    assert not _wgrad_name(big5).startswith("wgh_")
    # speech L2: x = N * 32 * 81 * 350 * 4 bytes (N = 500: 1.81e9; 700: 2.54e9)
    assert fwd(dataclasses.replace(sp2, N=500)) == "rows_f32_s11_256x32"
    assert not fwd(dataclasses.replace(sp2, N=700)).startswith("rows")

"""Channel-blocked layouts on the host (no GPU): the layout conversions the
tests use, descriptor validation and the kernel each blocking reaches.

Blocked layouts follow the zero-memory direct-convolution page ("Proposed
Method": blocked input, output and weight layouts of the same size as
standard storage); the reading taken is x as [N][C/cb][H][W][cb] and
filters as [K/kb][C/cb][R][S][cb][kb], with exact blocks.  The conversions
are pinned against those offset formulas written out element by element.
"""
import numpy as np
import pytest
import torch

import convolution_forward_conv2d_amd as mic
import gen

F32 = mic.MIC_DTYPE_F32


def test_activation_conversion_matches_the_offset_formula():
    N, C, H, W, cb = 2, 12, 3, 5, 4
    x = torch.from_numpy(gen.uniform(1700, (N, C, H, W), -1.0, 1.0))
    xb = mic.to_blocked(x, cb)
    assert xb.shape == (N, C // cb, H, W, cb) and xb.is_contiguous()
    flat = xb.reshape(-1)
    for n in range(N):
        for c in range(C):
            for h in range(H):
                for w in range(W):
                    off = n * C * H * W + (c // cb) * H * W * cb + h * W * cb + w * cb + c % cb
                    assert flat[off] == x[n, c, h, w]
    assert torch.equal(mic.from_blocked(xb), x)
    with pytest.raises(ValueError):
        mic.to_blocked(x, 5)


def test_filter_conversion_matches_the_offset_formula():
    K, C, R, S, kb, cb = 8, 6, 2, 3, 4, 3
    f = torch.from_numpy(gen.uniform(1701, (K, C, R, S), -1.0, 1.0))
    fb = mic.filters_to_blocked(f, kb, cb)
    assert fb.shape == (K // kb, C // cb, R, S, cb, kb) and fb.is_contiguous()
    flat = fb.reshape(-1)
    for k in range(K):
        for c in range(C):
            for r in range(R):
                for s in range(S):
                    off = ((k // kb) * (C // cb) + c // cb) * R * S * cb * kb + ((r * S + s) * cb + c % cb) * kb + k % kb
                    assert flat[off] == f[k, c, r, s]
    assert torch.equal(mic.filters_from_blocked(fb), f)


def test_blocked_descriptors_roundtrip_and_validation():
    d = mic.mic_tensor_desc_create()
    f = mic.mic_filter_desc_create()
    try:
        mic.mic_tensor_desc_set_blocked(d, F32, 2, 64, 13, 11, 16)
        assert mic.mic_tensor_desc_get_block(d) == (16, 13 * 11 * 16)
        dt, dims, strides = mic.mic_tensor_desc_get(d)
        assert dims == (2, 64, 13, 11) and strides == (64 * 13 * 11, 1, 11 * 16, 16)
        mic.mic_tensor_desc_set_packed(d, F32, mic.MIC_LAYOUT_NCHW, 2, 64, 13, 11)
        assert mic.mic_tensor_desc_get_block(d) == (0, 0)            # reset to unblocked
        for bad in [(2, 60, 13, 11, 16), (2, 64, 13, 11, 0), (0, 64, 13, 11, 16)]:
            with pytest.raises(mic.MicError) as e:
                mic.mic_tensor_desc_set_blocked(d, F32, *bad)
            assert e.value.status == mic.MIC_STATUS_BAD_PARAM
        mic.mic_filter_desc_set_blocked(f, F32, 64, 32, 3, 3, 16, 8)
        assert mic.mic_filter_desc_get_block(f) == (16, 8)
        assert mic.mic_filter_desc_get(f)[1] == (64, 32, 3, 3)
        mic.mic_filter_desc_set(f, F32, 64, 32, 3, 3)
        assert mic.mic_filter_desc_get_block(f) == (0, 0)
        for bad in [(64, 32, 3, 3, 24, 8), (64, 32, 3, 3, 16, 5), (64, 32, 3, 3, 0, 8)]:
            with pytest.raises(mic.MicError) as e:
                mic.mic_filter_desc_set_blocked(f, F32, *bad)
            assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    finally:
        mic.mic_tensor_desc_destroy(d)
        mic.mic_filter_desc_destroy(f)


def _choice(dtype, x_cb, w_blocks, y_kb, N=4, C=64, H=13, W=13, K=64, R=3, S=3, pads=(1, 1, 1, 1)):
    xd, yd, wd, cd = (mic.mic_tensor_desc_create(), mic.mic_tensor_desc_create(), mic.mic_filter_desc_create(),
                      mic.mic_conv_desc_create())
    try:
        if x_cb:
            mic.mic_tensor_desc_set_blocked(xd, dtype, N, C, H, W, x_cb)
        else:
            mic.mic_tensor_desc_set_packed(xd, dtype, mic.MIC_LAYOUT_NCHW, N, C, H, W)
        wdt = dtype
        if w_blocks:
            mic.mic_filter_desc_set_blocked(wd, wdt, K, C, R, S, *w_blocks)
        else:
            mic.mic_filter_desc_set(wd, wdt, K, C, R, S)
        mic.mic_conv_desc_set(cd, *pads, 1, 1)
        n, k, P, Q = mic.mic_conv_forward_output_dim(cd, xd, wd)
        ydt = F32 if dtype == mic.MIC_DTYPE_BF16 else dtype
        if y_kb:
            mic.mic_tensor_desc_set_blocked(yd, ydt, n, k, P, Q, y_kb)
        else:
            mic.mic_tensor_desc_set_packed(yd, ydt, mic.MIC_LAYOUT_NCHW, n, k, P, Q)
        return mic.mic_conv_forward_kernel_name(None, xd, wd, cd, yd)
    finally:
        for d, fn in ((xd, mic.mic_tensor_desc_destroy), (yd, mic.mic_tensor_desc_destroy),
                      (wd, mic.mic_filter_desc_destroy), (cd, mic.mic_conv_desc_destroy)):
            fn(d)


def test_blocked_kernel_choice():
    BF16, F64 = mic.MIC_DTYPE_BF16, mic.MIC_DTYPE_F64
    # blocks that hold whole channel chunks keep the tap-batched kernels
    assert _choice(F32, 16, (16, 16), 16).startswith("halo_f32_3x3_")
    assert _choice(F64, 16, (16, 16), 16).startswith("halo_f64_3x3_")
    assert _choice(F32, 32, None, 32).startswith("halo_f32_3x3_")
    assert _choice(BF16, 16, None, 16).startswith("halo_bf16_3x3_")
    # bf16 blocked filters: the tap-batched kernel's transposing loader when blocks of
    # 8 filters and 16 channels fit (kb % 8, cb % 16), else the gather kernel in tap
    # order (cb a multiple of 32), else direct
    assert _choice(BF16, 32, (32, 32), 32).startswith("halo_bf16_3x3_")
    assert _choice(BF16, 16, (16, 16), 16).startswith("halo_bf16_3x3_")
    assert _choice(BF16, 32, (4, 32), 32).endswith("_tap")
    assert _choice(BF16, 16, (4, 16), 16) == "direct"
    # x blocked by 2 (not a multiple of the 4-channel chunk): flat gather order
    name = _choice(F32, 2, None, 8)
    assert name.startswith("mfma_f32_") and not name.endswith("_tap")
    # filters blocked by 8 channels (no halo chunk fits kb = 2): tap order needs cb % 16 -> direct
    assert _choice(F32, 8, (2, 8), 8) == "direct"


def test_blocked_forced_variants(monkeypatch):
    monkeypatch.setenv("MIC_FORCE_VARIANT", "mfma_f32_128x128")          # flat order cannot read blocked filters
    with pytest.raises(mic.MicError) as e:
        _choice(F32, 16, (16, 16), 16)
    assert e.value.status == mic.MIC_STATUS_NOT_SUPPORTED
    monkeypatch.setenv("MIC_FORCE_VARIANT", "mfma_f32_128x128_tap")
    assert _choice(F32, 16, (16, 16), 16) == "mfma_f32_128x128_tap"
    with pytest.raises(mic.MicError):
        _choice(F32, 8, None, 8)                                      # tap order needs cb % 16 == 0
    monkeypatch.setenv("MIC_FORCE_VARIANT", "halo_bf16_3x3_128x128")
    assert _choice(mic.MIC_DTYPE_BF16, 32, (32, 32), 32) == "halo_bf16_3x3_128x128"
    with pytest.raises(mic.MicError):
        _choice(mic.MIC_DTYPE_BF16, 32, (4, 32), 32)                  # bf16 halo: blocks of 8 filters or more


def test_other_operations_refuse_blocked_descriptors():
    l = mic.lib()
    xd, dyd, wd, cd, pd = (mic.mic_tensor_desc_create(), mic.mic_tensor_desc_create(), mic.mic_filter_desc_create(),
                           mic.mic_conv_desc_create(), mic.mic_pool_desc_create())
    try:
        mic.mic_tensor_desc_set_blocked(xd, F32, 2, 16, 8, 8, 8)
        mic.mic_tensor_desc_set_packed(dyd, F32, mic.MIC_LAYOUT_NCHW, 2, 16, 8, 8)
        mic.mic_filter_desc_set(wd, F32, 16, 16, 3, 3)
        mic.mic_conv_desc_set(cd, 1, 1, 1, 1, 1, 1)
        mic.mic_pool_desc_set(pd, mic.MIC_POOL_MAX, 2, 2, 0, 0, 0, 0, 2, 2)
        import ctypes
        buf = ctypes.create_string_buffer(64)
        assert l.mic_conv_backward_data_kernel_name(None, wd, dyd, cd, xd, buf, 64) == mic.MIC_STATUS_NOT_SUPPORTED
        assert l.mic_conv_backward_filter_kernel_name(None, xd, dyd, cd, wd, buf, 64) == mic.MIC_STATUS_NOT_SUPPORTED
        yd = mic.mic_tensor_desc_create()
        mic.mic_tensor_desc_set_packed(yd, F32, mic.MIC_LAYOUT_NCHW, 2, 16, 4, 4)
        assert l.mic_pool_forward(1, 1.0, pd, xd, 16, 0.0, yd, 16) == mic.MIC_STATUS_NOT_SUPPORTED
        mic.mic_tensor_desc_destroy(yd)
    finally:
        mic.mic_tensor_desc_destroy(xd)
        mic.mic_tensor_desc_destroy(dyd)
        mic.mic_filter_desc_destroy(wd)
        mic.mic_conv_desc_destroy(cd)
        mic.mic_pool_desc_destroy(pd)

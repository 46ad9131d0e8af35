"""Python binding of libmiconv, the MI355X 2-D convolution forward pass and
its data gradient.

Argument marshalling only: every step of the convolution runs in the HIP
kernels of ``libmiconv.so`` behind the C ABI declared in
``include/miconv.h``.  PyTorch supplies device memory and the stream.
The ``mic_*`` functions mirror the C calls one for one (descriptors are
ctypes handles); ``conv2d_forward`` / ``ConvPlan`` and
``conv2d_backward_data`` / ``DgradPlan`` and ``conv2d_backward_filter`` /
``WgradPlan`` wrap them for torch tensors.

There is no fallback: if the library is missing the import fails.
"""
import ctypes
import os
import re

import torch  # loads the HIP runtime that libmiconv then shares

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmiconv.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "miconv.h")

# ---------------------------------------------------------------- enums (miconv.h)
MIC_STATUS_SUCCESS = 0
MIC_STATUS_BAD_PARAM = 1
MIC_STATUS_NOT_SUPPORTED = 2
MIC_STATUS_LAUNCH_FAILED = 3
MIC_STATUS_INTERNAL_ERROR = 4
MIC_STATUS_ALLOC_FAILED = 5

MIC_DTYPE_F32 = 0
MIC_DTYPE_F64 = 1
MIC_DTYPE_BF16 = 2

MIC_LAYOUT_NCHW = 0
MIC_LAYOUT_NHWC = 1

MIC_POOL_MAX = 0
MIC_POOL_AVG_INCLUDE_PAD = 1
MIC_POOL_AVG_EXCLUDE_PAD = 2
POOL_MODES = {"max": MIC_POOL_MAX, "avg_include_pad": MIC_POOL_AVG_INCLUDE_PAD,
              "avg_exclude_pad": MIC_POOL_AVG_EXCLUDE_PAD}

_TORCH_DTYPE = {torch.float32: MIC_DTYPE_F32, torch.float64: MIC_DTYPE_F64,
                torch.bfloat16: MIC_DTYPE_BF16}
_OUT_DTYPE = {torch.float32: torch.float32, torch.float64: torch.float64,
              torch.bfloat16: torch.float32}


class MicError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_ip = ctypes.POINTER(ctypes.c_int)
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "mic_status_string": ([_i], ctypes.c_char_p),
    "mic_get_version": ([_ip, _ip, _ip], _i),
    "mic_create": ([ctypes.POINTER(_vp)], _i),
    "mic_destroy": ([_vp], _i),
    "mic_set_stream": ([_vp, _vp], _i),
    "mic_get_stream": ([_vp, ctypes.POINTER(_vp)], _i),
    "mic_tensor_desc_create": ([ctypes.POINTER(_vp)], _i),
    "mic_tensor_desc_destroy": ([_vp], _i),
    "mic_tensor_desc_set": ([_vp, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64], _i),
    "mic_tensor_desc_set_packed": ([_vp, _i, _i, _i, _i, _i, _i], _i),
    "mic_tensor_desc_get": ([_vp, _ip, _ip, _ip, _ip, _ip, _i64p], _i),
    "mic_tensor_desc_set_blocked": ([_vp, _i, _i, _i, _i, _i, _i], _i),
    "mic_tensor_desc_get_block": ([_vp, _ip, _i64p], _i),
    "mic_filter_desc_create": ([ctypes.POINTER(_vp)], _i),
    "mic_filter_desc_destroy": ([_vp], _i),
    "mic_filter_desc_set": ([_vp, _i, _i, _i, _i, _i], _i),
    "mic_filter_desc_get": ([_vp, _ip, _ip, _ip, _ip, _ip], _i),
    "mic_filter_desc_set_blocked": ([_vp, _i, _i, _i, _i, _i, _i, _i], _i),
    "mic_filter_desc_get_block": ([_vp, _ip, _ip], _i),
    "mic_conv_desc_create": ([ctypes.POINTER(_vp)], _i),
    "mic_conv_desc_destroy": ([_vp], _i),
    "mic_conv_desc_set": ([_vp, _i, _i, _i, _i, _i, _i], _i),
    "mic_conv_desc_get": ([_vp, _ip, _ip, _ip, _ip, _ip, _ip], _i),
    "mic_conv_forward_output_dim": ([_vp, _vp, _vp, _ip, _ip, _ip, _ip], _i),
    "mic_conv_forward": ([_vp, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, ctypes.c_double,
                          _vp, _vp], _i),
    "mic_conv_forward_kernel_name": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_char_p, ctypes.c_size_t],
                                     _i),
    "mic_conv_backward_data": ([_vp, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, ctypes.c_double,
                                _vp, _vp], _i),
    "mic_conv_backward_data_kernel_name": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_char_p, ctypes.c_size_t],
                                           _i),
    "mic_conv_backward_filter": ([_vp, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, ctypes.c_double,
                                  _vp, _vp], _i),
    "mic_conv_backward_filter_kernel_name": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_char_p, ctypes.c_size_t],
                                             _i),
    "mic_pool_desc_create": ([ctypes.POINTER(_vp)], _i),
    "mic_pool_desc_destroy": ([_vp], _i),
    "mic_pool_desc_set": ([_vp, _i, _i, _i, _i, _i, _i, _i, _i, _i], _i),
    "mic_pool_desc_get": ([_vp, _ip, _ip, _ip, _ip, _ip, _ip, _ip, _ip, _ip], _i),
    "mic_pool_forward_output_dim": ([_vp, _vp, _ip, _ip, _ip, _ip], _i),
    "mic_pool_forward": ([_vp, ctypes.c_double, _vp, _vp, _vp, ctypes.c_double, _vp, _vp], _i),
    "mic_brgemm": ([_vp, _i, _i, _i, _i, _i, ctypes.c_double, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                    ctypes.c_double, _vp, _i64, _i64], _i),
    "mic_brgemm_kernel_name": ([_vp, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                ctypes.c_char_p, ctypes.c_size_t], _i),
}


def lib():
    """The loaded libmiconv (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmiconv.so is not built (%s); run "
                              "`python -m convolution_forward_conv2d_amd.build`" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = res
        _lib = l
    return _lib


def header_functions():
    """Names of every function miconv.h declares."""
    with open(HEADER_PATH) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mic_[a-z0-9_]+)\s*\(", text)))


def _check(status, where):
    if status != MIC_STATUS_SUCCESS:
        raise MicError(status, where)


# ---------------------------------------------------------------- one-for-one wrappers

def status_string(status):
    return lib().mic_status_string(int(status)).decode()


mic_status_string = status_string


def mic_get_version():
    a, b, c = _i(), _i(), _i()
    _check(lib().mic_get_version(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "mic_get_version")
    return a.value, b.value, c.value


def mic_create():
    h = _vp()
    _check(lib().mic_create(ctypes.byref(h)), "mic_create")
    return h


def mic_destroy(handle):
    _check(lib().mic_destroy(handle), "mic_destroy")


def mic_set_stream(handle, stream):
    """stream: a hipStream_t as an int (torch: ``stream.cuda_stream``) or None."""
    _check(lib().mic_set_stream(handle, _vp(stream or 0)), "mic_set_stream")


def mic_get_stream(handle):
    s = _vp()
    _check(lib().mic_get_stream(handle, ctypes.byref(s)), "mic_get_stream")
    return s.value or 0


def _create(fn, where):
    d = _vp()
    _check(fn(ctypes.byref(d)), where)
    return d


def mic_tensor_desc_create():
    return _create(lib().mic_tensor_desc_create, "mic_tensor_desc_create")


def mic_tensor_desc_destroy(d):
    _check(lib().mic_tensor_desc_destroy(d), "mic_tensor_desc_destroy")


def mic_tensor_desc_set(d, dtype, n, c, h, w, sn, sc, sh, sw):
    _check(lib().mic_tensor_desc_set(d, dtype, n, c, h, w, sn, sc, sh, sw), "mic_tensor_desc_set")


def mic_tensor_desc_set_packed(d, dtype, layout, n, c, h, w):
    _check(lib().mic_tensor_desc_set_packed(d, dtype, layout, n, c, h, w), "mic_tensor_desc_set_packed")


def mic_tensor_desc_get(d):
    dt, n, c, h, w = _i(), _i(), _i(), _i(), _i()
    st = (_i64 * 4)()
    _check(lib().mic_tensor_desc_get(d, ctypes.byref(dt), ctypes.byref(n), ctypes.byref(c),
                                     ctypes.byref(h), ctypes.byref(w), st), "mic_tensor_desc_get")
    return dt.value, (n.value, c.value, h.value, w.value), tuple(st)


def mic_tensor_desc_set_blocked(d, dtype, n, c, h, w, cb):
    _check(lib().mic_tensor_desc_set_blocked(d, dtype, n, c, h, w, cb), "mic_tensor_desc_set_blocked")


def mic_tensor_desc_get_block(d):
    cb, sb = _i(), _i64()
    _check(lib().mic_tensor_desc_get_block(d, ctypes.byref(cb), ctypes.byref(sb)), "mic_tensor_desc_get_block")
    return cb.value, sb.value


def mic_filter_desc_create():
    return _create(lib().mic_filter_desc_create, "mic_filter_desc_create")


def mic_filter_desc_destroy(d):
    _check(lib().mic_filter_desc_destroy(d), "mic_filter_desc_destroy")


def mic_filter_desc_set(d, dtype, k, c, r, s):
    _check(lib().mic_filter_desc_set(d, dtype, k, c, r, s), "mic_filter_desc_set")


def mic_filter_desc_set_blocked(d, dtype, k, c, r, s, kb, cb):
    _check(lib().mic_filter_desc_set_blocked(d, dtype, k, c, r, s, kb, cb), "mic_filter_desc_set_blocked")


def mic_filter_desc_get_block(d):
    kb, cb = _i(), _i()
    _check(lib().mic_filter_desc_get_block(d, ctypes.byref(kb), ctypes.byref(cb)), "mic_filter_desc_get_block")
    return kb.value, cb.value


def mic_filter_desc_get(d):
    vals = [_i() for _ in range(5)]
    _check(lib().mic_filter_desc_get(d, *[ctypes.byref(v) for v in vals]), "mic_filter_desc_get")
    return vals[0].value, tuple(v.value for v in vals[1:])


def mic_conv_desc_create():
    return _create(lib().mic_conv_desc_create, "mic_conv_desc_create")


def mic_conv_desc_destroy(d):
    _check(lib().mic_conv_desc_destroy(d), "mic_conv_desc_destroy")


def mic_conv_desc_set(d, pad_top, pad_bottom, pad_left, pad_right, stride_h, stride_w):
    _check(lib().mic_conv_desc_set(d, pad_top, pad_bottom, pad_left, pad_right, stride_h, stride_w),
           "mic_conv_desc_set")


def mic_conv_desc_get(d):
    vals = [_i() for _ in range(6)]
    _check(lib().mic_conv_desc_get(d, *[ctypes.byref(v) for v in vals]), "mic_conv_desc_get")
    return tuple(v.value for v in vals)


def mic_conv_forward_output_dim(conv, x_desc, w_desc):
    vals = [_i() for _ in range(4)]
    _check(lib().mic_conv_forward_output_dim(conv, x_desc, w_desc, *[ctypes.byref(v) for v in vals]),
           "mic_conv_forward_output_dim")
    return tuple(v.value for v in vals)


def mic_conv_forward(handle, alpha, x_desc, x_ptr, w_desc, w_ptr, conv, beta, y_desc, y_ptr):
    _check(lib().mic_conv_forward(handle, float(alpha), x_desc, _vp(x_ptr), w_desc, _vp(w_ptr),
                                  conv, float(beta), y_desc, _vp(y_ptr)), "mic_conv_forward")


def mic_conv_forward_kernel_name(handle, x_desc, w_desc, conv, y_desc):
    buf = ctypes.create_string_buffer(128)
    _check(lib().mic_conv_forward_kernel_name(handle, x_desc, w_desc, conv, y_desc, buf, 128),
           "mic_conv_forward_kernel_name")
    return buf.value.decode()


def mic_conv_backward_data(handle, alpha, w_desc, w_ptr, dy_desc, dy_ptr, conv, beta, dx_desc, dx_ptr):
    _check(lib().mic_conv_backward_data(handle, float(alpha), w_desc, _vp(w_ptr), dy_desc, _vp(dy_ptr),
                                        conv, float(beta), dx_desc, _vp(dx_ptr)), "mic_conv_backward_data")


def mic_conv_backward_data_kernel_name(handle, w_desc, dy_desc, conv, dx_desc):
    buf = ctypes.create_string_buffer(128)
    _check(lib().mic_conv_backward_data_kernel_name(handle, w_desc, dy_desc, conv, dx_desc, buf, 128),
           "mic_conv_backward_data_kernel_name")
    return buf.value.decode()


def mic_conv_backward_filter(handle, alpha, x_desc, x_ptr, dy_desc, dy_ptr, conv, beta, dw_desc, dw_ptr):
    _check(lib().mic_conv_backward_filter(handle, float(alpha), x_desc, _vp(x_ptr), dy_desc, _vp(dy_ptr),
                                          conv, float(beta), dw_desc, _vp(dw_ptr)), "mic_conv_backward_filter")


def mic_conv_backward_filter_kernel_name(handle, x_desc, dy_desc, conv, dw_desc):
    buf = ctypes.create_string_buffer(128)
    _check(lib().mic_conv_backward_filter_kernel_name(handle, x_desc, dy_desc, conv, dw_desc, buf, 128),
           "mic_conv_backward_filter_kernel_name")
    return buf.value.decode()


def mic_pool_desc_create():
    return _create(lib().mic_pool_desc_create, "mic_pool_desc_create")


def mic_pool_desc_destroy(d):
    _check(lib().mic_pool_desc_destroy(d), "mic_pool_desc_destroy")


def mic_pool_desc_set(d, mode, window_h, window_w, pad_top, pad_bottom, pad_left, pad_right, stride_h, stride_w):
    _check(lib().mic_pool_desc_set(d, mode, window_h, window_w, pad_top, pad_bottom, pad_left, pad_right,
                                   stride_h, stride_w), "mic_pool_desc_set")


def mic_pool_desc_get(d):
    vals = [_i() for _ in range(9)]
    _check(lib().mic_pool_desc_get(d, *[ctypes.byref(v) for v in vals]), "mic_pool_desc_get")
    return tuple(v.value for v in vals)


def mic_pool_forward_output_dim(pool, x_desc):
    vals = [_i() for _ in range(4)]
    _check(lib().mic_pool_forward_output_dim(pool, x_desc, *[ctypes.byref(v) for v in vals]),
           "mic_pool_forward_output_dim")
    return tuple(v.value for v in vals)


def mic_pool_forward(handle, alpha, pool, x_desc, x_ptr, beta, y_desc, y_ptr):
    _check(lib().mic_pool_forward(handle, float(alpha), pool, x_desc, _vp(x_ptr), float(beta), y_desc,
                                  _vp(y_ptr)), "mic_pool_forward")


def mic_brgemm(handle, dtype, m, n, k, batch, alpha, a_ptr, a_stride_batch, a_stride_m, a_stride_k, b_ptr,
               b_stride_batch, b_stride_k, b_stride_n, beta, c_ptr, c_stride_m, c_stride_n):
    _check(lib().mic_brgemm(handle, dtype, m, n, k, batch, float(alpha), _vp(a_ptr), a_stride_batch, a_stride_m,
                            a_stride_k, _vp(b_ptr), b_stride_batch, b_stride_k, b_stride_n, float(beta),
                            _vp(c_ptr), c_stride_m, c_stride_n), "mic_brgemm")


def mic_brgemm_kernel_name(handle, dtype, m, n, k, batch, a_stride_batch, a_stride_m, a_stride_k, b_stride_batch,
                           b_stride_k, b_stride_n, c_stride_m, c_stride_n):
    buf = ctypes.create_string_buffer(64)
    _check(lib().mic_brgemm_kernel_name(handle, dtype, m, n, k, batch, a_stride_batch, a_stride_m, a_stride_k,
                                        b_stride_batch, b_stride_k, b_stride_n, c_stride_m, c_stride_n, buf,
                                        len(buf)), "mic_brgemm_kernel_name")
    return buf.value.decode()


# ---------------------------------------------------------------- torch-facing helpers

_handles = {}


def handle_for(device=None):
    """One library handle per device, bound to torch's current stream at call time."""
    dev = torch.cuda.current_device() if device is None else torch.device(device).index
    if dev not in _handles:
        with torch.cuda.device(dev):
            _handles[dev] = mic_create()
    return _handles[dev]


def output_shape(x_shape, w_shape, stride=(1, 1), padding=(0, 0, 0, 0)):
    """(N, K, P, Q) from the library's own output-size rule (host only)."""
    xd, wd, cd = mic_tensor_desc_create(), mic_filter_desc_create(), mic_conv_desc_create()
    try:
        N, C, H, W = x_shape
        mic_tensor_desc_set_packed(xd, MIC_DTYPE_F32, MIC_LAYOUT_NCHW, N, C, H, W)
        mic_filter_desc_set(wd, MIC_DTYPE_F32, *w_shape)
        mic_conv_desc_set(cd, *padding, *stride)
        return mic_conv_forward_output_dim(cd, xd, wd)
    finally:
        mic_tensor_desc_destroy(xd)
        mic_filter_desc_destroy(wd)
        mic_conv_desc_destroy(cd)


def _element_strides(t):
    return tuple(int(s) for s in t.stride())


class ConvPlan:
    """Descriptors for one (x, w, y) triple, reusable across calls.

    x: (N, C, H, W) tensor of any strides; w: contiguous (K, C, R, S);
    y: (N, K, P, Q) tensor of any strides.  Tensors must stay alive and in
    place while the plan is used.
    """

    def __init__(self, x, w, y, stride=(1, 1), padding=(0, 0, 0, 0), handle=None):
        if x.dim() != 4 or w.dim() != 4 or y.dim() != 4:
            raise ValueError("x, w, y must be 4-D")
        if not w.is_contiguous():
            raise ValueError("w must be packed K,C,R,S (contiguous)")
        for t in (x, w, y):
            if t.dtype not in _TORCH_DTYPE:
                raise TypeError("unsupported dtype %s" % t.dtype)
        self.x, self.w, self.y = x, w, y
        self.handle = handle if handle is not None else handle_for(x.device)
        self.xd, self.wd, self.yd = mic_tensor_desc_create(), mic_filter_desc_create(), mic_tensor_desc_create()
        self.cd = mic_conv_desc_create()
        mic_tensor_desc_set(self.xd, _TORCH_DTYPE[x.dtype], *x.shape, *_element_strides(x))
        mic_filter_desc_set(self.wd, _TORCH_DTYPE[w.dtype], *w.shape)
        mic_tensor_desc_set(self.yd, _TORCH_DTYPE[y.dtype], *y.shape, *_element_strides(y))
        mic_conv_desc_set(self.cd, *padding, *stride)
        self.flops = 2.0 * y.shape[0] * y.shape[1] * y.shape[2] * y.shape[3] * w.shape[1] * w.shape[2] * w.shape[3]

    def kernel_name(self):
        return mic_conv_forward_kernel_name(self.handle, self.xd, self.wd, self.cd, self.yd)

    def __call__(self, alpha=1.0, beta=0.0, stream=None):
        s = stream if stream is not None else torch.cuda.current_stream(self.x.device)
        mic_set_stream(self.handle, s.cuda_stream)
        mic_conv_forward(self.handle, alpha, self.xd, self.x.data_ptr(), self.wd, self.w.data_ptr(),
                         self.cd, beta, self.yd, self.y.data_ptr())
        return self.y

    def close(self):
        for d, fn in ((self.xd, mic_tensor_desc_destroy), (self.yd, mic_tensor_desc_destroy),
                      (self.wd, mic_filter_desc_destroy), (self.cd, mic_conv_desc_destroy)):
            if d is not None:
                fn(d)
        self.xd = self.yd = self.wd = self.cd = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def conv2d_forward(x, w, stride=(1, 1), padding=(0, 0, 0, 0), y=None, alpha=1.0, beta=0.0):
    """y <- alpha * conv(x, w) + beta * y on torch's current stream.

    padding = (top, bottom, left, right); stride = (u along H, v along W).
    With y None a new output is allocated (caller memory, in x's memory
    format; fp32 for bf16 inputs) and beta must be 0.
    """
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    N, K, P, Q = output_shape(tuple(x.shape), tuple(w.shape), stride, padding)
    if y is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing y")
        fmt = torch.channels_last if (x.stride(1) == 1 and x.shape[1] > 1) else torch.contiguous_format
        y = torch.empty((N, K, P, Q), dtype=_OUT_DTYPE[x.dtype], device=x.device, memory_format=fmt)
    plan = ConvPlan(x, w.contiguous(), y, stride, padding)
    try:
        plan(alpha, beta)
    finally:
        plan.close()
    return y


class DgradPlan:
    """Descriptors for one data-gradient call (dy, w -> dx), reusable.

    dy: (N, K, P, Q) tensor of any strides; w: contiguous (K, C, R, S);
    dx: (N, C, H, W) tensor of any strides, the forward input's shape.
    """

    def __init__(self, dy, w, dx, stride=(1, 1), padding=(0, 0, 0, 0), handle=None):
        if dy.dim() != 4 or w.dim() != 4 or dx.dim() != 4:
            raise ValueError("dy, w, dx must be 4-D")
        if not w.is_contiguous():
            raise ValueError("w must be packed K,C,R,S (contiguous)")
        for t in (dy, w, dx):
            if t.dtype not in _TORCH_DTYPE:
                raise TypeError("unsupported dtype %s" % t.dtype)
        self.dy, self.w, self.dx = dy, w, dx
        self.handle = handle if handle is not None else handle_for(dy.device)
        self.dyd, self.wd, self.dxd = mic_tensor_desc_create(), mic_filter_desc_create(), mic_tensor_desc_create()
        self.cd = mic_conv_desc_create()
        mic_tensor_desc_set(self.dyd, _TORCH_DTYPE[dy.dtype], *dy.shape, *_element_strides(dy))
        mic_filter_desc_set(self.wd, _TORCH_DTYPE[w.dtype], *w.shape)
        mic_tensor_desc_set(self.dxd, _TORCH_DTYPE[dx.dtype], *dx.shape, *_element_strides(dx))
        mic_conv_desc_set(self.cd, *padding, *stride)
        # the forward pass's multiply-adds, counted once each
        self.flops = 2.0 * dy.shape[0] * dy.shape[1] * dy.shape[2] * dy.shape[3] * w.shape[1] * w.shape[2] * w.shape[3]

    def kernel_name(self):
        return mic_conv_backward_data_kernel_name(self.handle, self.wd, self.dyd, self.cd, self.dxd)

    def __call__(self, alpha=1.0, beta=0.0, stream=None):
        s = stream if stream is not None else torch.cuda.current_stream(self.dy.device)
        mic_set_stream(self.handle, s.cuda_stream)
        mic_conv_backward_data(self.handle, alpha, self.wd, self.w.data_ptr(), self.dyd, self.dy.data_ptr(),
                               self.cd, beta, self.dxd, self.dx.data_ptr())
        return self.dx

    def close(self):
        for d, fn in ((self.dyd, mic_tensor_desc_destroy), (self.dxd, mic_tensor_desc_destroy),
                      (self.wd, mic_filter_desc_destroy), (self.cd, mic_conv_desc_destroy)):
            if d is not None:
                fn(d)
        self.dyd = self.dxd = self.wd = self.cd = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def conv2d_backward_data(dy, w, x_shape, stride=(1, 1), padding=(0, 0, 0, 0), dx=None, alpha=1.0,
                         beta=0.0):
    """dx <- alpha * dgrad(dy, w) + beta * dx on torch's current stream.

    x_shape is the forward input's (N, C, H, W); with dx None a new one is
    allocated (caller memory, in dy's memory format; fp32 for bf16 inputs)
    and beta must be 0.
    """
    if not dy.is_cuda:
        raise ValueError("dy must be a GPU tensor")
    if dx is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing dx")
        fmt = torch.channels_last if (dy.stride(1) == 1 and dy.shape[1] > 1) else torch.contiguous_format
        dx = torch.empty(tuple(x_shape), dtype=_OUT_DTYPE[dy.dtype], device=dy.device, memory_format=fmt)
    plan = DgradPlan(dy, w.contiguous(), dx, stride, padding)
    try:
        plan(alpha, beta)
    finally:
        plan.close()
    return dx


class WgradPlan:
    """Descriptors for one filter-gradient call (x, dy -> dw), reusable.

    x: (N, C, H, W) and dy: (N, K, P, Q) tensors of any strides;
    dw: contiguous (K, C, R, S) (fp32 for bf16 inputs).
    """

    def __init__(self, x, dy, dw, stride=(1, 1), padding=(0, 0, 0, 0), handle=None):
        if x.dim() != 4 or dy.dim() != 4 or dw.dim() != 4:
            raise ValueError("x, dy, dw must be 4-D")
        if not dw.is_contiguous():
            raise ValueError("dw must be packed K,C,R,S (contiguous)")
        for t in (x, dy, dw):
            if t.dtype not in _TORCH_DTYPE:
                raise TypeError("unsupported dtype %s" % t.dtype)
        self.x, self.dy, self.dw = x, dy, dw
        self.handle = handle if handle is not None else handle_for(x.device)
        self.xd, self.dyd, self.wd = mic_tensor_desc_create(), mic_tensor_desc_create(), mic_filter_desc_create()
        self.cd = mic_conv_desc_create()
        mic_tensor_desc_set(self.xd, _TORCH_DTYPE[x.dtype], *x.shape, *_element_strides(x))
        mic_tensor_desc_set(self.dyd, _TORCH_DTYPE[dy.dtype], *dy.shape, *_element_strides(dy))
        mic_filter_desc_set(self.wd, _TORCH_DTYPE[dw.dtype], *dw.shape)
        mic_conv_desc_set(self.cd, *padding, *stride)
        # the forward pass's multiply-adds, counted once each
        self.flops = 2.0 * dy.shape[0] * dy.shape[1] * dy.shape[2] * dy.shape[3] * dw.shape[1] * dw.shape[2] * dw.shape[3]

    def kernel_name(self):
        return mic_conv_backward_filter_kernel_name(self.handle, self.xd, self.dyd, self.cd, self.wd)

    def __call__(self, alpha=1.0, beta=0.0, stream=None):
        s = stream if stream is not None else torch.cuda.current_stream(self.x.device)
        mic_set_stream(self.handle, s.cuda_stream)
        mic_conv_backward_filter(self.handle, alpha, self.xd, self.x.data_ptr(), self.dyd, self.dy.data_ptr(),
                                 self.cd, beta, self.wd, self.dw.data_ptr())
        return self.dw

    def close(self):
        for d, fn in ((self.xd, mic_tensor_desc_destroy), (self.dyd, mic_tensor_desc_destroy),
                      (self.wd, mic_filter_desc_destroy), (self.cd, mic_conv_desc_destroy)):
            if d is not None:
                fn(d)
        self.xd = self.dyd = self.wd = self.cd = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def conv2d_backward_filter(x, dy, w_shape, stride=(1, 1), padding=(0, 0, 0, 0), dw=None, alpha=1.0,
                           beta=0.0):
    """dw <- alpha * wgrad(x, dy) + beta * dw on torch's current stream.

    w_shape is the filter's (K, C, R, S); with dw None a new packed one is
    allocated (caller memory; fp32 for bf16 inputs) and beta must be 0.
    """
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if dw is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing dw")
        dw = torch.empty(tuple(w_shape), dtype=_OUT_DTYPE[x.dtype], device=x.device)
    plan = WgradPlan(x, dy, dw, stride, padding)
    try:
        plan(alpha, beta)
    finally:
        plan.close()
    return dw


def pool_output_shape(x_shape, window, stride=(1, 1), padding=(0, 0, 0, 0), mode="max"):
    """(N, C, P, Q) from the library's own output-size rule (host only)."""
    xd, pd = mic_tensor_desc_create(), mic_pool_desc_create()
    try:
        mic_tensor_desc_set_packed(xd, MIC_DTYPE_F32, MIC_LAYOUT_NCHW, *x_shape)
        mic_pool_desc_set(pd, POOL_MODES[mode], *window, *padding, *stride)
        return mic_pool_forward_output_dim(pd, xd)
    finally:
        mic_tensor_desc_destroy(xd)
        mic_pool_desc_destroy(pd)


class PoolPlan:
    """Descriptors for one pooling call (x -> y), reusable.  mode in POOL_MODES."""

    def __init__(self, x, y, window, stride=(1, 1), padding=(0, 0, 0, 0), mode="max", handle=None):
        if x.dim() != 4 or y.dim() != 4:
            raise ValueError("x, y must be 4-D")
        for t in (x, y):
            if t.dtype not in _TORCH_DTYPE:
                raise TypeError("unsupported dtype %s" % t.dtype)
        self.x, self.y = x, y
        self.handle = handle if handle is not None else handle_for(x.device)
        self.xd, self.yd, self.pd = mic_tensor_desc_create(), mic_tensor_desc_create(), mic_pool_desc_create()
        mic_tensor_desc_set(self.xd, _TORCH_DTYPE[x.dtype], *x.shape, *_element_strides(x))
        mic_tensor_desc_set(self.yd, _TORCH_DTYPE[y.dtype], *y.shape, *_element_strides(y))
        mic_pool_desc_set(self.pd, POOL_MODES[mode], *window, *padding, *stride)
        # algorithmic bytes: x read once, y written once
        self.bytes = x.numel() * x.element_size() + y.numel() * y.element_size()

    def kernel_name(self):
        return "pool_direct"

    def __call__(self, alpha=1.0, beta=0.0, stream=None):
        s = stream if stream is not None else torch.cuda.current_stream(self.x.device)
        mic_set_stream(self.handle, s.cuda_stream)
        mic_pool_forward(self.handle, alpha, self.pd, self.xd, self.x.data_ptr(), beta, self.yd, self.y.data_ptr())
        return self.y

    def close(self):
        for d, fn in ((self.xd, mic_tensor_desc_destroy), (self.yd, mic_tensor_desc_destroy),
                      (self.pd, mic_pool_desc_destroy)):
            if d is not None:
                fn(d)
        self.xd = self.yd = self.pd = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pool2d_forward(x, window, stride=(1, 1), padding=(0, 0, 0, 0), mode="max", y=None, alpha=1.0, beta=0.0):
    """y <- alpha * pool(x) + beta * y on torch's current stream (y allocated if None, beta then 0)."""
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    shape = pool_output_shape(tuple(x.shape), window, stride, padding, mode)
    if y is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing y")
        fmt = torch.channels_last if (x.stride(1) == 1 and x.shape[1] > 1) else torch.contiguous_format
        y = torch.empty(shape, dtype=_OUT_DTYPE[x.dtype], device=x.device, memory_format=fmt)
    plan = PoolPlan(x, y, window, stride, padding, mode)
    try:
        plan(alpha, beta)
    finally:
        plan.close()
    return y


def brgemm(a, b, c=None, alpha=1.0, beta=0.0):
    """c <- alpha * sum_i a[i] @ b[i] + beta * c on torch's current stream.

    a: (batch, m, k) and b: (batch, k, n) GPU tensors of one dtype (any
    element strides, e.g. views of blocks of a larger matrix); c: (m, n),
    allocated when None (fp32 for bf16 inputs; beta must then be 0).
    """
    if not a.is_cuda or not b.is_cuda:
        raise ValueError("a and b must be GPU tensors")
    if a.dim() != 3 or b.dim() != 3:
        raise ValueError("a must be (batch, m, k) and b (batch, k, n)")
    batch, m, k = a.shape
    if b.shape[0] != batch or b.shape[1] != k:
        raise ValueError("a %s and b %s do not chain" % (tuple(a.shape), tuple(b.shape)))
    if a.dtype != b.dtype or a.dtype not in _TORCH_DTYPE:
        raise TypeError("a and b need one supported dtype, got %s and %s" % (a.dtype, b.dtype))
    n = b.shape[2]
    if c is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing c")
        c = torch.empty((m, n), dtype=_OUT_DTYPE[a.dtype], device=a.device)
    if c.dim() != 2 or tuple(c.shape) != (m, n) or c.dtype != _OUT_DTYPE[a.dtype]:
        raise ValueError("c must be (%d, %d) of %s" % (m, n, _OUT_DTYPE[a.dtype]))
    h = handle_for(a.device)
    mic_set_stream(h, torch.cuda.current_stream(a.device).cuda_stream)
    mic_brgemm(h, _TORCH_DTYPE[a.dtype], m, n, k, batch, alpha, a.data_ptr(), *a.stride(), b.data_ptr(),
               *b.stride(), beta, c.data_ptr(), *c.stride())
    return c


def brgemm_kernel_name(dtype, m, n, k, batch=1, a_strides=None, b_strides=None, c_strides=None):
    """Kernel variant mic_brgemm picks (host only; dtype a torch dtype).

    Strides in elements as mic_brgemm takes them; by default A (batch, m, k),
    B (batch, k, n) and C (m, n) packed row-major.  Also accepts tensors'
    .stride() tuples."""
    sa = tuple(a_strides) if a_strides is not None else (m * k, k, 1)
    sb = tuple(b_strides) if b_strides is not None else (k * n, n, 1)
    sc = tuple(c_strides) if c_strides is not None else (n, 1)
    return mic_brgemm_kernel_name(None, _TORCH_DTYPE[dtype], m, n, k, batch, *sa, *sb, *sc)


def brgemm_kernel_name_for(a, b, c):
    """Kernel variant mic_brgemm picks for these tensors (as brgemm() would pass them)."""
    batch, m, k = a.shape
    return brgemm_kernel_name(a.dtype, m, b.shape[2], k, batch, a.stride(), b.stride(), c.stride())


# ---------------------------------------------------------------- channel-blocked layouts

def to_blocked(t, cb):
    """(N, C, H, W) -> packed channel-blocked (N, C/cb, H, W, cb) (a copy; C % cb == 0)."""
    n, c, h, w = t.shape
    if c % cb:
        raise ValueError("C = %d is not a multiple of the block %d" % (c, cb))
    return t.reshape(n, c // cb, cb, h, w).permute(0, 1, 3, 4, 2).contiguous()


def from_blocked(tb):
    """(N, C/cb, H, W, cb) -> logical (N, C, H, W) view."""
    n, nb, h, w, cb = tb.shape
    return tb.permute(0, 1, 4, 2, 3).reshape(n, nb * cb, h, w)


def filters_to_blocked(f, kb, cb):
    """(K, C, R, S) -> packed blocked filters (K/kb, C/cb, R, S, cb, kb) (a copy)."""
    k, c, r, s = f.shape
    if k % kb or c % cb:
        raise ValueError("K, C = %d, %d are not multiples of the blocks %d, %d" % (k, c, kb, cb))
    return f.reshape(k // kb, kb, c // cb, cb, r, s).permute(0, 2, 4, 5, 3, 1).contiguous()


def filters_from_blocked(fb):
    """(K/kb, C/cb, R, S, cb, kb) -> logical (K, C, R, S) view."""
    nk, nc, r, s, cb, kb = fb.shape
    return fb.permute(0, 5, 1, 4, 2, 3).reshape(nk * kb, nc * cb, r, s)


class BlockedConvPlan(ConvPlan):
    """ConvPlan for channel-blocked operands.

    x: (N, C, H, W) of any strides, or channel-blocked (N, C/cb, H, W, cb)
    contiguous; y likewise with the output channels; w: packed (K, C, R, S)
    or blocked (K/kb, C/cb, R, S, cb, kb) contiguous.  Logical shapes follow
    from the blocked ones.
    """

    def __init__(self, x, w, y, stride=(1, 1), padding=(0, 0, 0, 0), handle=None):
        for t in (x, w, y):
            if t.dtype not in _TORCH_DTYPE:
                raise TypeError("unsupported dtype %s" % t.dtype)
        if x.dim() not in (4, 5) or y.dim() not in (4, 5) or w.dim() not in (4, 6):
            raise ValueError("x, y must be 4-D or blocked 5-D, w 4-D or blocked 6-D")
        for t in (x, w, y):
            if t.dim() > 4 and not t.is_contiguous():
                raise ValueError("blocked operands must be contiguous")
        if w.dim() == 4 and not w.is_contiguous():
            raise ValueError("w must be packed K,C,R,S (contiguous)")
        self.x, self.w, self.y = x, w, y
        self.handle = handle if handle is not None else handle_for(x.device)
        self.xd, self.wd, self.yd = mic_tensor_desc_create(), mic_filter_desc_create(), mic_tensor_desc_create()
        self.cd = mic_conv_desc_create()

        def set_act(d, t):
            if t.dim() == 5:
                n, nb, h, w_, cb = t.shape
                mic_tensor_desc_set_blocked(d, _TORCH_DTYPE[t.dtype], n, nb * cb, h, w_, cb)
                return (n, nb * cb, h, w_)
            mic_tensor_desc_set(d, _TORCH_DTYPE[t.dtype], *t.shape, *_element_strides(t))
            return tuple(t.shape)

        xs = set_act(self.xd, x)
        ys = set_act(self.yd, y)
        if w.dim() == 6:
            nk, nc, r, s_, cb, kb = w.shape
            mic_filter_desc_set_blocked(self.wd, _TORCH_DTYPE[w.dtype], nk * kb, nc * cb, r, s_, kb, cb)
            ws = (nk * kb, nc * cb, r, s_)
        else:
            mic_filter_desc_set(self.wd, _TORCH_DTYPE[w.dtype], *w.shape)
            ws = tuple(w.shape)
        mic_conv_desc_set(self.cd, *padding, *stride)
        self.shapes = (xs, ws, ys)
        self.flops = 2.0 * ys[0] * ys[1] * ys[2] * ys[3] * ws[1] * ws[2] * ws[3]

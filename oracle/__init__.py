"""CPU oracle for the 2-D convolution forward pass, its data and filter
gradients, pooling and the batch-reduce GEMM (fp64, plain nested loops).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library and never imports it.

The arithmetic lives in ``conv_oracle.c`` (see its header for the definition
and the page passages it follows: maxDNN "Proposed Method", the zero-memory
direct-convolution page's Abstract and "Proposed Method", and the cuDNN
page's "Proposed Method").  This module only builds that file with gcc,
loads it, and marshals numpy arrays in and out.

Every function here is pinned by ``tests/test_oracle.py`` against a dense
Toeplitz-matrix product, closed forms and invariants.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(verbose=False):
    """Compile conv_oracle.c into liboracle.so (gcc, OpenMP, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-std=c11", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)


class Problem(ctypes.Structure):
    """Field-for-field mirror of ``oracle_conv_problem`` in conv_oracle.c."""
    _fields_ = [(name, ctypes.c_int64) for name in (
        "N", "C", "H", "W", "sn", "sc", "sh", "sw", "K", "R", "S",
        "pad_top", "pad_bottom", "pad_left", "pad_right", "u", "v")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")      # a mutant build, for the pin self-test
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        pp = ctypes.POINTER(Problem)
        lib.oracle_output_dims.argtypes = [pp, ip, ip]
        lib.oracle_output_dims.restype = ctypes.c_int
        lib.oracle_conv2d_fprop.argtypes = [pp, dp, dp, ctypes.c_double, ctypes.c_double,
                                            dp, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_fprop.restype = ctypes.c_int
        lib.oracle_conv2d_fprop_at.argtypes = [pp, dp, dp, ctypes.c_double, ctypes.c_double,
                                               dp, ip, ctypes.c_int64, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_fprop_at.restype = ctypes.c_int
        lib.oracle_conv2d_bwd_data.argtypes = [pp, dp, ip, dp, ctypes.c_double, ctypes.c_double,
                                               dp, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_bwd_data.restype = ctypes.c_int
        lib.oracle_conv2d_bwd_data_at.argtypes = [pp, dp, ip, dp, ctypes.c_double, ctypes.c_double,
                                                  dp, ip, ctypes.c_int64, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_bwd_data_at.restype = ctypes.c_int
        lib.oracle_conv2d_bwd_filter.argtypes = [pp, dp, dp, ip, ctypes.c_double, ctypes.c_double,
                                                 dp, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_bwd_filter.restype = ctypes.c_int
        lib.oracle_conv2d_bwd_filter_at.argtypes = [pp, dp, dp, ip, ctypes.c_double, ctypes.c_double,
                                                    dp, ip, ctypes.c_int64, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_bwd_filter_at.restype = ctypes.c_int
        lib.oracle_pool_forward.argtypes = [pp, dp, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                            dp, dp, ctypes.c_int]
        lib.oracle_pool_forward.restype = ctypes.c_int
        i64 = ctypes.c_int64
        lib.oracle_brgemm.argtypes = [i64, i64, i64, i64, dp, i64, i64, i64, dp, i64, i64, i64,
                                      ctypes.c_double, ctypes.c_double, dp, dp, dp, ctypes.c_int]
        lib.oracle_brgemm.restype = ctypes.c_int
        lib.oracle_default_threads.argtypes = []
        lib.oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads():
    return int(_load().oracle_default_threads())


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def _input_view(x):
    """(base array, element strides) of a float64 ndarray view, without copying.

    The oracle reads x through element strides, so NCHW, NHWC and padded-row
    views all reach it as they are.
    """
    if x.dtype != np.float64:
        raise TypeError("oracle inputs are float64 (widen fp32/bf16 exactly first)")
    if x.ndim != 4:
        raise ValueError("x must be 4-D (N, C, H, W) in logical order")
    strides = [s // 8 for s in x.strides]
    if any(s * 8 != b for s, b in zip(strides, x.strides)) or any(s < 0 for s in strides):
        raise ValueError("x strides must be non-negative multiples of 8 bytes")
    return x, strides


def make_problem(x_shape, x_strides, w_shape, stride=(1, 1), padding=(0, 0, 0, 0)):
    """padding = (top, bottom, left, right); stride = (u along H, v along W)."""
    N, C, H, W = x_shape
    K, C2, R, S = w_shape
    if C2 != C:
        raise ValueError("filter C %d != input C %d" % (C2, C))
    pt, pb, pl, pr = padding
    return Problem(N, C, H, W, *x_strides, K, R, S, pt, pb, pl, pr, stride[0], stride[1])


def output_dims(pb):
    P = ctypes.c_int64()
    Q = ctypes.c_int64()
    if _load().oracle_output_dims(ctypes.byref(pb), ctypes.byref(P), ctypes.byref(Q)) != 0:
        raise ValueError("malformed convolution problem or empty output")
    return P.value, Q.value


def conv2d_fprop(x, w, stride=(1, 1), padding=(0, 0, 0, 0), alpha=1.0, beta=0.0,
                 y_old=None, nthreads=0):
    """Whole output.  Returns (y, bound), both float64 packed (N, K, P, Q).

    x: float64 (N, C, H, W), any non-negative strides (a view is fine).
    w: float64 (K, C, R, S); made contiguous (packed K,C,R,S) here.
    """
    xb, xs = _input_view(x)
    wc = np.ascontiguousarray(w, dtype=np.float64)
    pb = make_problem(x.shape, xs, wc.shape, stride, padding)
    P, Q = output_dims(pb)
    N, K = x.shape[0], wc.shape[0]
    y = np.empty((N, K, P, Q), dtype=np.float64)
    bound = np.empty((N, K, P, Q), dtype=np.float64)
    yo = None
    if beta != 0.0:
        if y_old is None:
            raise ValueError("beta != 0 needs y_old")
        yo = np.ascontiguousarray(y_old, dtype=np.float64)
        if yo.shape != y.shape:
            raise ValueError("y_old shape %s != output shape %s" % (yo.shape, y.shape))
    rc = _load().oracle_conv2d_fprop(ctypes.byref(pb), _dptr(xb), _dptr(wc), float(alpha),
                                     float(beta), _dptr(yo), _dptr(y), _dptr(bound),
                                     int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return y, bound


def conv2d_fprop_at(x, w, idx, stride=(1, 1), padding=(0, 0, 0, 0), alpha=1.0, beta=0.0,
                    y_old_vals=None, nthreads=0):
    """Selected outputs.  idx: int64 array (count, 4) of (n, k, p, q).

    Returns (y_vals, bound_vals), float64 arrays of length count.
    """
    xb, xs = _input_view(x)
    wc = np.ascontiguousarray(w, dtype=np.float64)
    pb = make_problem(x.shape, xs, wc.shape, stride, padding)
    ic = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 4)
    count = ic.shape[0]
    y = np.empty(count, dtype=np.float64)
    bound = np.empty(count, dtype=np.float64)
    yo = None
    if beta != 0.0:
        if y_old_vals is None:
            raise ValueError("beta != 0 needs y_old_vals")
        yo = np.ascontiguousarray(y_old_vals, dtype=np.float64).reshape(-1)
        if yo.shape[0] != count:
            raise ValueError("y_old_vals must hold one value per coordinate")
    rc = _load().oracle_conv2d_fprop_at(
        ctypes.byref(pb), _dptr(xb), _dptr(wc), float(alpha), float(beta), _dptr(yo),
        ic.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), count, _dptr(y), _dptr(bound),
        int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem or a coordinate")
    return y, bound


def _dgrad_problem(dy, w, x_shape, stride, padding):
    db, ds = _input_view(dy)
    wc = np.ascontiguousarray(w, dtype=np.float64)
    N, C, H, W = x_shape
    # the forward problem of the same geometry; its input strides are unused
    pb = make_problem(x_shape, (C * H * W, H * W, W, 1), wc.shape, stride, padding)
    P, Q = output_dims(pb)
    if tuple(dy.shape) != (N, wc.shape[0], P, Q):
        raise ValueError("dy shape %s != forward output shape %s" % (tuple(dy.shape), (N, wc.shape[0], P, Q)))
    sdy = np.asarray(ds, dtype=np.int64)
    return pb, db, sdy, wc


def conv2d_bwd_data(dy, w, x_shape, stride=(1, 1), padding=(0, 0, 0, 0), alpha=1.0, beta=0.0,
                    dx_old=None, nthreads=0):
    """Whole data gradient of the forward convolution with input shape x_shape.

    dy: float64 (N, K, P, Q), any non-negative strides; w: float64 (K, C, R, S).
    Returns (dx, bound), both float64 packed (N, C, H, W).
    """
    pb, db, sdy, wc = _dgrad_problem(dy, w, x_shape, stride, padding)
    dx = np.empty(tuple(x_shape), dtype=np.float64)
    bound = np.empty(tuple(x_shape), dtype=np.float64)
    xo = None
    if beta != 0.0:
        if dx_old is None:
            raise ValueError("beta != 0 needs dx_old")
        xo = np.ascontiguousarray(dx_old, dtype=np.float64)
        if xo.shape != dx.shape:
            raise ValueError("dx_old shape %s != input shape %s" % (xo.shape, dx.shape))
    rc = _load().oracle_conv2d_bwd_data(
        ctypes.byref(pb), _dptr(db), sdy.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(wc),
        float(alpha), float(beta), _dptr(xo), _dptr(dx), _dptr(bound), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return dx, bound


def conv2d_bwd_data_at(dy, w, x_shape, idx, stride=(1, 1), padding=(0, 0, 0, 0), alpha=1.0,
                       beta=0.0, dx_old_vals=None, nthreads=0):
    """Selected data-gradient values.  idx: int64 array (count, 4) of (n, c, h, w)."""
    pb, db, sdy, wc = _dgrad_problem(dy, w, x_shape, stride, padding)
    ic = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 4)
    count = ic.shape[0]
    dx = np.empty(count, dtype=np.float64)
    bound = np.empty(count, dtype=np.float64)
    xo = None
    if beta != 0.0:
        if dx_old_vals is None:
            raise ValueError("beta != 0 needs dx_old_vals")
        xo = np.ascontiguousarray(dx_old_vals, dtype=np.float64).reshape(-1)
        if xo.shape[0] != count:
            raise ValueError("dx_old_vals must hold one value per coordinate")
    rc = _load().oracle_conv2d_bwd_data_at(
        ctypes.byref(pb), _dptr(db), sdy.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(wc),
        float(alpha), float(beta), _dptr(xo), ic.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        count, _dptr(dx), _dptr(bound), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem or a coordinate")
    return dx, bound


def conv2d_bwd_filter(x, dy, w_shape, stride=(1, 1), padding=(0, 0, 0, 0), alpha=1.0, beta=0.0,
                      dw_old=None, nthreads=0):
    """Whole filter gradient of the forward convolution of x with a (K, C, R, S) filter.

    x: float64 (N, C, H, W) and dy: float64 (N, K, P, Q), any non-negative strides.
    Returns (dw, bound), both float64 packed (K, C, R, S).
    """
    xb, xs = _input_view(x)
    db, ds = _input_view(dy)
    pb = make_problem(x.shape, xs, tuple(w_shape), stride, padding)
    P, Q = output_dims(pb)
    if tuple(dy.shape) != (x.shape[0], w_shape[0], P, Q):
        raise ValueError("dy shape %s != forward output shape %s" % (tuple(dy.shape), (x.shape[0], w_shape[0], P, Q)))
    sdy = np.asarray(ds, dtype=np.int64)
    dw = np.empty(tuple(w_shape), dtype=np.float64)
    bound = np.empty(tuple(w_shape), dtype=np.float64)
    wo = None
    if beta != 0.0:
        if dw_old is None:
            raise ValueError("beta != 0 needs dw_old")
        wo = np.ascontiguousarray(dw_old, dtype=np.float64)
        if wo.shape != dw.shape:
            raise ValueError("dw_old shape %s != filter shape %s" % (wo.shape, dw.shape))
    rc = _load().oracle_conv2d_bwd_filter(
        ctypes.byref(pb), _dptr(xb), _dptr(db), sdy.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        float(alpha), float(beta), _dptr(wo), _dptr(dw), _dptr(bound), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return dw, bound


def conv2d_bwd_filter_at(x, dy, w_shape, idx, stride=(1, 1), padding=(0, 0, 0, 0), alpha=1.0, beta=0.0,
                         dw_old_vals=None, nthreads=0):
    """Selected filter-gradient values.  idx: int64 array (count, 4) of (k, c, r, s)."""
    xb, xs = _input_view(x)
    db, ds = _input_view(dy)
    pb = make_problem(x.shape, xs, tuple(w_shape), stride, padding)
    P, Q = output_dims(pb)
    if tuple(dy.shape) != (x.shape[0], w_shape[0], P, Q):
        raise ValueError("dy shape %s != forward output shape %s" % (tuple(dy.shape), (x.shape[0], w_shape[0], P, Q)))
    sdy = np.asarray(ds, dtype=np.int64)
    ic = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 4)
    count = ic.shape[0]
    dw = np.empty(count, dtype=np.float64)
    bound = np.empty(count, dtype=np.float64)
    wo = None
    if beta != 0.0:
        if dw_old_vals is None:
            raise ValueError("beta != 0 needs dw_old_vals")
        wo = np.ascontiguousarray(dw_old_vals, dtype=np.float64).reshape(-1)
    rc = _load().oracle_conv2d_bwd_filter_at(
        ctypes.byref(pb), _dptr(xb), _dptr(db), sdy.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        float(alpha), float(beta), _dptr(wo), ic.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), count,
        _dptr(dw), _dptr(bound), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem or a coordinate")
    return dw, bound


POOL_MODES = {"max": 0, "avg_include_pad": 1, "avg_exclude_pad": 2}


def pool2d_forward(x, window, stride=(1, 1), padding=(0, 0, 0, 0), mode="max", alpha=1.0, beta=0.0,
                   y_old=None, nthreads=0):
    """Pooled output, float64 packed (N, C, P, Q).  window = (R, S); mode in POOL_MODES."""
    xb, xs = _input_view(x)
    N, C = x.shape[:2]
    pb = make_problem(x.shape, xs, (1, C) + tuple(window), stride, padding)
    P, Q = output_dims(pb)
    y = np.empty((N, C, P, Q), dtype=np.float64)
    yo = None
    if beta != 0.0:
        if y_old is None:
            raise ValueError("beta != 0 needs y_old")
        yo = np.ascontiguousarray(y_old, dtype=np.float64)
        if yo.shape != y.shape:
            raise ValueError("y_old shape %s != output shape %s" % (yo.shape, y.shape))
    rc = _load().oracle_pool_forward(ctypes.byref(pb), _dptr(xb), POOL_MODES[mode], float(alpha), float(beta),
                                     _dptr(yo), _dptr(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return y


def brgemm(a, b, alpha=1.0, beta=0.0, c_old=None, nthreads=0):
    """Batch-reduce GEMM: C = alpha * sum_i a[i] @ b[i] + beta * c_old.

    a: float64 (batch, M, K), b: float64 (batch, K, N), any non-negative
    strides (views are fine).  Returns (C, bound), float64 packed (M, N).
    """
    if a.dtype != np.float64 or b.dtype != np.float64:
        raise TypeError("oracle inputs are float64")
    if a.ndim != 3 or b.ndim != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[1]:
        raise ValueError("shapes must be (batch, M, K) and (batch, K, N)")
    sa = [s // 8 for s in a.strides]
    sb = [s // 8 for s in b.strides]
    if any(s < 0 for s in sa + sb):
        raise ValueError("strides must be non-negative")
    batch, M, K = a.shape
    N = b.shape[2]
    c = np.empty((M, N))
    bound = np.empty((M, N))
    co = None
    if beta != 0.0:
        if c_old is None:
            raise ValueError("beta != 0 needs c_old")
        co = np.ascontiguousarray(c_old, dtype=np.float64)
    rc = _load().oracle_brgemm(M, N, K, batch, _dptr(a), sa[0], sa[1], sa[2], _dptr(b), sb[0], sb[1], sb[2],
                               float(alpha), float(beta), _dptr(co), _dptr(c), _dptr(bound), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return c, bound

"""Shared helpers for the GPU parity tests: seeded inputs, device layouts,
oracle comparison with the tolerances of each element type.

Tolerances (per element type, fixed in the tests, not tuned to results):
  f32 : relative L2 error <= 1e-5 and |y - y_ref| <= 2e-6 * B per element,
        B = sum |x*f| over the receptive field (the oracle returns it);
        with alpha/beta the bound is 2e-6 * (|alpha| B + |beta y_old|).
        The filter gradient sums over N*P*Q positions, up to 50x more terms
        than any forward sum: its relative-L2 gate grows with the square
        root of the reduction length (rel_l2_scale), the per-element bound
        does not change.
  f64 : relative L2 error <= 1e-12.
  bf16: relative L2 error <= 1e-2 (bf16 inputs, fp32 accumulation and output).
        The oracle reads the same bf16-rounded inputs and the kernels
        accumulate in fp32, so the fp32 per-element bound 2e-6 * B is
        asserted as well: a packing slip that touches a few outputs breaks it
        long before it moves the relative L2 error past 1e-2.
"""
import numpy as np
import torch

import gen
import oracle
from gen import workloads

TORCH_DT = {"f32": torch.float32, "f64": torch.float64, "bf16": torch.bfloat16}
OUT_DT = {"f32": torch.float32, "f64": torch.float64, "bf16": torch.float32}
RELL2 = {"f32": 1e-5, "f64": 1e-12, "bf16": 1e-2}
ELEM_BOUND = {"f32": 2e-6, "bf16": 2e-6}


def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda", 0)


def inputs(lay, x_dist=None, w_dist=None):
    """float64 numpy x (N,C,H,W), w (K,C,R,S), rounded to the layer's storage type."""
    x = gen.draw(x_dist or lay.x_dist, gen.derive_seed(lay.config, lay.layer, 0), lay.x_shape)
    w = gen.draw(w_dist or lay.w_dist, gen.derive_seed(lay.config, lay.layer, 1), lay.w_shape)
    return gen.round_to(x, lay.dtype), gen.round_to(w, lay.dtype)


def strided_empty(shape, strides, dtype, device, fill=float("nan")):
    """A tensor view of the given element strides over a fresh allocation."""
    N, C, H, W = shape
    n = workloads.storage_elems(N, C, H, W, strides)
    base = torch.full((n,), fill, dtype=dtype, device=device)
    return base.as_strided(shape, strides)


# NaN canary cells placed directly before and after an output's storage
GUARD = 4096


def guarded_empty(shape, strides, dtype, device=None):
    """A NaN-filled strided tensor inside one allocation that also holds GUARD
    NaN cells before and after it (and, for padded strides, the pad cells
    between its rows).  Returns (tensor, whole allocation)."""
    device = device or dev()
    n = workloads.storage_elems(*shape, strides)
    base = torch.full((n + 2 * GUARD,), float("nan"), dtype=dtype, device=device)
    return base.as_strided(shape, strides, GUARD), base


def assert_only_tensor_written(t, base, what=""):
    """Every cell of the allocation that is not an element of t still holds NaN."""
    mask = torch.zeros(base.numel(), dtype=torch.bool, device=base.device)
    mask.as_strided(t.shape, t.stride(), t.storage_offset()).fill_(True)
    outside = base[~mask]
    bad = int((~torch.isnan(outside)).sum())
    assert bad == 0, "%s: %d cells outside the output were written" % (what, bad)


def to_device(a64, dtype_key, layout="nchw", row_pitch=0, device=None):
    """Upload logical N,C,H,W float64 data into a tensor of the given layout."""
    device = device or dev()
    N, C, H, W = a64.shape
    st = workloads.padded_strides(N, C, H, W, layout, row_pitch)
    t = strided_empty(a64.shape, st, TORCH_DT[dtype_key], device)
    t.copy_(torch.from_numpy(a64).to(TORCH_DT[dtype_key]))
    return t


def out_tensor(lay, shape, device=None, fill=float("nan")):
    device = device or dev()
    st = workloads.padded_strides(*shape, lay.layout, lay.row_pitch)
    return strided_empty(shape, st, OUT_DT[lay.dtype], device, fill)


def guarded_out(lay, shape):
    """out_tensor's layout, NaN-filled, with canary cells around it: (tensor, allocation)."""
    st = workloads.padded_strides(*shape, lay.layout, lay.row_pitch)
    return guarded_empty(shape, st, OUT_DT[lay.dtype])


def full_order(layers):
    """Layers ordered so that the layouts of one logical layer (same config,
    layer and element type: the same generated values) run one after another
    and share one oracle result."""
    return sorted(layers, key=lambda l: (l.config, l.dtype, l.layer, l.layout))


def to_host(t):
    """Device tensor -> float64 numpy in logical N,C,H,W order."""
    return t.double().cpu().numpy()


def sample_coords(rng, N, K, P, Q, count):
    """Random output coordinates plus every corner and edge midpoint."""
    pts = {(n, k, p, q) for n in (0, N - 1) for k in (0, K // 2, K - 1)
           for p in (0, P // 2, P - 1) for q in (0, Q // 2, Q - 1)}
    rnd = np.stack([rng.integers(0, N, count), rng.integers(0, K, count),
                    rng.integers(0, P, count), rng.integers(0, Q, count)], axis=1)
    return np.concatenate([np.array(sorted(pts), dtype=np.int64), rnd.astype(np.int64)])


def gather(y, idx):
    t = torch.from_numpy(idx).to(y.device)
    return y[t[:, 0], t[:, 1], t[:, 2], t[:, 3]].double().cpu().numpy()


# The forward pass's longest reduction in the workloads (Overfeat L5: C*R*S).
FWD_MAX_REDUCTION = 1024 * 9


def rel_l2_scale(reduction_length):
    """Factor on the fp32/bf16 relative-L2 gate for a reduction of the given length.

    The gate is stated for the forward pass, whose sums run over at most
    C*R*S = 9216 terms.  With terms of mixed sign, the rounding error of an
    fp32 sum of L terms relative to its value grows like u * sqrt(L) (the
    partial sums and their roundings both random-walk), so a sum over
    L > 9216 terms gets the gate times sqrt(L / 9216); never less than 1.
    """
    return max(1.0, float(np.sqrt(reduction_length / FWD_MAX_REDUCTION)))


def check(dtype_key, got, ref, bound, alpha=1.0, beta=0.0, y_old=None, what="", rel_scale=1.0):
    """Assert the element type's tolerance; return (rel_l2, max_err/bound).

    rel_scale multiplies the relative-L2 gate (see rel_l2_scale); the
    per-element bound 2e-6 * B is never relaxed."""
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    gate = RELL2[dtype_key] * (rel_scale if dtype_key != "f64" else 1.0)
    assert rel <= gate, "%s: relative L2 error %.3e > %.1e" % (what, rel, gate)
    worst = 0.0
    if dtype_key in ELEM_BOUND:
        scale = abs(alpha) * bound
        if beta != 0.0:
            scale = scale + np.abs(beta * y_old)
        lim = ELEM_BOUND[dtype_key] * scale
        bad = np.abs(diff) > lim
        assert not np.any(bad), "%s: %d elements beyond 2e-6*B (worst ratio %.3g)" % (
            what, int(bad.sum()), float(np.max(np.abs(diff)[bad] / np.maximum(lim[bad], 1e-300))))
        nz = scale > 0
        worst = float(np.max(np.abs(diff[nz]) / scale[nz])) if np.any(nz) else 0.0
    return rel, worst

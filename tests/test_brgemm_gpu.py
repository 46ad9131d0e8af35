"""GPU parity of the batch-reduce GEMM (mic_brgemm) against the oracle.

C = alpha * sum_i A_i B_i + beta * C (single-building-block page, "Proposed
Method").  Small cases spanning several tiles with ragged edges run in full
for every kernel variant and every dtype, with operands laid out as plain
packed batches, transposed views, blocks cut out of one larger matrix and a
column-major or padded C; AlexNet's fully-connected layers run at full size
and are compared on sampled rows and columns; integer-valued inputs are
bit-exact and reruns bit-identical.

Tolerances are the convolution's (gpu_harness): fp32 relative L2 <= 1e-5 and
|err| <= 2e-6 * sum_i sum_k |A_i[m,k] B_i[k,n]| per element, fp64 relative
L2 <= 1e-12, bf16 (bf16 inputs, fp32 accumulation) relative L2 <= 1e-2.
The longest reduction here (fc6, 9216 terms) equals the forward pass's
longest, so the fp32 gate needs no length scaling.
"""
import ctypes

import numpy as np
import pytest
import torch

import convolution_forward_conv2d_amd as mic
import gen
import oracle
from gen import workloads

import gpu_harness as H

pytestmark = pytest.mark.gpu

BR_VARIANTS = {
    "f32": ["br_f32_128x128", "br_f32_64x64", "br_f32_32x64", "ws_f32_64x64", "ws_f32_32x64", "ws_f32_16x32"],
    "f64": ["br_f64_64x64", "br_f64_32x64", "ws_f64_32x64", "ws_f64_16x32"],
    "bf16": ["br_bf16_128x128", "br_bf16_64x64", "br_bf16_32x128", "ws_bf16_32x64", "ws_bf16_16x32"],
}
_ran = set()


def _vals(seed, shape, dtype, integer=False):
    v = gen.integers(seed, shape, -4, 4) if integer else gen.uniform(seed, shape, -1.0, 1.0)
    return gen.round_to(v, dtype)


def _place(vals, strides, dtype_key, fill=float("nan")):
    """A device view with the given element strides holding float64 vals (logical shape)."""
    n = 1 + sum((d - 1) * s for d, s in zip(vals.shape, strides)) if min(vals.shape) > 0 else 1
    base = torch.full((n,), fill, dtype=H.TORCH_DT[dtype_key], device=H.dev())
    t = base.as_strided(vals.shape, strides)
    if strides[0] == 0:                  # a shared block: write it once (the batch entries are equal)
        t[:1].copy_(torch.from_numpy(vals[:1]).to(H.TORCH_DT[dtype_key]))
    else:
        t.copy_(torch.from_numpy(vals).to(H.TORCH_DT[dtype_key]))
    return t


def _packed(shape):
    st, acc = [], 1
    for d in reversed(shape):
        st.append(acc)
        acc *= d
    return tuple(reversed(st))


def _operands(case, dtype, integer=False, seed=0):
    """Logical A (batch, m, k), B (batch, k, n) as float64 plus device views in the case's layout."""
    m, n, k, batch, lay = case["m"], case["n"], case["k"], case["batch"], case["layout"]
    a = _vals(seed + 11, (batch, m, k), dtype, integer)
    b = _vals(seed + 12, (batch, k, n), dtype, integer)
    if lay == "packed":                  # A (batch, m, k), B (batch, k, n) row-major
        sa, sb = _packed((batch, m, k)), _packed((batch, k, n))
    elif lay == "b_kmajor":              # B stored (batch, n, k): weights as rows of inputs
        sa, sb = _packed((batch, m, k)), (n * k, 1, k)
    elif lay == "a_transposed":          # A stored (batch, k, m)
        sa, sb = (k * m, 1, m), (n * k, 1, k)
    elif lay == "blocks":                # blocks of X (m, batch*k + 3) and W (n, batch*k + 5)
        sa, sb = (k, batch * k + 3, 1), (k, 1, batch * k + 5)
    elif lay == "blocks8":               # the same with row pitches padded by 8 (16-byte aligned rows)
        sa, sb = (k, batch * k + 8, 1), (k, 1, batch * k + 8)
    elif lay == "shared_b":              # every A_i multiplies the same B (batch stride 0)
        sa, sb = _packed((batch, m, k)), (0, n, 1)
        b = np.broadcast_to(b[:1], b.shape).copy()
    else:
        raise ValueError(lay)
    return a, b, _place(a, sa, dtype), _place(b, sb, dtype)


def _c_view(m, n, cl, dtype, fill=float("nan")):
    """C of shape (m, n): row-major, column-major or with a padded row pitch; returns (view, base)."""
    out_dt = H.OUT_DT[dtype]
    if cl == "row":
        st, size = (n, 1), m * n
    elif cl == "col":
        st, size = (1, m), m * n
    else:                                # "pitch": rows of n + 7
        st, size = (n + 7, 1), max(m * (n + 7), 1)
    base = torch.full((max(size, 1),), fill, dtype=out_dt, device=H.dev())
    return base.as_strided((m, n), st), base


SMALL = [
    dict(name="ragged_packed", m=70, n=100, k=37, batch=3, layout="packed", c="row"),
    dict(name="vec_bkmajor", m=96, n=160, k=64, batch=2, layout="b_kmajor", c="row"),
    dict(name="a_transposed", m=45, n=131, k=40, batch=2, layout="a_transposed", c="col"),
    dict(name="blocks_of_matrix", m=130, n=67, k=32, batch=5, layout="blocks", c="pitch"),
    dict(name="shared_b", m=33, n=65, k=17, batch=4, layout="shared_b", c="row"),
    dict(name="tall_vec", m=260, n=64, k=128, batch=1, layout="b_kmajor", c="col"),
    dict(name="one_element", m=1, n=1, k=1, batch=1, layout="packed", c="row"),
    dict(name="ragged_kmajor", m=50, n=70, k=96, batch=3, layout="b_kmajor", c="pitch"),
    dict(name="blocks8", m=45, n=100, k=32, batch=5, layout="blocks8", c="col"),
    dict(name="short_k_many_blocks", m=20, n=36, k=8, batch=37, layout="b_kmajor", c="row"),
]


def _supported(var, a, b, c):
    """Whether a forced variant can read these operands (the wave-split ones need k-contiguous runs)."""
    try:
        mic.brgemm_kernel_name_for(a, b, c)
        return True
    except mic.MicError as e:
        assert e.status == mic.MIC_STATUS_NOT_SUPPORTED and var.startswith("ws_"), (var, e)
        return False


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: c["name"])
def test_small_full_parity_every_variant(dtype, case, monkeypatch):
    a64, b64, a, b = _operands(case, dtype, seed=100 * SMALL.index(case))
    ref, bound = oracle.brgemm(a64, b64)
    for var in BR_VARIANTS[dtype]:
        monkeypatch.setenv("MIC_FORCE_BRGEMM_VARIANT", var)
        print("case", case["name"], dtype, var, flush=True)
        c, base = _c_view(case["m"], case["n"], case["c"], dtype)
        if not _supported(var, a, b, c):
            continue
        mic.brgemm(a, b, c)
        torch.cuda.synchronize()
        H.check(dtype, c.double().cpu().numpy(), ref, bound, what="%s/%s/%s" % (case["name"], dtype, var))
        if case["c"] == "pitch":         # the row padding stays untouched
            pad = base.view(case["m"], case["n"] + 7)[:, case["n"]:]
            assert bool(torch.isnan(pad).all()), "write outside C"
        # the same tiles in reverse order give the same bits
        monkeypatch.setenv("MIC_TILE_ORDER", "reverse")
        c_rev, _ = _c_view(case["m"], case["n"], case["c"], dtype)
        mic.brgemm(a, b, c_rev)
        torch.cuda.synchronize()
        monkeypatch.delenv("MIC_TILE_ORDER")
        assert torch.equal(c, c_rev), "%s/%s/%s: reversed tile order changed the result" % (
            case["name"], dtype, var)
        _ran.add(var)


def test_every_brgemm_variant_was_exercised():
    want = {v for vs in BR_VARIANTS.values() for v in vs}
    assert want <= _ran, "batch-reduce GEMM variants never run: %s" % sorted(want - _ran)


@pytest.mark.parametrize("dtype", ["f32", "f64", "bf16"])
def test_alpha_beta_integer_exact(dtype, monkeypatch):
    case = dict(m=77, n=90, k=64, batch=3, layout="blocks8")
    a64, b64, a, b = _operands(case, dtype, integer=True, seed=7)
    acc, _ = oracle.brgemm(a64, b64)
    old = gen.integers(98, acc.shape, -4, 4)
    want, _ = oracle.brgemm(a64, b64, alpha=0.5, beta=-0.25, c_old=old)
    assert np.array_equal(want, 0.5 * acc - 0.25 * old)
    for var in BR_VARIANTS[dtype]:
        monkeypatch.setenv("MIC_FORCE_BRGEMM_VARIANT", var)
        c = torch.from_numpy(old).to(H.OUT_DT[dtype]).to(H.dev())
        assert _supported(var, a, b, c), var
        mic.brgemm(a, b, c, alpha=0.5, beta=-0.25)
        torch.cuda.synchronize()
        assert np.array_equal(c.double().cpu().numpy(), want), var


def fc_operands(lay, integer=False):
    """Seeded activations X (m, F) and weights W (n, F), F = batch*k, rounded to the layer's type."""
    F = lay.features
    xd = ("integers", -4, 4) if integer else lay.x_dist
    wd = ("integers", -4, 4) if integer else lay.w_dist
    x = gen.round_to(gen.draw(xd, gen.derive_seed(lay.config, lay.layer, 0), (lay.m, F)), lay.dtype)
    w = gen.round_to(gen.draw(wd, gen.derive_seed(lay.config, lay.layer, 1), (lay.n, F)), lay.dtype)
    return x, w


def fc_views(lay, xt, wt):
    """A_i = X[:, i*k:(i+1)*k], B_i = W[:, i*k:(i+1)*k]^T as strided device views."""
    F = lay.features
    a = xt.as_strided((lay.batch, lay.m, lay.k), (lay.k, F, 1))
    b = wt.as_strided((lay.batch, lay.k, lay.n), (lay.k, 1, F))
    return a, b


def _fc_run(lay, x, w):
    xt = torch.from_numpy(x).to(H.TORCH_DT[lay.dtype]).to(H.dev())
    wt = torch.from_numpy(w).to(H.TORCH_DT[lay.dtype]).to(H.dev())
    a, b = fc_views(lay, xt, wt)
    c = torch.full((lay.m, lay.n), float("nan"), dtype=H.OUT_DT[lay.dtype], device=H.dev())
    mic.brgemm(a, b, c)
    torch.cuda.synchronize()
    return a, b, c


def _fc_sample(lay, rng, count=48):
    rows = np.unique(np.concatenate([[0, lay.m - 1], rng.integers(0, lay.m, count)]))
    cols = np.unique(np.concatenate([[0, lay.n // 2, lay.n - 1], rng.integers(0, lay.n, count)]))
    return rows, cols


def _fc_ref(lay, x, w, rows, cols):
    a = x[rows].reshape(len(rows), lay.batch, lay.k).transpose(1, 0, 2)
    b = w[cols].reshape(len(cols), lay.batch, lay.k).transpose(1, 2, 0)
    return oracle.brgemm(np.ascontiguousarray(a), np.ascontiguousarray(b))


@pytest.mark.parametrize("lay", workloads.FC, ids=lambda l: l.name)
def test_fc_layer_sampled(lay):
    """Full-size layer, default variant: sampled parity, NaN-safe beta=0, rerun bit-identity."""
    x, w = fc_operands(lay)
    a, b, c = _fc_run(lay, x, w)
    print("layer", lay.name, mic.brgemm_kernel_name_for(a, b, c), flush=True)
    assert bool(torch.isfinite(c).all()), "unwritten or non-finite C"
    rows, cols = _fc_sample(lay, np.random.default_rng(lay.layer + 61))
    ref, bound = _fc_ref(lay, x, w, rows, cols)
    got = c.double().cpu().numpy()[np.ix_(rows, cols)]
    rel, worst = H.check(lay.dtype, got, ref, bound, what=lay.name)
    print("  sampled rel-L2 %.3e, worst |err|/B %.3e" % (rel, worst), flush=True)
    c2 = torch.zeros_like(c)
    mic.brgemm(a, b, c2)
    torch.cuda.synchronize()
    assert torch.equal(c, c2), "rerun not bit-identical"


@pytest.mark.parametrize("lay", [l for l in workloads.FC if l.dtype != "f64"], ids=lambda l: l.name)
def test_fc_layer_integer_exact(lay):
    """Integer X, W in [-4, 4]: |partial sums| <= 16 * 9216 < 2^24, all exact in fp32."""
    assert 16 * lay.features < 2 ** 24
    x, w = fc_operands(lay, integer=True)
    _, _, c = _fc_run(lay, x, w)
    rows, cols = _fc_sample(lay, np.random.default_rng(lay.layer + 67))
    ref, _ = _fc_ref(lay, x, w, rows, cols)
    got = c.double().cpu().numpy()[np.ix_(rows, cols)]
    assert np.array_equal(got, ref), "%s: %d mismatches" % (lay.name, int((got != ref).sum()))


def test_degenerate_sizes():
    """k == 0 or batch == 0 scales C by beta; m == 0 or n == 0 touches nothing."""
    c = torch.full((5, 6), 3.0, device=H.dev())
    a = torch.zeros((2, 5, 0), device=H.dev())
    b = torch.zeros((2, 0, 6), device=H.dev())
    mic.brgemm(a, b, c, alpha=2.0, beta=0.5)
    torch.cuda.synchronize()
    assert bool((c == 1.5).all())
    a = torch.zeros((0, 5, 4), device=H.dev())
    b = torch.zeros((0, 4, 6), device=H.dev())
    mic.brgemm(a, b, c, beta=0.0)
    torch.cuda.synchronize()
    assert bool((c == 0.0).all())
    c = torch.full((0, 6), 1.0, device=H.dev())
    mic.brgemm(torch.zeros((1, 0, 3), device=H.dev()), torch.zeros((1, 3, 6), device=H.dev()), c)
    torch.cuda.synchronize()


def test_brgemm_error_statuses_on_device():
    a = torch.zeros((1, 8, 8), device=H.dev())
    b = torch.zeros((1, 8, 8), device=H.dev())
    c = torch.zeros((8, 8), device=H.dev())
    h = mic.handle_for(H.dev())
    with pytest.raises(mic.MicError) as e:            # misaligned A
        mic.mic_brgemm(h, mic.MIC_DTYPE_F32, 8, 8, 7, 1, 1.0, a.data_ptr() + 2, 64, 8, 1, b.data_ptr(), 64, 8, 1,
                       0.0, c.data_ptr(), 8, 1)
    assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    with pytest.raises(mic.MicError) as e:            # null C
        mic.mic_brgemm(h, mic.MIC_DTYPE_F32, 8, 8, 8, 1, 1.0, a.data_ptr(), 64, 8, 1, b.data_ptr(), 64, 8, 1,
                       0.0, 0, 8, 1)
    assert e.value.status == mic.MIC_STATUS_BAD_PARAM
    with pytest.raises(ValueError):
        mic.brgemm(a, torch.zeros((1, 7, 8), device=H.dev()), c)

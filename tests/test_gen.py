"""The seeded generator: determinism, index-addressing, distributions, rounding."""
import numpy as np
import torch

import gen
from gen import workloads


def test_splitmix_finaliser_known_values():
    # SplitMix64 with state 0: outputs are finaliser(gamma), finaliser(2*gamma), ...
    # (the generator's published first outputs for seed 0).
    z = gen._finalise(np.array([0x9E3779B97F4A7C15, 0x3C6EF372FE94F82A], dtype=np.uint64))
    assert int(z[0]) == 0xE220A8397B1DCDAF
    assert int(z[1]) == 0x6E789E6AA1B965F4


def test_counter_addressing_and_determinism():
    a = gen.uniform(123, (1000,))
    b = gen.uniform(123, (1000,))
    assert np.array_equal(a, b)
    c = gen.uniform(124, (1000,))
    assert not np.array_equal(a, c)
    # a slice drawn on its own equals the same slice of the whole
    z_all = gen.raw_u64(7, 0, 500)
    z_mid = gen.raw_u64(7, 200, 100)
    assert np.array_equal(z_all[200:300], z_mid)
    # chunked fill (tensors larger than the chunk) agrees with direct draws
    big = gen.uniform(9, (gen._CHUNK + 17,))
    tail = gen._unit(gen.raw_u64(9, gen._CHUNK, 17)) * 2.0 - 1.0
    assert np.array_equal(big[-17:], tail)


def test_distributions_roughly_right():
    n = 200_000
    u = gen.uniform(1, (n,), -1.0, 1.0)
    assert u.min() >= -1.0 and u.max() < 1.0
    assert abs(u.mean()) < 0.01 and abs(u.var() - 1.0 / 3.0) < 0.01
    g = gen.normal(2, (n,), 0.0, 0.01)
    assert abs(g.mean()) < 1e-4 and abs(g.std() - 0.01) < 2e-4
    he = gen.draw(("he_normal", 2304), 3, (n,))
    assert abs(he.std() - np.sqrt(2.0 / 2304)) < 1e-3
    ln = gen.lognormal(4, (n,))
    assert ln.min() > 0 and abs(np.log(ln).mean()) < 0.01 and abs(np.log(ln).std() - 1) < 0.01
    it = gen.integers(5, (n,), -4, 4)
    assert set(np.unique(it)) == set(range(-4, 5))


def test_round_to_f32_and_bf16():
    x = gen.normal(6, (10000,), 0.0, 3.0)
    f = gen.round_to(x, "f32")
    assert np.array_equal(f, x.astype(np.float32).astype(np.float64))
    b = gen.round_to(x, "bf16")
    # every value is exactly a bf16 value: round trip through torch is exact
    t = torch.from_numpy(b.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(t, b.astype(np.float32))
    # nearest: error at most half a bf16 ulp (2**-8 relative to the leading bit)
    m, e = np.frexp(x)
    assert np.all(np.abs(b - x) <= np.ldexp(1.0, e - 9) * (1 + 1e-12))
    # ties go to even
    one = 1.0
    assert gen.round_to(np.array([one + 2.0 ** -8]), "bf16")[0] == 1.0
    assert gen.round_to(np.array([one + 3 * 2.0 ** -8]), "bf16")[0] == one + 2.0 ** -6
    # agrees with torch's fp32 -> bf16 (RNE) for values that are fp32 already
    assert np.array_equal(gen.round_to(f, "bf16").astype(np.float32),
                          torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16).float().numpy())


def test_seeds_distinct_per_tensor():
    seeds = {gen.derive_seed(l.config, l.layer, t) for l in workloads.ALL_LAYERS for t in range(3)}
    # precision variants reuse their source layer's seeds (same logical values)
    assert len(seeds) == 3 * len({(l.config, l.layer) for l in workloads.ALL_LAYERS})


def test_padded_strides():
    assert workloads.padded_strides(64, 256, 13, 13, "nchw", 16) == (256 * 13 * 16, 13 * 16, 16, 1)
    assert workloads.padded_strides(64, 256, 13, 13, "nhwc", 16) == (13 * 16 * 256, 1, 16 * 256, 256)
    assert workloads.padded_strides(2, 3, 4, 5, "nchw", 0) == (60, 20, 5, 1)
    assert workloads.storage_elems(2, 3, 4, 5, (60, 20, 5, 1)) == 120

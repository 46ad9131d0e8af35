"""Seeded synthetic inputs for the 2-D convolution workloads.

This module serves both the CPU oracle and the GPU path (tests, benchmark,
smoke check).  It holds none of the convolution's arithmetic: it only draws
numbers.

Counter-based generator: the value at logical index i of a tensor is a pure
function of (seed, i), so a tensor generated in one piece, in slices, in
NCHW or in NHWC order, holds the same logical values.  The mixing function is
SplitMix64's finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), applied to ``key + (counter + 1) * gamma``
with gamma = 0x9E3779B97F4A7C15 and key = finaliser(seed).

Draws:
  * uniform(0,1): top 53 bits of a 64-bit draw times 2**-53;
  * normal: Box-Muller, cosine branch, two independent draws per value
    (streams 0 and 1 of the same counter);
  * log-normal: exp of a normal;
  * integers in [lo, hi]: a 64-bit draw reduced modulo (hi - lo + 1).

Values come out as float64 already rounded to the requested storage type
("f64", "f32" or "bf16", round-to-nearest-even), so the oracle (which reads
float64) and the GPU (which reads the storage type) see the same numbers.
"""
import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _finalise(z):
    """SplitMix64 finaliser on a uint64 ndarray (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed):
    return _finalise(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]


def raw_u64(seed, start, count, stream=0):
    """64-bit draws for logical indices start .. start+count-1 of one stream."""
    key = _key(seed)
    i = np.arange(start, start + count, dtype=np.uint64)
    ctr = i * np.uint64(2) + np.uint64(stream) + np.uint64(1)
    return _finalise(key + ctr * _GAMMA)


def _unit(z):
    """uniform [0, 1) from the top 53 bits."""
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def _fill(shape, fn):
    count = int(np.prod(shape, dtype=np.int64))
    out = np.empty(count, dtype=np.float64)
    for s in range(0, count, _CHUNK):
        e = min(count, s + _CHUNK)
        out[s:e] = fn(s, e - s)
    return out.reshape(shape)


def uniform(seed, shape, lo=-1.0, hi=1.0):
    return _fill(shape, lambda s, n: lo + (hi - lo) * _unit(raw_u64(seed, s, n, 0)))


def normal(seed, shape, mean=0.0, std=1.0):
    def fn(s, n):
        u1 = 1.0 - _unit(raw_u64(seed, s, n, 0))      # (0, 1]: log is finite
        u2 = _unit(raw_u64(seed, s, n, 1))
        return mean + std * np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return _fill(shape, fn)


def lognormal(seed, shape, mu=0.0, sigma=1.0):
    return np.exp(normal(seed, shape, mu, sigma))


def integers(seed, shape, lo=-4, hi=4):
    span = np.uint64(hi - lo + 1)
    return _fill(shape, lambda s, n: (raw_u64(seed, s, n, 0) % span).astype(np.float64) + lo)


def round_to(values, storage):
    """Round float64 values to the set a storage type holds (RNE), keep float64.

    "bf16" rounds straight from float64 to 8 significant bits (no detour
    through float32, so no double rounding).  Values are assumed finite and
    inside the normal range of the target type.
    """
    v = np.asarray(values, dtype=np.float64)
    if storage == "f64":
        return v.copy()
    if storage == "f32":
        return v.astype(np.float32).astype(np.float64)
    if storage == "bf16":
        m, e = np.frexp(v)                      # v = m * 2**e, 0.5 <= |m| < 1
        return np.ldexp(np.rint(m * 256.0) / 256.0, e)
    raise ValueError("unknown storage type %r" % (storage,))


def derive_seed(config, layer, tensor_id):
    """Seed of one tensor of one layer: tensor_id 0 = x, 1 = w, 2 = y_old."""
    base = 0x5EED0000 + 256 * int(config) + 16 * int(layer) + int(tensor_id)
    return int(_finalise(np.array([base], dtype=np.uint64))[0])


def draw(dist, seed, shape):
    """dist is a tuple: ("uniform", lo, hi) | ("normal", mean, std) |
    ("he_normal", fan_in) | ("lognormal", mu, sigma) | ("integers", lo, hi) |
    ("ones",)."""
    kind = dist[0]
    if kind == "uniform":
        return uniform(seed, shape, dist[1], dist[2])
    if kind == "normal":
        return normal(seed, shape, dist[1], dist[2])
    if kind == "he_normal":
        return normal(seed, shape, 0.0, float(np.sqrt(2.0 / dist[1])))
    if kind == "lognormal":
        return lognormal(seed, shape, dist[1], dist[2])
    if kind == "integers":
        return integers(seed, shape, dist[1], dist[2])
    if kind == "ones":
        return np.ones(shape, dtype=np.float64)
    raise ValueError("unknown distribution %r" % (kind,))

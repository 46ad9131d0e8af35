"""The convolution workloads, as plain data (shapes, strides, distributions).

Layer shapes follow the networks the pages measure on: AlexNet v.2 and
Overfeat (maxDNN page, "Key Findings"), and non-square speech inputs with
asymmetric padding (cuDNN page, "Proposed Method" and "Key Findings").
Datasets and trained weights are not used: every tensor is drawn by ``gen``
from a seed, with the value distribution stated per workload.

No convolution arithmetic here (output sizes and FLOP counts come from the
library or the oracle).
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Layer:
    name: str
    config: int                  # workload number 1..5
    layer: int                   # layer number inside the workload
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    stride: Tuple[int, int]      # (u along H, v along W)
    padding: Tuple[int, int, int, int]   # (top, bottom, left, right)
    dtype: str                   # "f32" | "f64" | "bf16" (bf16 in, fp32 out)
    x_dist: tuple
    w_dist: tuple
    layout: str = "nchw"         # "nchw" | "nhwc"
    row_pitch: int = 0           # 0: packed; else padded row pitch (elements of W)
    tags: Tuple[str, ...] = field(default_factory=tuple)

    @property
    def x_shape(self):
        return (self.N, self.C, self.H, self.W)

    @property
    def w_shape(self):
        return (self.K, self.C, self.R, self.S)


U11 = ("uniform", -1.0, 1.0)


def _he(C, R, S):
    return ("he_normal", C * R * S)


TINY = [Layer("tiny", 1, 1, 2, 8, 12, 12, 16, 3, 3, (1, 1), (1, 1, 1, 1), "f32", U11, U11)]

ALEXNET = [
    Layer("alexnet_conv2", 2, 2, 128, 96, 27, 27, 256, 5, 5, (1, 1), (2, 2, 2, 2), "f32",
          U11, _he(96, 5, 5)),
    Layer("alexnet_conv3", 2, 3, 128, 256, 13, 13, 384, 3, 3, (1, 1), (1, 1, 1, 1), "f32",
          U11, _he(256, 3, 3), tags=("target70",)),
    Layer("alexnet_conv4", 2, 4, 128, 384, 13, 13, 384, 3, 3, (1, 1), (1, 1, 1, 1), "f32",
          U11, _he(384, 3, 3), tags=("target70",)),
    Layer("alexnet_conv5", 2, 5, 128, 384, 13, 13, 256, 3, 3, (1, 1), (1, 1, 1, 1), "f32",
          U11, _he(384, 3, 3), tags=("target70",)),
]

N001 = ("normal", 0.0, 0.01)
OVERFEAT = [
    Layer("overfeat_l1", 3, 1, 128, 3, 231, 231, 96, 11, 11, (4, 4), (0, 0, 0, 0), "f32",
          U11, N001),
    Layer("overfeat_l2", 3, 2, 128, 96, 24, 24, 256, 5, 5, (1, 1), (0, 0, 0, 0), "f32",
          U11, N001),
    Layer("overfeat_l3", 3, 3, 128, 256, 12, 12, 512, 3, 3, (1, 1), (1, 1, 1, 1), "f32",
          U11, N001, tags=("target70",)),
    Layer("overfeat_l4", 3, 4, 128, 512, 12, 12, 1024, 3, 3, (1, 1), (1, 1, 1, 1), "f32",
          U11, N001, tags=("target70",)),
    Layer("overfeat_l5", 3, 5, 128, 1024, 12, 12, 1024, 3, 3, (1, 1), (1, 1, 1, 1), "f32",
          U11, N001, tags=("target70",)),
]

LOGN = ("lognormal", 0.0, 1.0)
N002 = ("normal", 0.0, 0.02)
SPEECH = [
    Layer("speech_l1", 4, 1, 32, 1, 161, 700, 32, 41, 11, (2, 2), (20, 20, 0, 10), "f32",
          LOGN, N002),
    # input of layer 2 = output size of layer 1 (81 x 350), drawn fresh
    Layer("speech_l2", 4, 2, 32, 32, 81, 350, 32, 21, 11, (2, 1), (10, 10, 0, 10), "f32",
          LOGN, N002),
]


def _precision():
    out = []
    for dt in ("f64", "bf16"):
        for lay in ("nchw", "nhwc"):
            for src in ALEXNET[1:]:
                out.append(Layer("%s_%s_%s" % (src.name.replace("alexnet_", "prec_"), dt, lay),
                                 5, src.layer, 64, src.C, src.H, src.W, src.K, src.R, src.S,
                                 src.stride, src.padding, dt, src.x_dist, src.w_dist,
                                 layout=lay, row_pitch=16))
    return out


PRECISION = _precision()

# Pooling between AlexNet's convolutions (3x3 windows, stride 2, no padding,
# max): after conv2 (27x27x256 -> 13x13, conv3's input size) and after
# conv5 (13x13x256 -> 6x6).  R, S are the window; K and w_dist are unused.
POOLING = [
    Layer("alexnet_pool2", 6, 2, 128, 256, 27, 27, 256, 3, 3, (2, 2), (0, 0, 0, 0), "f32", U11, U11,
          tags=("pool", "max")),
    Layer("alexnet_pool5", 6, 5, 128, 256, 13, 13, 256, 3, 3, (2, 2), (0, 0, 0, 0), "f32", U11, U11,
          tags=("pool", "max")),
]


@dataclass(frozen=True)
class FcLayer:
    """A fully-connected layer as a batch-reduce GEMM: y[m, n] = sum_i x_i[m, :] . W_i[:, n].

    The layer's input features are cut into ``batch`` blocks of ``k``; with
    batch 1 it is one plain product.  Activations x are (m, batch*k) row-major,
    weights W are (n, batch*k) row-major (one row of input weights per output).
    """
    name: str
    config: int
    layer: int
    m: int                       # minibatch rows
    n: int                       # output features
    k: int                       # input features per block
    batch: int                   # blocks reduced into one output
    dtype: str
    x_dist: tuple
    w_dist: tuple

    @property
    def features(self):
        return self.k * self.batch


# AlexNet's fully-connected layers at minibatch 128: fc6 reads conv5's pooled
# 256 x 6 x 6 = 9216 features, fc7 and fc8 4096; fc8's 1000 outputs leave a
# ragged tile edge.  fc6 also as 36 blocks of 256 features (one block per
# spatial position of the pooled map).
FC = [
    FcLayer("alexnet_fc6", 7, 6, 128, 4096, 9216, 1, "f32", U11, ("he_normal", 9216)),
    FcLayer("alexnet_fc7", 7, 7, 128, 4096, 4096, 1, "f32", U11, ("he_normal", 4096)),
    FcLayer("alexnet_fc8", 7, 8, 128, 1000, 4096, 1, "f32", U11, ("he_normal", 4096)),
    FcLayer("alexnet_fc6_blocked", 7, 16, 128, 4096, 256, 36, "f32", U11, ("he_normal", 9216)),
    FcLayer("alexnet_fc6_f64", 7, 26, 128, 4096, 9216, 1, "f64", U11, ("he_normal", 9216)),
    FcLayer("alexnet_fc6_bf16", 7, 36, 128, 4096, 9216, 1, "bf16", U11, ("he_normal", 9216)),
]


def fc_by_name(name):
    for lay in FC:
        if lay.name == name:
            return lay
    raise KeyError(name)


CONFIGS = {1: TINY, 2: ALEXNET, 3: OVERFEAT, 4: SPEECH, 5: PRECISION}
ALL_LAYERS = [l for c in sorted(CONFIGS) for l in CONFIGS[c]]


def pool_by_name(name):
    for lay in POOLING:
        if lay.name == name:
            return lay
    raise KeyError(name)


def by_name(name):
    for l in ALL_LAYERS:
        if l.name == name:
            return l
    raise KeyError(name)


def padded_strides(N, C, H, W, layout, row_pitch):
    """Element strides (sn, sc, sh, sw) of an N,C,H,W tensor.

    row_pitch = 0 gives packed storage.  Otherwise each image row (the W
    extent) is padded to row_pitch positions: NCHW rows hold row_pitch
    elements; NHWC rows hold row_pitch pixels of C channels.
    """
    Wp = row_pitch if row_pitch else W
    if Wp < W:
        raise ValueError("row pitch below W")
    if layout == "nchw":
        return (C * H * Wp, H * Wp, Wp, 1)
    if layout == "nhwc":
        return (H * Wp * C, 1, Wp * C, C)
    raise ValueError(layout)


def storage_elems(N, C, H, W, strides):
    """Elements an allocation needs to hold every index of a strided tensor."""
    sn, sc, sh, sw = strides
    return (N - 1) * sn + (C - 1) * sc + (H - 1) * sh + (W - 1) * sw + 1

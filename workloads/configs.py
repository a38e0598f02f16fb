"""The synthetic layer configurations the library is measured and tested on.

Shapes stand in for the CNN layers that the im2win paper (Table I) and the
openCNN article (ResNet Conv2-Conv5) benchmark on: no dataset is involved,
every tensor is drawn from a seeded generator (see ``gen.py``).

Distributions:
  * ``"normal"``   -> N(0, 1)
  * ``"uniform"``  -> U(-1, 1)
  * ``"he"``       -> N(0, 2 / (Cin * KH * KW))   (He initialisation of a filter)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    N: int
    Cin: int
    H: int
    W: int
    Cout: int
    KH: int
    KW: int
    stride: int
    pad: int
    dtypes: Tuple[str, ...]
    seed: int
    x_dist: str = "normal"
    w_dist: str = "he"
    note: str = ""

    @property
    def x_shape(self):
        return (self.N, self.Cin, self.H, self.W)

    @property
    def w_shape(self):
        return (self.Cout, self.Cin, self.KH, self.KW)

    def out_hw(self):
        ho = (self.H + 2 * self.pad - self.KH) // self.stride + 1
        wo = (self.W + 2 * self.pad - self.KW) // self.stride + 1
        return ho, wo

    def desc(self):
        return dict(N=self.N, Cin=self.Cin, H=self.H, W=self.W, Cout=self.Cout,
                    KH=self.KH, KW=self.KW, stride=self.stride, pad=self.pad)


def nominal_flops(N, Cin, H, W, Cout, KH, KW, stride, pad) -> int:
    """2 * multiply-adds of the layer, padded taps included (the usual TFLOPS convention)."""
    ho = (H + 2 * pad - KH) // stride + 1
    wo = (W + 2 * pad - KW) // stride + 1
    return 2 * N * Cout * ho * wo * Cin * KH * KW


CONFIGS: Dict[str, LayerConfig] = {c.name: c for c in [
    LayerConfig("tiny", 1, 3, 32, 32, 16, 3, 3, 1, 1, ("f32",), 1, "normal", "normal",
                "tiny conv, oracle finishes in well under a second"),
    LayerConfig("resnet3x3", 32, 64, 56, 56, 64, 3, 3, 1, 1, ("f32", "f16"), 2, "normal", "he",
                "ResNet-style 3x3 layer"),
    LayerConfig("deep3x3", 64, 256, 14, 14, 256, 3, 3, 1, 1, ("bf16",), 3, "normal", "he",
                "deep 3x3 layer, bf16 in, fp32 accumulate and output"),
    LayerConfig("stem7x7", 32, 3, 224, 224, 64, 7, 7, 2, 3, ("f32", "f16"), 4, "uniform", "he",
                "stem conv, 7x7 stride 2, output 112x112"),
    LayerConfig("mix5x5", 64, 128, 28, 28, 128, 5, 5, 1, 2, ("f16",), 51, "normal", "he",
                "mixed-kernel sweep: 5x5"),
    LayerConfig("mix512", 64, 512, 7, 7, 512, 3, 3, 1, 1, ("f16",), 52, "normal", "he",
                "mixed-kernel sweep: 512 channels at 7x7"),
    LayerConfig("mix3x3s2", 64, 256, 28, 28, 512, 3, 3, 2, 1, ("f16",), 53, "normal", "he",
                "mixed-kernel sweep: 3x3 stride 2"),
    LayerConfig("mix1x1", 64, 64, 56, 56, 256, 1, 1, 1, 0, ("f16",), 54, "normal", "he",
                "mixed-kernel sweep: 1x1"),
]}


# The twelve layers of Table I of "Enabling Memory-efficient Im2win Convolution
# with Multi-precision Support on GPU CUDA and Tensor Cores" (Sec. IV-B), at the
# batch the paper measures them with (N = 256) and with no padding, as printed.
# Each runs in fp32 (vector ALU) and fp16 (matrix cores); inputs N(0,1), filters
# He-initialised, one seed per layer.
_TABLE1_SHAPES = [
    # name, Cin, Hi, Wi, Cout, KH, KW, stride
    ("cv1", 3, 227, 227, 96, 11, 11, 4),
    ("cv2", 3, 231, 231, 96, 11, 11, 4),
    ("cv3", 3, 227, 227, 64, 7, 7, 2),
    ("cv4", 64, 224, 224, 64, 7, 7, 2),
    ("cv5", 96, 24, 24, 256, 5, 5, 1),
    ("cv6", 256, 12, 12, 512, 3, 3, 1),
    ("cv7", 3, 224, 224, 64, 3, 3, 1),
    ("cv8", 64, 112, 112, 128, 3, 3, 1),
    ("cv9", 64, 56, 56, 64, 3, 3, 1),
    ("cv10", 128, 28, 28, 128, 3, 3, 1),
    ("cv11", 256, 14, 14, 256, 3, 3, 1),
    ("cv12", 512, 7, 7, 512, 3, 3, 1),
]
TABLE1: Dict[str, LayerConfig] = {
    name: LayerConfig(name, 256, ci, h, w, co, kh, kw, s, 0, ("f16", "f32"), 100 + i,
                      "normal", "he", "Table I layer of the im2win paper, N=256, no padding")
    for i, (name, ci, h, w, co, kh, kw, s) in enumerate(_TABLE1_SHAPES, start=1)
}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name] if name in CONFIGS else TABLE1[name]

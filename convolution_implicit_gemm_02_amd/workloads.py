"""Seeded synthetic workloads: layer shape tables and input generators.

This module holds no arithmetic of the conv path.  It only draws the inputs
(activations, weights, batch-norm statistics) that both the GPU library and
the CPU oracle consume, and it fixes the INT8 calibration input s_x by the
workload's calibration rule (the 99.999th percentile of |x| divided by 127,
computed with numpy's percentile), the way an offline calibration pass fixes
it before deployment in the edge-optimization README ("Highlights":
percentile calibration; "Results": INT8 variants calibrated on separate
images).

Shapes follow the YOLO26n network that the vision-rs "YOLO26N Inference
Optimisation" page profiles (section "nsys kernel-level breakdown": stem
through FPN, 640x640 input, batch 1): five backbone stages at 320..20 pixels,
a neck and a detection head at three scales.  There are no datasets or
trained weights here, so every value is synthetic:
  x ~ N(0, 1) (the 3-channel 640x640 image ~ U(0, 1)),
  W ~ N(0, std = 1/sqrt(C_in*k*k)),
  gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1), running_mean ~ N(0, 0.1),
  running_var ~ U(0.5, 2), eps = 1e-3,
drawn from numpy.random.default_rng(seed), one generator per workload, per
layer in list order: x, W, gamma, beta, mean, var.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# eps = 1e-3, carried as the fp32 value the C ABI descriptor holds (both sides
# then fold with the same double: (double)(float)1e-3).
BN_EPS = float(np.float32(1e-3))
CALIB_PERCENTILE = 99.999


@dataclass(frozen=True)
class LayerSpec:
    name: str
    c_in: int
    c_out: int
    h: int  # input height
    w: int  # input width
    k: int
    stride: int
    pad: int
    dist: str = "normal"  # input distribution: "normal" N(0,1) or "uniform" U(0,1)

    @property
    def oh(self) -> int:
        return (self.h + 2 * self.pad - self.k) // self.stride + 1

    @property
    def ow(self) -> int:
        return (self.w + 2 * self.pad - self.k) // self.stride + 1

    def flops(self, n: int = 1) -> int:
        return 2 * n * self.oh * self.ow * self.c_out * self.c_in * self.k * self.k


def _c3(name, cin, cout, h, k, s, dist="normal"):
    return LayerSpec(name, cin, cout, h, h, k, s, k // 2, dist)


def single_layer():
    """One fused 3x3 s1 p1 conv, 32 -> 32 channels on 40x40."""
    return [_c3("single.3x3", 32, 32, 40, 3, 1)]


def ragged_sweep():
    """3x3 s1 p1 C->C and 1x1 2C->C at (C, H=W) = (64,80), (128,40), (256,20):
    output widths 80, 40 and 20 are the ones whose tail tiles overflowed on the
    vision-rs page (section "Bug fixed: TMA overflow")."""
    out = []
    for c, hw in ((64, 80), (128, 40), (256, 20)):
        out.append(_c3("ragged.3x3.c%d" % c, c, c, hw, 3, 1))
    for c, hw in ((64, 80), (128, 40), (256, 20)):
        out.append(_c3("ragged.1x1.c%d" % c, 2 * c, c, hw, 1, 1))
    return out


def stem_layers():
    """Large-spatial layers: 3x3 s2 3->16 on the 640x640 image, 3x3 s2 16->32 on
    320x320, 3x3 s1 16->16 on 160x160 (independent layers)."""
    return [_c3("stem.s2.3to16", 3, 16, 640, 3, 2, "uniform"),
            _c3("stem.s2.16to32", 16, 32, 320, 3, 2),
            _c3("stem.s1.16to16", 16, 16, 160, 3, 1)]


def yolo26n_layers():
    """The 37 conv layers of the YOLO26n-shaped list.

    Backbone, per stage c in {16,32,64,128,256} at output H=W in {320,...,20}:
    3x3 s2 downsample c/2 -> c (3 -> 16 for the first), 1x1 c -> c, two 3x3 s1
    c/2 -> c/2, 1x1 1.5c -> c.  Neck: 1x1 C -> C and 3x3 C -> C at
    (C,H) = (64,80), (128,40), (256,20).  Head: 3x3 C -> 64 and 1x1 64 -> 80
    at the same three scales.  Every layer reads its own generated input.
    """
    out = []
    for c, hw in ((16, 320), (32, 160), (64, 80), (128, 40), (256, 20)):
        cin_down = 3 if c == 16 else c // 2
        out.append(_c3("s%d.down" % c, cin_down, c, 2 * hw, 3, 2, "uniform" if c == 16 else "normal"))
        out.append(_c3("s%d.1x1" % c, c, c, hw, 1, 1))
        out.append(_c3("s%d.3x3a" % c, c // 2, c // 2, hw, 3, 1))
        out.append(_c3("s%d.3x3b" % c, c // 2, c // 2, hw, 3, 1))
        out.append(_c3("s%d.1x1cat" % c, c + c // 2, c, hw, 1, 1))
    for c, hw in ((64, 80), (128, 40), (256, 20)):
        out.append(_c3("neck%d.1x1" % c, c, c, hw, 1, 1))
        out.append(_c3("neck%d.3x3" % c, c, c, hw, 3, 1))
    for c, hw in ((64, 80), (128, 40), (256, 20)):
        out.append(_c3("head%d.3x3" % c, c, 64, hw, 3, 1))
        out.append(_c3("head%d.1x1" % c, 64, 80, hw, 1, 1))
    return out


WORKLOADS = {
    "single": single_layer,
    "ragged": ragged_sweep,
    "stem": stem_layers,
    "yolo26n": yolo26n_layers,
}


@dataclass
class LayerInputs:
    spec: LayerSpec
    n: int
    x: np.ndarray      # NCHW float32
    w: np.ndarray      # OIHW float32
    gamma: np.ndarray  # [C_out] float32
    beta: np.ndarray
    mean: np.ndarray
    var: np.ndarray
    eps: float = BN_EPS


def draw_layer(rng: np.random.Generator, spec: LayerSpec, n: int) -> LayerInputs:
    """Draw one layer's inputs, in the fixed order x, W, gamma, beta, mean, var."""
    shape = (n, spec.c_in, spec.h, spec.w)
    if spec.dist == "uniform":
        x = rng.random(shape, dtype=np.float32)
    else:
        x = rng.standard_normal(shape, dtype=np.float32)
    fan_in = spec.c_in * spec.k * spec.k
    w = (rng.standard_normal((spec.c_out, spec.c_in, spec.k, spec.k), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(fan_in))).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, spec.c_out).astype(np.float32)
    beta = (0.1 * rng.standard_normal(spec.c_out)).astype(np.float32)
    mean = (0.1 * rng.standard_normal(spec.c_out)).astype(np.float32)
    var = rng.uniform(0.5, 2.0, spec.c_out).astype(np.float32)
    return LayerInputs(spec, n, x, w, gamma, beta, mean, var)


def generate(workload: str, n: int = 1, seed: int = 0, specs=None):
    """All layers of a named workload (or the given specs) at batch n."""
    rng = np.random.default_rng(seed)
    specs = WORKLOADS[workload]() if specs is None else specs
    return [draw_layer(rng, s, n) for s in specs]


def calibration_scale(x: np.ndarray, percentile: float = CALIB_PERCENTILE) -> np.float32:
    """The workload's INT8 calibration input: s_x = fp32(P_q(|x|) / 127), with
    numpy's default ('linear') percentile over the whole tensor."""
    p = float(np.percentile(np.abs(np.asarray(x, dtype=np.float64)), percentile))
    return np.float32(p / 127.0)


def calibration_u8(x: np.ndarray):
    """The asymmetric uint8 calibration input (min/max, range widened to hold
    0): s = fp32((hi - lo) / 255) and z = clamp(rne(-lo / s), 0, 255), so that
    lo and hi map onto the ends of the code range and 0.0 onto the code z."""
    a = np.asarray(x, dtype=np.float64)
    lo, hi = min(float(a.min()), 0.0), max(float(a.max()), 0.0)
    if hi == lo:
        return np.float32(1.0), 0
    s = np.float32((hi - lo) / 255.0)
    return s, int(min(255, max(0, int(np.rint(-lo / float(s))))))


def random_case(rng: np.random.Generator, max_hw: int = 24, max_c: int = 40, n_max: int = 2):
    """A random small layer shape for property sweeps (k in {1,3}, s in {1,2})."""
    k = int(rng.choice([1, 3]))
    s = int(rng.choice([1, 2]))
    spec = LayerSpec("rand", int(rng.integers(1, max_c + 1)), int(rng.integers(1, max_c + 1)),
                     int(rng.integers(1, max_hw + 1)), int(rng.integers(1, max_hw + 1)), k, s, k // 2)
    return spec, int(rng.integers(1, n_max + 1))

"""CPU oracle for the fused Conv2d + BatchNorm + SiLU block (FP32 and INT8).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its binding.  It
shares no code with the GPU path.  The arithmetic lives in ``oracle.c`` (plain
C, double precision, nested loops over NCHW tensors); this module builds it
with gcc and marshals numpy arrays.

Sources (the pages the method comes from):
  * "YOLO26N Inference Optimisation" (vision-rs docs): section "nsys
    kernel-level breakdown" (the fused conv + BN + SiLU op), "Baseline
    benchmark" (BN folded at load), "NHWC migration" (the convolution as a
    contraction over C_in, kH, kW).
  * "Edge optimisation of YOLO26" (edge-optimization README): "Highlights" and
    "Design notes" (per-output-channel int8 weights, symmetric scales,
    percentile calibration of activations; INT8 end to end).
  * "YOLO26N Inference Optimisation", section "Improvements" #6 and #7 and
    "NHWC migration -- Op-by-op impact across the graph": bias-only convs,
    residual adds after the activation, channel cat / chunk (the layout side
    of these is plain numpy slicing in the tests; the oracle sees NCHW).

Every function is pinned by ``tests/test_oracle_pins.py`` against closed forms,
invariants, numpy library routines on special cases and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP, no FP contraction)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            D = ctypes.c_double
            L = ctypes.c_long
            F = ctypes.c_float
            lib.oracle_out_dim.argtypes = [I, I, I, I]
            lib.oracle_out_dim.restype = I
            lib.oracle_conv2d.argtypes = [P, P, I, I, I, I, I, I, I, I, P]
            lib.oracle_conv2d.restype = None
            lib.oracle_silu1.argtypes = [D]
            lib.oracle_silu1.restype = D
            lib.oracle_silu.argtypes = [P, P, L]
            lib.oracle_silu.restype = None
            lib.oracle_batchnorm.argtypes = [P, I, I, I, P, P, P, P, D]
            lib.oracle_batchnorm.restype = None
            lib.oracle_bn_fold.argtypes = [P, I, I, P, P, P, P, D, P, P]
            lib.oracle_bn_fold.restype = None
            lib.oracle_conv_bn_silu_f32.argtypes = [P, P, P, P, P, P, D, I, I, I, I, I, I, I, I, P, P]
            lib.oracle_conv_bn_silu_f32.restype = None
            lib.oracle_quantize_weights.argtypes = [P, I, I, P, P]
            lib.oracle_quantize_weights.restype = None
            lib.oracle_quantize_activations.argtypes = [P, L, F, P]
            lib.oracle_quantize_activations.restype = None
            lib.oracle_conv_i8_acc.argtypes = [P, P, I, I, I, I, I, I, I, I, P]
            lib.oracle_conv_i8_acc.restype = L
            lib.oracle_conv_i8_absacc.argtypes = [P, P, I, I, I, I, I, I, I, I, P]
            lib.oracle_conv_i8_absacc.restype = None
            lib.oracle_epilogue_i8.argtypes = [P, I, I, I, F, P, P, P, P]
            lib.oracle_epilogue_i8.restype = None
            lib.oracle_percentile_abs.argtypes = [P, L, D]
            lib.oracle_percentile_abs.restype = D
            lib.oracle_conv_bn_silu_i8.argtypes = [P, F, P, P, P, P, P, D, I, I, I, I, I, I, I, I,
                                                   P, P, P, P, P, P]
            lib.oracle_conv_bn_silu_i8.restype = L
            lib.oracle_conv_bn_silu_f32_points.argtypes = [P, P, P, P, P, P, D, I, I, I, I, I, I, I, I,
                                                           P, L, P, P]
            lib.oracle_conv_bn_silu_f32_points.restype = None
            lib.oracle_conv_bn_silu_i8_points.argtypes = [P, F, P, P, P, P, P, D, I, I, I, I, I, I, I, I,
                                                          P, L, P, P, P]
            lib.oracle_conv_bn_silu_i8_points.restype = L
            lib.oracle_conv_bn_act_f32.argtypes = [P, P, P, P, P, P, D, I, I, I, I, I, I, I, I, I, P, P, P]
            lib.oracle_conv_bn_act_f32.restype = None
            lib.oracle_conv_bn_act_f32_points.argtypes = [P, P, P, P, P, P, D, I, I, I, I, I, I, I, I, I, P,
                                                          P, L, P, P]
            lib.oracle_conv_bn_act_f32_points.restype = None
            lib.oracle_epilogue_i8_act.argtypes = [P, I, I, I, F, P, P, I, P, P, P]
            lib.oracle_epilogue_i8_act.restype = None
            lib.oracle_conv_bn_act_i8.argtypes = [P, F, P, P, P, P, P, D, I, I, I, I, I, I, I, I, I, P,
                                                  P, P, P, P, P, P]
            lib.oracle_conv_bn_act_i8.restype = L
            lib.oracle_conv_bn_act_i8_points.argtypes = [P, F, P, P, P, P, P, D, I, I, I, I, I, I, I, I, I,
                                                         P, P, L, P, P, P]
            lib.oracle_conv_bn_act_i8_points.restype = L
            lib.oracle_quantize_activations_u8.argtypes = [P, L, F, I, P]
            lib.oracle_quantize_activations_u8.restype = None
            lib.oracle_conv_u8_acc.argtypes = [P, I, P, I, I, I, I, I, I, I, I, P, P]
            lib.oracle_conv_u8_acc.restype = L
            lib.oracle_conv_bn_act_u8.argtypes = [P, F, I, P, P, P, P, P, D, I, I, I, I, I, I, I, I, I, P,
                                                  P, P, P, P, P, P]
            lib.oracle_conv_bn_act_u8.restype = L
            lib.oracle_set_threads.argtypes = [I]
            lib.oracle_set_threads.restype = None
            lib.oracle_get_threads.argtypes = []
            lib.oracle_get_threads.restype = I
            _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# Epilogue activations: "silu" (the block's SiLU) or "none" (identity: a plain
# conv + bias, as the head's final convs).
_ACT = {"silu": 0, "none": 1}


def _act(act: str) -> int:
    if act not in _ACT:
        raise ValueError("activation %r not in %s" % (act, sorted(_ACT)))
    return _ACT[act]


def _res(residual, shape):
    """Residual as a C-contiguous float64 array of the output's shape (or None)."""
    if residual is None:
        return None
    r = np.ascontiguousarray(residual, dtype=np.float64)
    if r.shape != tuple(shape):
        raise ValueError("residual shape %s != output shape %s" % (r.shape, tuple(shape)))
    return r


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def out_dim(size: int, k: int, s: int, p: int) -> int:
    """floor((size + 2p - k)/s) + 1."""
    return _load().oracle_out_dim(size, k, s, p)


def conv2d(x, w, stride: int, pad: int) -> np.ndarray:
    """Plain zero-padded 2-D cross-correlation, NCHW fp32 in, NCHW float64 out."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, c_in2, k, k2 = w.shape
    assert c_in2 == c_in and k2 == k
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    y = np.empty((n, c_out, oh, ow), np.float64)
    _load().oracle_conv2d(_p(x), _p(w), n, c_in, h, wd, c_out, k, stride, pad, _p(y))
    return y


def silu(z) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float64)
    y = np.empty_like(z)
    _load().oracle_silu(_p(z), _p(y), z.size)
    return y


def batchnorm(t, gamma, beta, mean, var, eps: float) -> np.ndarray:
    """Inference batch norm of an NCHW float64 tensor (returns a new array)."""
    t = np.array(t, dtype=np.float64, copy=True, order="C")
    n, c, h, w = t.shape
    _load().oracle_batchnorm(_p(t), n, c, h * w, _p(_f32(gamma)), _p(_f32(beta)), _p(_f32(mean)),
                             _p(_f32(var)), float(eps))
    return t


def bn_fold(w, gamma, beta, mean, var, eps: float):
    """Fold BN into the weights: returns (W' float64 OIHW, b' float64 [C_out])."""
    w = _f32(w)
    c_out = w.shape[0]
    per_co = int(np.prod(w.shape[1:]))
    wf = np.empty(w.shape, np.float64)
    bf = np.empty((c_out,), np.float64)
    _load().oracle_bn_fold(_p(w), c_out, per_co, _p(_f32(gamma)), _p(_f32(beta)), _p(_f32(mean)),
                           _p(_f32(var)), float(eps), _p(wf), _p(bf))
    return wf, bf


def conv_bn_silu_f32(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int,
                     with_bound: bool = True):
    """y = SiLU(BN(conv(x, W))) in double; also S = sum |W' * x| per output.

    Returns (y, S) as NCHW float64 arrays (S is None when with_bound is False).
    """
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    y = np.empty((n, c_out, oh, ow), np.float64)
    s = np.empty_like(y) if with_bound else None
    _load().oracle_conv_bn_silu_f32(_p(x), _p(w), _p(_f32(gamma)), _p(_f32(beta)), _p(_f32(mean)),
                                    _p(_f32(var)), float(eps), n, c_in, h, wd, c_out, k, stride, pad,
                                    _p(y), _p(s))
    return y, s


def conv_bn_act_f32(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, act: str = "silu",
                    residual=None, with_bound: bool = True):
    """y = act(BN(conv(x, W))) + residual in double (residual NCHW like y, or None);
    also S = sum |W' * x| per output.  Returns (y, S)."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    y = np.empty((n, c_out, oh, ow), np.float64)
    r = _res(residual, y.shape)
    s = np.empty_like(y) if with_bound else None
    _load().oracle_conv_bn_act_f32(_p(x), _p(w), _p(_f32(gamma)), _p(_f32(beta)), _p(_f32(mean)),
                                   _p(_f32(var)), float(eps), n, c_in, h, wd, c_out, k, stride, pad, _act(act),
                                   _p(r), _p(y), _p(s))
    return y, s


def quantize_weights(w_folded):
    """Per-output-channel symmetric int8: returns (q int8 same shape, s_w float64 [C_out])."""
    wf = np.ascontiguousarray(w_folded, dtype=np.float64)
    c_out = wf.shape[0]
    per_co = int(np.prod(wf.shape[1:]))
    q = np.empty(wf.shape, np.int8)
    sw = np.empty((c_out,), np.float64)
    _load().oracle_quantize_weights(_p(wf), c_out, per_co, _p(q), _p(sw))
    return q, sw


def quantize_activations(x, s_x: float) -> np.ndarray:
    x = _f32(x)
    q = np.empty(x.shape, np.int8)
    _load().oracle_quantize_activations(_p(x), x.size, float(np.float32(s_x)), _p(q))
    return q


def requantize(y, s_y: float) -> np.ndarray:
    """INT8 output codes of a layer: the activation quantiser applied to the
    fp32 value of y (float64 -> float32 rounds to nearest even), i.e. the codes
    the next INT8 layer would get from this layer's fp32 output."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    return quantize_activations(y32, s_y)


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (n <= 0: unchanged)."""
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def quantize_activations_u8(x, s_x: float, z: int) -> np.ndarray:
    """Asymmetric uint8: q = clamp(rne(fp32(x / s_x)) + z, 0, 255)."""
    x = _f32(x)
    q = np.empty(x.shape, np.uint8)
    _load().oracle_quantize_activations_u8(_p(x), x.size, float(np.float32(s_x)), int(z), _p(q))
    return q


def requantize_u8(y, s_y: float, z: int) -> np.ndarray:
    """Asymmetric uint8 output codes: the u8 quantiser applied to the fp32 value of y."""
    return quantize_activations_u8(np.asarray(y, dtype=np.float64).astype(np.float32), s_y, z)


def conv_u8_acc(qx, z: int, qw, stride: int, pad: int, with_abs: bool = False):
    """sum q_w (q - z) over the taps inside the image (int32); with_abs also returns sum |.| (int64)."""
    qx = np.ascontiguousarray(qx, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    n, c_in, h, wd = qx.shape
    c_out, _, k, _ = qw.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    acc = np.empty((n, c_out, oh, ow), np.int32)
    absacc = np.empty((n, c_out, oh, ow), np.int64) if with_abs else None
    ovf = _load().oracle_conv_u8_acc(_p(qx), int(z), _p(qw), n, c_in, h, wd, c_out, k, stride, pad, _p(acc),
                                     _p(absacc))
    if ovf:
        raise OverflowError("%d accumulators outside int32" % ovf)
    return (acc, absacc) if with_abs else acc


def conv_i8_acc(qx, qw, stride: int, pad: int) -> np.ndarray:
    """Exact integer convolution (int32 result; raises if any sum leaves int32)."""
    qx = np.ascontiguousarray(qx, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    n, c_in, h, wd = qx.shape
    c_out, _, k, _ = qw.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    acc = np.empty((n, c_out, oh, ow), np.int32)
    ovf = _load().oracle_conv_i8_acc(_p(qx), _p(qw), n, c_in, h, wd, c_out, k, stride, pad, _p(acc))
    if ovf:
        raise OverflowError("%d accumulators outside int32" % ovf)
    return acc


def conv_i8_absacc(qx, qw, stride: int, pad: int) -> np.ndarray:
    qx = np.ascontiguousarray(qx, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    n, c_in, h, wd = qx.shape
    c_out, _, k, _ = qw.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    out = np.empty((n, c_out, oh, ow), np.int64)
    _load().oracle_conv_i8_absacc(_p(qx), _p(qw), n, c_in, h, wd, c_out, k, stride, pad, _p(out))
    return out


def epilogue_i8(acc, s_x: float, s_w, b_folded):
    """y = SiLU(acc * fp32(s_x*s_w[co]) + b'[co]); returns (y float64, f float32 [C_out])."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    n, c_out, oh, ow = acc.shape
    y = np.empty(acc.shape, np.float64)
    f = np.empty((c_out,), np.float32)
    _load().oracle_epilogue_i8(_p(acc), n, c_out, oh * ow, float(np.float32(s_x)),
                               _p(np.ascontiguousarray(s_w, dtype=np.float64)),
                               _p(np.ascontiguousarray(b_folded, dtype=np.float64)), _p(y), _p(f))
    return y, f


def epilogue_i8_act(acc, s_x: float, s_w, b_folded, act: str = "silu", residual=None):
    """y = act(acc * fp32(s_x*s_w[co]) + b'[co]) + residual; returns (y float64, f float32 [C_out])."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    n, c_out, oh, ow = acc.shape
    y = np.empty(acc.shape, np.float64)
    r = _res(residual, y.shape)
    f = np.empty((c_out,), np.float32)
    _load().oracle_epilogue_i8_act(_p(acc), n, c_out, oh * ow, float(np.float32(s_x)),
                                   _p(np.ascontiguousarray(s_w, dtype=np.float64)),
                                   _p(np.ascontiguousarray(b_folded, dtype=np.float64)), _act(act), _p(r),
                                   _p(y), _p(f))
    return y, f


def percentile_abs(x, q: float) -> float:
    """q-th percentile of |x| ('linear' definition)."""
    x = _f32(x).ravel()
    return _load().oracle_percentile_abs(_p(x), x.size, float(q))


def conv_bn_silu_i8(x, s_x: float, w, gamma, beta, mean, var, eps: float, stride: int, pad: int,
                    with_bound: bool = True) -> dict:
    """The whole INT8 block.  Returns a dict with y (float64 NCHW), acc (int32 NCHW),
    qw (int8 OIHW), s_w (float64), f (float32 dequant factors) and absacc (int64 NCHW
    sum |q_w q_x|, or None)."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    y = np.empty((n, c_out, oh, ow), np.float64)
    acc = np.empty((n, c_out, oh, ow), np.int32)
    qw = np.empty(w.shape, np.int8)
    sw = np.empty((c_out,), np.float64)
    f = np.empty((c_out,), np.float32)
    absacc = np.empty((n, c_out, oh, ow), np.int64) if with_bound else None
    ovf = _load().oracle_conv_bn_silu_i8(_p(x), float(np.float32(s_x)), _p(w), _p(_f32(gamma)),
                                         _p(_f32(beta)), _p(_f32(mean)), _p(_f32(var)), float(eps),
                                         n, c_in, h, wd, c_out, k, stride, pad, _p(y), _p(acc), _p(qw),
                                         _p(sw), _p(f), _p(absacc))
    if ovf != 0:
        raise OverflowError("int8 oracle: %d accumulators outside int32 (or allocation failure)" % ovf)
    return {"y": y, "acc": acc, "qw": qw, "s_w": sw, "f": f, "absacc": absacc}


def conv_bn_act_i8(x, s_x: float, w, gamma, beta, mean, var, eps: float, stride: int, pad: int,
                   act: str = "silu", residual=None, with_bound: bool = True) -> dict:
    """The INT8 block with the epilogue options: y = act(acc * f + b') + residual
    (residual float64 NCHW like y, or None).  Same dict as conv_bn_silu_i8."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    y = np.empty((n, c_out, oh, ow), np.float64)
    r = _res(residual, y.shape)
    acc = np.empty((n, c_out, oh, ow), np.int32)
    qw = np.empty(w.shape, np.int8)
    sw = np.empty((c_out,), np.float64)
    f = np.empty((c_out,), np.float32)
    absacc = np.empty((n, c_out, oh, ow), np.int64) if with_bound else None
    ovf = _load().oracle_conv_bn_act_i8(_p(x), float(np.float32(s_x)), _p(w), _p(_f32(gamma)),
                                        _p(_f32(beta)), _p(_f32(mean)), _p(_f32(var)), float(eps),
                                        n, c_in, h, wd, c_out, k, stride, pad, _act(act), _p(r), _p(y), _p(acc),
                                        _p(qw), _p(sw), _p(f), _p(absacc))
    if ovf != 0:
        raise OverflowError("int8 oracle: %d accumulators outside int32 (or allocation failure)" % ovf)
    return {"y": y, "acc": acc, "qw": qw, "s_w": sw, "f": f, "absacc": absacc}


def conv_bn_act_u8(x, s_x: float, z_x: int, w, gamma, beta, mean, var, eps: float, stride: int, pad: int,
                   act: str = "silu", residual=None, with_bound: bool = True) -> dict:
    """The block with asymmetric uint8 activations (zero point z_x).  Same dict as
    conv_bn_act_i8 (absacc = sum |q_w (q - z_x)|)."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    oh, ow = out_dim(h, k, stride, pad), out_dim(wd, k, stride, pad)
    y = np.empty((n, c_out, oh, ow), np.float64)
    r = _res(residual, y.shape)
    acc = np.empty((n, c_out, oh, ow), np.int32)
    qw = np.empty(w.shape, np.int8)
    sw = np.empty((c_out,), np.float64)
    f = np.empty((c_out,), np.float32)
    absacc = np.empty((n, c_out, oh, ow), np.int64) if with_bound else None
    ovf = _load().oracle_conv_bn_act_u8(_p(x), float(np.float32(s_x)), int(z_x), _p(w), _p(_f32(gamma)),
                                        _p(_f32(beta)), _p(_f32(mean)), _p(_f32(var)), float(eps), n, c_in, h, wd,
                                        c_out, k, stride, pad, _act(act), _p(r), _p(y), _p(acc), _p(qw), _p(sw),
                                        _p(f), _p(absacc))
    if ovf != 0:
        raise OverflowError("u8 oracle: %d accumulators outside int32 (or allocation failure)" % ovf)
    return {"y": y, "acc": acc, "qw": qw, "s_w": sw, "f": f, "absacc": absacc}


def _points(pts):
    pts = np.ascontiguousarray(pts, dtype=np.int32).reshape(-1, 4)
    return pts, pts.shape[0]


def conv_bn_silu_f32_points(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, pts):
    """The FP32 block at the outputs pts[i] = (b, co, oh, ow) only: returns (y, S) float64 [npts]."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    pts, npts = _points(pts)
    y = np.empty((npts,), np.float64)
    s = np.empty((npts,), np.float64)
    _load().oracle_conv_bn_silu_f32_points(_p(x), _p(w), _p(_f32(gamma)), _p(_f32(beta)), _p(_f32(mean)),
                                           _p(_f32(var)), float(eps), n, c_in, h, wd, c_out, k, stride, pad,
                                           _p(pts), npts, _p(y), _p(s))
    return y, s


def conv_bn_silu_i8_points(x, s_x: float, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, pts):
    """The INT8 block at the outputs pts[i] = (b, co, oh, ow) only: returns (y float64, acc int32,
    absacc int64), each [npts]."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    pts, npts = _points(pts)
    y = np.empty((npts,), np.float64)
    acc = np.empty((npts,), np.int32)
    absacc = np.empty((npts,), np.int64)
    ovf = _load().oracle_conv_bn_silu_i8_points(_p(x), float(np.float32(s_x)), _p(w), _p(_f32(gamma)),
                                                _p(_f32(beta)), _p(_f32(mean)), _p(_f32(var)), float(eps),
                                                n, c_in, h, wd, c_out, k, stride, pad, _p(pts), npts,
                                                _p(y), _p(acc), _p(absacc))
    if ovf != 0:
        raise OverflowError("int8 oracle points: %d accumulators outside int32 (or allocation failure)" % ovf)
    return y, acc, absacc


def _res_pts(res_pts, npts):
    if res_pts is None:
        return None
    r = np.ascontiguousarray(res_pts, dtype=np.float64).ravel()
    if r.size != npts:
        raise ValueError("residual values %d != points %d" % (r.size, npts))
    return r


def conv_bn_act_f32_points(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, pts,
                           act: str = "silu", res_pts=None):
    """conv_bn_act_f32 at the outputs pts[i] = (b, co, oh, ow) only; res_pts[i] is the
    residual at output i (or None).  Returns (y, S) float64 [npts]."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    pts, npts = _points(pts)
    r = _res_pts(res_pts, npts)
    y = np.empty((npts,), np.float64)
    s = np.empty((npts,), np.float64)
    _load().oracle_conv_bn_act_f32_points(_p(x), _p(w), _p(_f32(gamma)), _p(_f32(beta)), _p(_f32(mean)),
                                          _p(_f32(var)), float(eps), n, c_in, h, wd, c_out, k, stride, pad,
                                          _act(act), _p(r), _p(pts), npts, _p(y), _p(s))
    return y, s


def conv_bn_act_i8_points(x, s_x: float, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, pts,
                          act: str = "silu", res_pts=None):
    """conv_bn_act_i8 at the outputs pts only: returns (y float64, acc int32, absacc int64), each [npts]."""
    x = _f32(x)
    w = _f32(w)
    n, c_in, h, wd = x.shape
    c_out, _, k, _ = w.shape
    pts, npts = _points(pts)
    r = _res_pts(res_pts, npts)
    y = np.empty((npts,), np.float64)
    acc = np.empty((npts,), np.int32)
    absacc = np.empty((npts,), np.int64)
    ovf = _load().oracle_conv_bn_act_i8_points(_p(x), float(np.float32(s_x)), _p(w), _p(_f32(gamma)),
                                               _p(_f32(beta)), _p(_f32(mean)), _p(_f32(var)), float(eps),
                                               n, c_in, h, wd, c_out, k, stride, pad, _act(act), _p(r), _p(pts),
                                               npts, _p(y), _p(acc), _p(absacc))
    if ovf != 0:
        raise OverflowError("int8 oracle points: %d accumulators outside int32 (or allocation failure)" % ovf)
    return y, acc, absacc

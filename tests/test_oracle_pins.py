"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each pin is a function of the implementation under test so that the
"mutant" tests at the bottom can show that a plausible mistake (a flipped
kernel, a dropped channel, an off-by-one pad, a sign error in the batch-norm
fold, a wrong rounding rule) fails at least one of them.  Mutants are built
from the oracle on the CPU; nothing here touches the GPU library.

Sources: the vision-rs page "YOLO26N Inference Optimisation" (sections "nsys
kernel-level breakdown", "NHWC migration", "Bug fixed: TMA overflow") and the
edge-optimization README ("Highlights", "Design notes").
"""
import math
import os

import numpy as np
import pytest

import oracle
from convolution_implicit_gemm_02_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


# ------------------------------------------------------------- helpers ----

def np_conv_im2col(x, w, stride, pad):
    """Independent vectorised conv: zero-pad with np.pad, gather patches by
    slicing, contract with one float64 matmul (the library routine)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    n, c, h, wd = x.shape
    co, _, k, _ = w.shape
    oh = (h + 2 * pad - k) // stride + 1
    ow = (wd + 2 * pad - k) // stride + 1
    xp = np.pad(x, ((0, 0), (0, 0), (pad, pad), (pad, pad)))
    cols = np.empty((n, c, k, k, oh, ow))
    for i in range(k):
        for j in range(k):
            cols[:, :, i, j] = xp[:, :, i:i + stride * oh:stride, j:j + stride * ow:stride]
    cols = cols.transpose(0, 4, 5, 1, 2, 3).reshape(n * oh * ow, c * k * k)
    y = cols @ w.reshape(co, -1).T
    return y.reshape(n, oh, ow, co).transpose(0, 3, 1, 2)


def np_im2col_int(qx, k, stride, pad):
    qx = np.asarray(qx, np.int64)
    n, c, h, wd = qx.shape
    oh = (h + 2 * pad - k) // stride + 1
    ow = (wd + 2 * pad - k) // stride + 1
    xp = np.pad(qx, ((0, 0), (0, 0), (pad, pad), (pad, pad)))
    cols = np.empty((n, c, k, k, oh, ow), np.int64)
    for i in range(k):
        for j in range(k):
            cols[:, :, i, j] = xp[:, :, i:i + stride * oh:stride, j:j + stride * ow:stride]
    return cols.transpose(0, 4, 5, 1, 2, 3).reshape(n * oh * ow, c * k * k), oh, ow


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------- the pins ----
# Each returns True when the implementation satisfies the pin.

def pin_delta_kernel(conv):
    """W[co,ci,1,1] = delta(co,ci), 3x3 s1 p1: the conv reproduces x exactly."""
    r = rng(1)
    x = r.standard_normal((2, 5, 7, 6)).astype(np.float32)
    w = np.zeros((5, 5, 3, 3), np.float32)
    for c in range(5):
        w[c, c, 1, 1] = 1.0
    y = conv(x, w, 1, 1)
    return y.shape == x.shape and np.array_equal(y, x.astype(np.float64))


def pin_1x1_matmul(conv):
    """k=1, s=1, p=0 is the matmul W[:,:,0,0] @ x.reshape(C_in, H*W) (numpy float64 BLAS)."""
    r = rng(2)
    x = r.standard_normal((2, 13, 5, 7)).astype(np.float32)
    w = r.standard_normal((9, 13, 1, 1)).astype(np.float32)
    y = conv(x, w, 1, 0)
    ref = np.einsum("oc,nchw->nohw", w[:, :, 0, 0].astype(np.float64), x.astype(np.float64))
    ref2 = np.stack([w[:, :, 0, 0].astype(np.float64) @ x[b].reshape(13, -1).astype(np.float64)
                     for b in range(2)]).reshape(2, 9, 5, 7)
    return y.shape == ref.shape and np.allclose(y, ref2, rtol=1e-12, atol=1e-12)


def pin_zero_padding_closed_form(conv):
    """x == c and W == 1 (3x3 s1 p1): conv = c * C_in * {4 corner, 6 edge, 9 interior}."""
    c_in, h, wd, cval = 3, 5, 6, 0.5
    x = np.full((1, c_in, h, wd), cval, np.float32)
    w = np.ones((2, c_in, 3, 3), np.float32)
    y = conv(x, w, 1, 1)
    exp = np.full((h, wd), 9.0)
    exp[0, :] = exp[-1, :] = 6.0
    exp[:, 0] = exp[:, -1] = 6.0
    exp[0, 0] = exp[0, -1] = exp[-1, 0] = exp[-1, -1] = 4.0
    exp = exp * cval * c_in
    return all(np.array_equal(y[0, co], exp) for co in range(2))


def _brute_2x2(x, w, k, s):
    """Hand-written outputs for a 2x2 input (C_in = C_out in {1,2})."""
    c = x.shape[1]
    a, b, cc, d = x[0, :, 0, 0], x[0, :, 0, 1], x[0, :, 1, 0], x[0, :, 1, 1]
    out = []
    for co in range(w.shape[0]):
        wk = w[co]
        if k == 3 and s == 1:
            o = np.array([
                [sum(wk[ci, 1, 1] * a[ci] + wk[ci, 1, 2] * b[ci] + wk[ci, 2, 1] * cc[ci] + wk[ci, 2, 2] * d[ci] for ci in range(c)),
                 sum(wk[ci, 1, 0] * a[ci] + wk[ci, 1, 1] * b[ci] + wk[ci, 2, 0] * cc[ci] + wk[ci, 2, 1] * d[ci] for ci in range(c))],
                [sum(wk[ci, 0, 1] * a[ci] + wk[ci, 0, 2] * b[ci] + wk[ci, 1, 1] * cc[ci] + wk[ci, 1, 2] * d[ci] for ci in range(c)),
                 sum(wk[ci, 0, 0] * a[ci] + wk[ci, 0, 1] * b[ci] + wk[ci, 1, 0] * cc[ci] + wk[ci, 1, 1] * d[ci] for ci in range(c))]])
        elif k == 3 and s == 2:
            o = np.array([[sum(wk[ci, 1, 1] * a[ci] + wk[ci, 1, 2] * b[ci] + wk[ci, 2, 1] * cc[ci] + wk[ci, 2, 2] * d[ci]
                               for ci in range(c))]])
        elif k == 1 and s == 1:
            o = np.array([[sum(wk[ci, 0, 0] * a[ci] for ci in range(c)), sum(wk[ci, 0, 0] * b[ci] for ci in range(c))],
                          [sum(wk[ci, 0, 0] * cc[ci] for ci in range(c)), sum(wk[ci, 0, 0] * d[ci] for ci in range(c))]])
        else:  # k == 1, s == 2
            o = np.array([[sum(wk[ci, 0, 0] * a[ci] for ci in range(c))]])
        out.append(o)
    return np.array(out, dtype=np.float64)[None]


def pin_brute_force_2x2(conv):
    """Every output of a 2x2 input by hand-written four-term formulas (integer data: exact)."""
    r = rng(3)
    for c in (1, 2):
        x = r.integers(-4, 5, (1, c, 2, 2)).astype(np.float32)
        for k, s in ((3, 1), (3, 2), (1, 1), (1, 2)):
            w = r.integers(-3, 4, (c, c, k, k)).astype(np.float32)
            y = conv(x, w, s, k // 2)
            exp = _brute_2x2(x.astype(np.float64), w.astype(np.float64), k, s)
            if y.shape != exp.shape or not np.array_equal(y, exp):
                return False
    return True


def pin_translation_equivariance(conv):
    """Stride 1: shifting x by (dy, dx) with zero fill shifts the outputs that
    do not see the bottom/right border, bit for bit."""
    r = rng(4)
    x = r.standard_normal((1, 4, 9, 8)).astype(np.float32)
    w = r.standard_normal((3, 4, 3, 3)).astype(np.float32)
    dy, dx = 2, 1
    xs = np.zeros_like(x)
    xs[:, :, dy:, dx:] = x[:, :, :-dy, :-dx]
    y = conv(x, w, 1, 1)
    ys = conv(xs, w, 1, 1)
    h, wd = x.shape[2:]
    a = y[:, :, 0:h - dy - 1, 0:wd - dx - 1]
    b = ys[:, :, dy:h - 1, dx:wd - 1]
    return np.array_equal(a, b)


def pin_stride2_subsample(conv):
    """k=3 p=1: the stride-2 output is the stride-1 output at even positions, bit for bit."""
    r = rng(5)
    for h, wd in ((9, 8), (10, 7)):
        x = r.standard_normal((2, 3, h, wd)).astype(np.float32)
        w = r.standard_normal((4, 3, 3, 3)).astype(np.float32)
        y1 = conv(x, w, 1, 1)
        y2 = conv(x, w, 2, 1)
        if not np.array_equal(y2, y1[:, :, ::2, ::2]):
            return False
    return True


def pin_random_vs_im2col(conv):
    """Random shapes (k in {1,3}, s in {1,2}) against the independent im2col + matmul."""
    r = rng(6)
    for _ in range(12):
        spec, n = W.random_case(r, max_hw=11, max_c=9)
        x = r.standard_normal((n, spec.c_in, spec.h, spec.w)).astype(np.float32)
        w = r.standard_normal((spec.c_out, spec.c_in, spec.k, spec.k)).astype(np.float32)
        y = conv(x, w, spec.stride, spec.pad)
        ref = np_conv_im2col(x, w, spec.stride, spec.pad)
        if y.shape != ref.shape or not np.allclose(y, ref, rtol=1e-12, atol=1e-12):
            return False
    return True


CONV_PINS = [pin_delta_kernel, pin_1x1_matmul, pin_zero_padding_closed_form, pin_brute_force_2x2,
             pin_translation_equivariance, pin_stride2_subsample, pin_random_vs_im2col]


@pytest.mark.parametrize("pin", CONV_PINS, ids=[p.__name__ for p in CONV_PINS])
def test_oracle_conv_pins(pin):
    assert pin(oracle.conv2d)


def test_out_dim_closed_form():
    for h in range(1, 30):
        for k, p in ((1, 0), (3, 1)):
            for s in (1, 2):
                assert oracle.out_dim(h, k, s, p) == (h + 2 * p - k) // s + 1
    # the page's shapes: 640 -> 320 (3x3 s2 p1), 40 -> 40 (3x3 s1 p1), 20 -> 10
    assert oracle.out_dim(640, 3, 2, 1) == 320
    assert oracle.out_dim(40, 3, 1, 1) == 40
    assert oracle.out_dim(20, 3, 2, 1) == 10


# --------------------------------------------------------------- SiLU ----

def test_silu_golden_and_identity():
    g = read_golden("silu_values.txt")
    got = oracle.silu(g[:, 0])
    assert np.allclose(got, g[:, 1], rtol=0, atol=1e-16)
    assert got[0] == 0.0
    z = np.linspace(-30, 30, 1201)
    # SiLU(z) - SiLU(-z) = z * (sigmoid(z) + sigmoid(-z)) = z
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-14, atol=1e-13)
    # large |z|: SiLU -> z and -> 0
    assert abs(oracle.silu(np.array([50.0]))[0] - 50.0) < 1e-12
    assert abs(oracle.silu(np.array([-50.0]))[0]) < 1e-18


# -------------------------------------------------------- batch norm ----

def _bn_params(r, c):
    return (r.uniform(0.5, 1.5, c).astype(np.float32), (0.1 * r.standard_normal(c)).astype(np.float32),
            (0.1 * r.standard_normal(c)).astype(np.float32), r.uniform(0.5, 2.0, c).astype(np.float32))


def pin_fold_equals_unfolded(bn_fold, batchnorm):
    """conv(W') + b' == BN(conv(W)) to 1e-12 (W' applied with numpy im2col + matmul)."""
    r = rng(7)
    x = r.standard_normal((2, 6, 7, 5)).astype(np.float32)
    w = r.standard_normal((4, 6, 3, 3)).astype(np.float32)
    g, b, m, v = _bn_params(r, 4)
    eps = W.BN_EPS
    wf, bf = bn_fold(w, g, b, m, v, eps)
    folded = np_conv_im2col(x, wf, 1, 1) + bf[None, :, None, None]
    unfolded = batchnorm(oracle.conv2d(x, w, 1, 1), g, b, m, v, eps)
    return np.allclose(folded, unfolded, rtol=1e-12, atol=1e-12)


def pin_bn_closed_form(batchnorm):
    """BN of a constant map: (t - mean)/sqrt(var + eps)*gamma + beta with gamma=2, beta=1,
    mean=0.5, var=3.999, eps=0.001 -> (t - 0.5)/2*2 + 1 = t + 0.5."""
    t = np.full((1, 1, 2, 2), 3.0)
    out = batchnorm(t, np.array([2.0]), np.array([1.0]), np.array([0.5]), np.array([3.999], np.float32),
                    float(np.float32(0.001)))
    expect = (3.0 - 0.5) / math.sqrt(float(np.float32(3.999)) + float(np.float32(0.001))) * 2.0 + 1.0
    return np.allclose(out, expect, rtol=1e-15) and abs(expect - 3.5) < 1e-6


def test_bn_pins():
    assert pin_fold_equals_unfolded(oracle.bn_fold, oracle.batchnorm)
    assert pin_bn_closed_form(oracle.batchnorm)


def test_fused_f32_is_composition_and_bound():
    r = rng(8)
    for spec, n in [W.random_case(r, 10, 8) for _ in range(6)]:
        L = W.draw_layer(r, spec, n)
        y, s = oracle.conv_bn_silu_f32(L.x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, spec.stride, spec.pad)
        conv = oracle.conv2d(L.x, L.w, spec.stride, spec.pad)
        ref = oracle.silu(oracle.batchnorm(conv, L.gamma, L.beta, L.mean, L.var, L.eps))
        assert np.array_equal(y, ref)
        # S = sum |W' x| = |x| im2col @ |W'| since |w x| = |w| |x|
        wf, _ = oracle.bn_fold(L.w, L.gamma, L.beta, L.mean, L.var, L.eps)
        sref = np_conv_im2col(np.abs(L.x), np.abs(wf), spec.stride, spec.pad)
        assert np.allclose(s, sref, rtol=1e-12, atol=1e-12)
        # points evaluation agrees with the whole-tensor evaluation
        pts = np.array([[b, c, i, j] for b in range(n) for c in range(spec.c_out)
                        for i in range(spec.oh) for j in range(spec.ow)])[::3]
        yp, sp = oracle.conv_bn_silu_f32_points(L.x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps,
                                                spec.stride, spec.pad, pts)
        assert np.array_equal(yp, y[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]])
        assert np.array_equal(sp, s[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]])


# --------------------------------------------------------------- INT8 ----

def pin_quantize_weights(qw_fn):
    """Per-channel symmetric int8 (edge-optimization README, "Design notes"):
    the largest |w| maps to +-127, s_w = max/127, ties round to even, an
    all-zero channel gets s_w = 1 and q = 0."""
    s = 0.01
    wf = np.array([
        [127 * s, 2.5 * s, -2.5 * s, 3.5 * s, 0.0, -127 * s],   # max 1.27 -> s_w = 0.01
        [0, 0, 0, 0, 0, 0],                                    # zero channel
        [-4.0, 1.0, 0.5, -0.25, 2.0, 3.0],                     # max 4 -> s_w = 4/127
    ], np.float64)
    q, sw = qw_fn(wf)
    ok = sw[0] == (127 * s) / 127.0 and sw[1] == 1.0 and sw[2] == 4.0 / 127.0
    ok &= q[0, 0] == 127 and q[0, 5] == -127
    exp0 = [int(np.rint(v / sw[0])) for v in wf[0]]
    ok &= list(q[0]) == exp0
    ok &= list(q[1]) == [0] * 6
    ok &= q[2, 0] == -127
    exp2 = [int(np.clip(np.rint(v / sw[2]), -127, 127)) for v in wf[2]]
    ok &= list(q[2]) == exp2
    # random: |q| <= 127 and each channel reaches 127 in magnitude
    r = rng(9)
    wr = r.standard_normal((7, 50))
    q, sw = qw_fn(wr)
    ok &= np.abs(q.astype(int)).max() <= 127 and all(np.abs(q[c].astype(int)).max() == 127 for c in range(7))
    ok &= np.array_equal(sw, np.abs(wr).max(axis=1) / 127.0)
    ok &= np.array_equal(q, np.clip(np.rint(wr / sw[:, None]), -127, 127).astype(np.int8))
    return bool(ok)


def pin_quantize_activations(qa_fn):
    """q = clamp(rne(fp32(x / s_x)), +-127): fp32 division, ties to even, clamp."""
    s_x = np.float32(0.5)
    x = np.array([0.0, 0.25, 0.75, 1.25, -0.25, -0.75, 63.25, 63.75, 100.0, -100.0, 0.2, -0.2], np.float32)
    q = qa_fn(x, s_x)
    exp = np.array([0, 0, 2, 2, 0, -2, 126, 127, 127, -127, 0, 0], np.int8)
    ok = np.array_equal(q, exp)
    r = rng(10)
    xr = (3 * r.standard_normal(10000)).astype(np.float32)
    s = W.calibration_scale(xr)
    ref = np.clip(np.rint(xr / s), -127, 127).astype(np.int8)   # numpy: fp32 / fp32 -> fp32
    ok &= np.array_equal(qa_fn(xr, s), ref)
    return bool(ok)


def test_int8_quantiser_pins():
    assert pin_quantize_weights(oracle.quantize_weights)
    assert pin_quantize_activations(oracle.quantize_activations)


def test_int8_acc_exact_vs_integer_matmul():
    """The integer accumulators equal an int64 numpy matmul of the im2col'd integers."""
    r = rng(11)
    for spec, n in [W.random_case(r, 12, 20) for _ in range(10)]:
        qx = r.integers(-127, 128, (n, spec.c_in, spec.h, spec.w)).astype(np.int8)
        qw = r.integers(-127, 128, (spec.c_out, spec.c_in, spec.k, spec.k)).astype(np.int8)
        acc = oracle.conv_i8_acc(qx, qw, spec.stride, spec.pad)
        cols, oh, ow = np_im2col_int(qx, spec.k, spec.stride, spec.pad)
        ref = (cols @ qw.astype(np.int64).reshape(spec.c_out, -1).T).reshape(n, oh, ow, spec.c_out)
        assert np.array_equal(acc, ref.transpose(0, 3, 1, 2).astype(np.int32))
        absacc = oracle.conv_i8_absacc(qx, qw, spec.stride, spec.pad)
        aref = (np.abs(cols) @ np.abs(qw.astype(np.int64)).reshape(spec.c_out, -1).T)
        assert np.array_equal(absacc, aref.reshape(n, oh, ow, spec.c_out).transpose(0, 3, 1, 2))


def test_int8_extreme_accumulators_fit_int32():
    """|acc| <= 127^2 * C_in * 9: the largest layer (C_in = 256, 3x3) stays exact."""
    qx = np.full((1, 256, 3, 3), 127, np.int8)
    qw = np.full((2, 256, 3, 3), -127, np.int8)
    acc = oracle.conv_i8_acc(qx, qw, 1, 1)
    assert acc[0, 0, 1, 1] == -127 * 127 * 256 * 9
    assert acc[0, 0, 0, 0] == -127 * 127 * 256 * 4


def test_int8_epilogue_special_cases():
    """Dequant + bias + SiLU at points with known values: acc*f + b' = 0, 1, -1
    lands on the golden SiLU values; f = fp32(s_x * s_w) is exact for powers of two."""
    g = read_golden("silu_values.txt")
    s_x = np.float32(0.5)
    s_w = np.array([0.25, 2.0, 1.0], np.float64)           # f = 0.125, 1.0, 0.5 exactly
    b = np.array([0.0, -1.0, 1.5], np.float64)
    acc = np.array([0, 8, 2, 0, -3, -5], np.int32).reshape(1, 3, 1, 2)
    # z: co0: 0*0.125+0 = 0, 8*0.125+0 = 1 | co1: 2*1-1 = 1, 0-1 = -1 | co2: -3*0.5+1.5 = 0, -5*0.5+1.5 = -1
    y, f = oracle.epilogue_i8(acc, s_x, s_w, b)
    assert list(f) == [0.125, 1.0, 0.5]
    exp = {0.0: g[0, 1], 1.0: g[1, 1], -1.0: g[2, 1]}
    want = np.array([exp[0.0], exp[1.0], exp[1.0], exp[-1.0], exp[0.0], exp[-1.0]]).reshape(1, 3, 1, 2)
    assert np.allclose(y, want, rtol=0, atol=1e-16)


def test_int8_epilogue_and_composition():
    r = rng(12)
    spec = W.LayerSpec("t", 6, 5, 7, 6, 3, 1, 1)
    L = W.draw_layer(r, spec, 2)
    s_x = W.calibration_scale(L.x)
    res = oracle.conv_bn_silu_i8(L.x, s_x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, 1, 1)
    wf, bf = oracle.bn_fold(L.w, L.gamma, L.beta, L.mean, L.var, L.eps)
    qw, sw = oracle.quantize_weights(wf)
    qx = oracle.quantize_activations(L.x, s_x)
    acc = oracle.conv_i8_acc(qx, qw, 1, 1)
    assert np.array_equal(res["qw"], qw) and np.array_equal(res["s_w"], sw)
    assert np.array_equal(res["acc"], acc)
    f = (np.float64(s_x) * sw).astype(np.float32)
    assert np.array_equal(res["f"], f)
    z = acc.astype(np.float64) * f.astype(np.float64)[None, :, None, None] + bf[None, :, None, None]
    assert np.allclose(res["y"], z / (1 + np.exp(-z)), rtol=1e-15, atol=1e-15)
    # dequantised int8 output stays close to the fp32 block (quantisation error, not exact)
    yf, _ = oracle.conv_bn_silu_f32(L.x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, 1, 1)
    assert np.abs(res["y"] - yf).max() < 0.1
    # points evaluation agrees
    pts = np.array([[1, 4, 6, 5], [0, 0, 0, 0], [1, 2, 3, 0]])
    yp, ap, absp = oracle.conv_bn_silu_i8_points(L.x, s_x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, 1, 1, pts)
    assert np.array_equal(ap, res["acc"][pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]])
    assert np.array_equal(yp, res["y"][pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]])
    assert np.array_equal(absp, res["absacc"][pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]])


# --------------------------------------------------------- calibration ----

def test_percentile_matches_numpy_and_normal_quantile():
    r = rng(13)
    for n in (1, 2, 17, 1000, 100003):
        x = r.standard_normal(n).astype(np.float32)
        for q in (0.0, 50.0, 99.0, 99.999, 100.0):
            got = oracle.percentile_abs(x, q)
            ref = np.percentile(np.abs(x.astype(np.float64)), q)
            assert abs(got - ref) <= 1e-12 * max(1.0, abs(ref)), (n, q, got, ref)
    # large N(0,1) sample: P99.999(|x|) -> Phi^-1(1 - 5e-6) = 4.4172 (sampling sd ~0.03 at n = 4e6)
    x = r.standard_normal(4_000_000).astype(np.float32)
    assert abs(oracle.percentile_abs(x, 99.999) - 4.4172) < 0.15
    # calibration input of the workloads uses the same rule
    s = W.calibration_scale(x)
    assert s == np.float32(np.percentile(np.abs(x.astype(np.float64)), 99.999) / 127.0)
    assert abs(float(s) * 127.0 - oracle.percentile_abs(x, 99.999)) < 1e-5


# ----------------------------------------------- golden: the page's bug ----

def buggy_tile_store(ow, block_ow, buggy):
    """CPU model of the page's tiled row store.  With the bug, the row stride is
    max(ow, block_ow) rounded to a multiple of 4 while the last tile still writes
    block_ow columns; returns the per-row count of columns written past OW."""
    stride = -(-max(ow, block_ow) // 4) * 4 if buggy else -(-ow // block_ow) * block_ow
    written = -(-ow // block_ow) * block_ow
    # columns of the last tile that land in the storage of the next row
    return max(0, written - stride)


def test_golden_tma_overflow_counts():
    """The page's printed damage: 8 columns per row at OW=40, 12 at OW=20 (BLOCK_OW=16)."""
    g = read_golden("tma_overflow.txt")
    for block_ow, ow, corrupted in g:
        block_ow, ow = int(block_ow), int(ow)
        assert block_ow - ow % block_ow == corrupted
        assert buggy_tile_store(ow, block_ow, buggy=True) == corrupted
        assert buggy_tile_store(ow, block_ow, buggy=False) == 0


# ------------------------------------------------------------- mutants ----
# Plausible mistakes, built on the CPU from the oracle; each must fail a pin.

def mutant_flipped_kernel(x, w, s, p):          # true convolution instead of cross-correlation
    return oracle.conv2d(x, np.ascontiguousarray(w[:, :, ::-1, ::-1]), s, p)


def mutant_dropped_channel(x, w, s, p):         # last input channel never summed
    w2 = np.array(w, copy=True)
    w2[:, -1] = 0
    return oracle.conv2d(x, w2, s, p)


def mutant_pad_off_by_one(x, w, s, p):          # window shifted by one pixel (pad - 1 on the left)
    xp = np.pad(x, ((0, 0), (0, 0), (0, 1), (0, 1)))
    y = oracle.conv2d(xp, w, s, p)
    return y[:, :, 1:1 + oracle.out_dim(x.shape[2], w.shape[2], s, p), 1:1 + oracle.out_dim(x.shape[3], w.shape[2], s, p)] \
        if y.shape[2] > 1 else y


def mutant_transposed_weights(x, w, s, p):      # kernel rows and columns swapped
    return oracle.conv2d(x, np.ascontiguousarray(w.transpose(0, 1, 3, 2)), s, p)


@pytest.mark.parametrize("mutant", [mutant_flipped_kernel, mutant_dropped_channel, mutant_pad_off_by_one,
                                    mutant_transposed_weights])
def test_conv_mutants_fail_some_pin(mutant):
    failed = [p.__name__ for p in CONV_PINS if not p(mutant)]
    assert failed, "mutant %s passed every pin" % mutant.__name__


def test_bn_mutants_fail():
    def fold_sign_error(w, g, b, m, v, eps):
        wf, bf = oracle.bn_fold(w, g, b, m, v, eps)
        sc = g.astype(np.float64) / np.sqrt(v.astype(np.float64) + eps)
        return wf, b.astype(np.float64) + m.astype(np.float64) * sc      # + mean instead of - mean

    def fold_no_sqrt(w, g, b, m, v, eps):
        sc = g.astype(np.float64) / (v.astype(np.float64) + eps)
        return w.astype(np.float64) * sc[:, None, None, None], b - m * sc

    def bn_eps_dropped(t, g, b, m, v, eps):
        return oracle.batchnorm(t, g, b, m, v, 0.0)

    assert not pin_fold_equals_unfolded(fold_sign_error, oracle.batchnorm)
    assert not pin_fold_equals_unfolded(fold_no_sqrt, oracle.batchnorm)
    assert not pin_bn_closed_form(bn_eps_dropped)


def test_quantiser_mutants_fail():
    def round_half_away(wf):
        q, sw = oracle.quantize_weights(wf)
        q2 = np.clip(np.sign(wf / sw[:, None]) * np.floor(np.abs(wf / sw[:, None]) + 0.5), -127, 127)
        return q2.astype(np.int8), sw

    def scale_255(wf):
        sw = np.abs(wf).max(axis=1) / 255.0
        sw[sw == 0] = 1.0
        return np.clip(np.rint(wf / sw[:, None]), -127, 127).astype(np.int8), sw

    def act_truncate(x, s):
        return np.clip(np.trunc(np.asarray(x, np.float32) / np.float32(s)), -127, 127).astype(np.int8)

    def act_no_clamp(x, s):
        return np.rint(np.asarray(x, np.float32) / np.float32(s)).astype(np.int64).astype(np.int8)

    assert not pin_quantize_weights(round_half_away)
    assert not pin_quantize_weights(scale_255)
    assert not pin_quantize_activations(act_truncate)
    assert not pin_quantize_activations(act_no_clamp)

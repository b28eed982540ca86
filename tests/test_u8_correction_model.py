"""CPU model of how the uint8-input kernels reach the exact asymmetric sum.

The int8 MFMA multiplies signed bytes, so a uint8 code q enters as q ^ 0x80 =
q - 128; a zero-padding tap, read as the byte 0 and flipped the same way,
enters as -128.  Each accumulator starts at 128 Wsum[co] - z Win[co, class],
where Wsum is the sum of the channel's int8 weights, Win the sum over the taps
whose window row and column lie inside the image, and the class is
(row mask) * 8 + (column mask) of the output pixel.  This test rebuilds that
arithmetic in numpy (independently of the kernels and of the host table code)
and checks it against the oracle's sum over q - z on the taps inside the
image, for k in {1, 3}, stride in {1, 2}, pad in {0, 1} and zero points at
both ends of the range.
"""
import numpy as np
import pytest

import oracle


def flipped_padded(q, pad):
    """The signed operand the MFMA sees: q - 128 inside, -128 on the padding."""
    v = q.astype(np.int64) - 128
    return np.pad(v, ((0, 0), (0, 0), (pad, pad), (pad, pad)), constant_values=-128)


def model_acc(q, z, qw, stride, pad):
    n, c, h, w = q.shape
    co, _, k, _ = qw.shape
    oh = (h + 2 * pad - k) // stride + 1
    ow = (w + 2 * pad - k) // stride + 1
    xp = flipped_padded(q, pad)
    wq = qw.astype(np.int64)
    s = np.zeros((n, co, oh, ow), np.int64)
    for i in range(k):
        for j in range(k):
            win = xp[:, :, i:i + stride * (oh - 1) + 1:stride, j:j + stride * (ow - 1) + 1:stride]
            s += np.einsum("oc,nchw->nohw", wq[:, :, i, j], win)
    T = wq.sum(axis=1)  # [co, k, k]
    wsum = T.reshape(co, -1).sum(axis=1)
    start = np.zeros((n, co, oh, ow), np.int64)
    for y in range(oh):
        for x in range(ow):
            iy0, ix0 = y * stride - pad, x * stride - pad
            rm = sum(1 << i for i in range(k) if 0 <= iy0 + i < h)
            cm = sum(1 << j for j in range(k) if 0 <= ix0 + j < w)
            win_sum = sum(T[:, i, j] for i in range(k) for j in range(k) if (rm >> i) & 1 and (cm >> j) & 1)
            start[:, :, y, x] = (128 * wsum - z * np.asarray(win_sum))[None, :]
    return s + start


@pytest.mark.parametrize("k,stride,pad", [(1, 1, 0), (1, 2, 0), (3, 1, 1), (3, 2, 1), (3, 1, 0), (3, 2, 0)])
@pytest.mark.parametrize("z", [0, 1, 77, 128, 254, 255])
def test_model_equals_asymmetric_sum(k, stride, pad, z):
    rng = np.random.default_rng(1000 + 7 * k + stride + 13 * pad + z)
    q = rng.integers(0, 256, (2, 5, 7, 6)).astype(np.uint8)
    qw = rng.integers(-127, 128, (6, 5, k, k)).astype(np.int8)
    got = model_acc(q, z, qw, stride, pad)
    want = oracle.conv_u8_acc(q, z, qw, stride, pad).astype(np.int64)
    assert np.array_equal(got, want)


def test_model_catches_a_wrong_padding_value():
    """The start value is tied to padding entering as -128: with padding read as 0
    (no flip) the same correction is wrong on the border, and only there."""
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, (1, 4, 6, 6)).astype(np.uint8)
    qw = rng.integers(-127, 128, (3, 4, 3, 3)).astype(np.int8)
    z = 40
    orig = flipped_padded
    try:
        globals()["flipped_padded"] = lambda q_, p_: np.pad(q_.astype(np.int64) - 128,
                                                             ((0, 0), (0, 0), (p_, p_), (p_, p_)))
        bad = model_acc(q, z, qw, 1, 1)
    finally:
        globals()["flipped_padded"] = orig
    want = oracle.conv_u8_acc(q, z, qw, 1, 1).astype(np.int64)
    diff = bad != want
    assert diff[:, :, 1:-1, 1:-1].sum() == 0 and diff.any()

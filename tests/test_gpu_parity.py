"""GPU parity: libcbs (through its C ABI) against the CPU oracle.

FP32: |y_gpu - y| <= 1e-4 * sum|W' x| + 1e-6 per output.
INT8: int32 accumulators and quantised weights bit-exact; outputs within
1e-4 * f[co] * sum|q_w q_x| + 1e-6.
Every run also checks that the guard pixels after each output row (and a
guard row after the tensor) are untouched and that padded output channels
are +0.0.

Workloads (seeded, synthetic): one 3x3 32->32 layer on 40x40; the ragged
sweep at output widths 80/40/20; the large-spatial stem layers; the 37-layer
YOLO26n-shaped list at batch 1 and batch 16, every output compared with the
whole-tensor oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from convolution_implicit_gemm_02_amd import workloads as W

pytestmark = pytest.mark.gpu

cbs = pytest.importorskip("convolution_implicit_gemm_02_amd.cbs") if torch.cuda.is_available() else None
if torch.cuda.is_available():
    from gpu_helpers import (SENTINEL, assert_f32_parity, assert_i8_parity, check_guards, create, dev,
                             pack_input, run_f32, run_i8, sample_points, alloc_out, split_out)


def _oracle_f32(L):
    return oracle.conv_bn_silu_f32(L.x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, L.spec.stride, L.spec.pad)


def _check_f32_full(L, **kw):
    r = run_f32(L, **kw)
    y, s = _oracle_f32(L)
    name = "%s n=%d %s" % (L.spec.name, L.n, r["info"]["config_name"])
    assert_f32_parity(r["y"], y, s, name)
    assert check_guards(r["host"], L, r["info"]) == 0, name + ": guard pixels written"
    pad = r["valid"][..., L.spec.c_out:]
    assert np.all(pad == 0), name + ": padded channels not +0.0"
    return r


def _check_i8_full(L, **kw):
    s_x = W.calibration_scale(L.x)
    r = run_i8(L, s_x, **kw)
    ref = oracle.conv_bn_silu_i8(L.x, s_x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, L.spec.stride, L.spec.pad)
    name = "%s n=%d %s int8" % (L.spec.name, L.n, r["info"]["config_name"])
    assert np.array_equal(r["acc"], ref["acc"]), name + ": int32 accumulators differ (%d)" % int(
        np.count_nonzero(r["acc"] != ref["acc"]))
    qw, sw = cbs.cbs_get_qweights(r["layer"])
    assert np.array_equal(qw, ref["qw"]) and np.array_equal(sw, ref["s_w"]), name + ": quantised weights differ"
    assert_i8_parity(r["y"], ref["y"], ref["f"], ref["absacc"], name)
    assert check_guards(r["host"], L, r["info"]) == 0, name + ": guard pixels written"
    assert check_guards(r["acc_host"], L, r["info"], fill=np.int32(np.uint32(0xA5A5A5A5).view(np.int32))) == 0
    assert np.all(r["valid"][..., L.spec.c_out:] == 0), name + ": padded channels not +0.0"
    assert np.all(r["acc_valid"][..., L.spec.c_out:] == 0)
    return r


# ------------------------------------------------------- graph-entry ops --

def test_pack_nhwc_f32_exact():
    rng = np.random.default_rng(0)
    for n, c, h, w in ((1, 3, 17, 9), (2, 8, 5, 6), (1, 13, 4, 4), (3, 64, 7, 3)):
        cpad = -(-c // 4) * 4
        x = rng.standard_normal((n, c, h, w)).astype(np.float32)
        xd = torch.from_numpy(x).to(dev())
        out = torch.full((n * h * w * cpad,), float("nan"), dtype=torch.float32, device=dev())
        cbs.cbs_pack_nhwc_f32(xd, out, n, c, h, w, cpad)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(n, h, w, cpad)
        exp = np.zeros((n, h, w, cpad), np.float32)
        exp[..., :c] = x.transpose(0, 2, 3, 1)
        assert np.array_equal(got.view(np.int32), exp.view(np.int32))


def test_quantize_nhwc_i8_bit_exact():
    rng = np.random.default_rng(1)
    for n, c, h, w in ((1, 3, 31, 7), (2, 24, 5, 6), (1, 64, 9, 9)):
        cpad = -(-c // 4) * 4
        x = (2 * rng.standard_normal((n, c, h, w))).astype(np.float32)
        x.flat[:8] = [0.5, -0.5, 1.5, 2.5, -2.5, 1e9, -1e9, 0.0]  # ties and clamps (scaled below)
        s_x = W.calibration_scale(x)
        xd = torch.from_numpy(x).to(dev())
        out = torch.full((n * h * w * cpad,), 99, dtype=torch.int8, device=dev())
        cbs.cbs_quantize_nhwc_i8(xd, out, s_x, n, c, h, w, cpad)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(n, h, w, cpad)
        ref = oracle.quantize_activations(x, s_x).transpose(0, 2, 3, 1)
        assert np.array_equal(got[..., :c], ref)
        assert np.all(got[..., c:] == 0)
    # exact ties: s_x = 1 -> x.5 rounds to even
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.5, -127.5, 200.0], np.float32).reshape(1, 10, 1, 1)
    out = torch.zeros(12, dtype=torch.int8, device=dev())
    cbs.cbs_quantize_nhwc_i8(torch.from_numpy(x).to(dev()), out, 1.0, 1, 10, 1, 1, 12)
    torch.cuda.synchronize()
    assert list(out.cpu().numpy()[:10]) == [0, 2, 2, 0, -2, -2, 126, 127, -127, 127]


def test_quantize_nhwc_u8_bit_exact():
    """Asymmetric uint8 graph-entry quantiser: the oracle's codes bit for bit, padded
    lanes set to the zero point, ties to even before the zero point is added."""
    rng = np.random.default_rng(2)
    for n, c, h, w, dist in ((1, 3, 31, 7, "uniform"), (2, 24, 5, 6, "normal"), (1, 64, 9, 9, "normal")):
        cpad = -(-c // 4) * 4
        x = (rng.random((n, c, h, w)) if dist == "uniform" else 2 * rng.standard_normal((n, c, h, w)))
        x = x.astype(np.float32)
        x.flat[:6] = [1e9, -1e9, 0.0, -0.0, 3.0, -3.0]
        s_x, z = W.calibration_u8(x)
        xd = torch.from_numpy(x).to(dev())
        out = torch.full((n * h * w * cpad,), 77, dtype=torch.uint8, device=dev())
        cbs.cbs_quantize_nhwc_u8(xd, out, s_x, z, n, c, h, w, cpad)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(n, h, w, cpad)
        ref = oracle.quantize_activations_u8(x, s_x, z).transpose(0, 2, 3, 1)
        assert np.array_equal(got[..., :c], ref), "%d codes differ" % int(np.count_nonzero(got[..., :c] != ref))
        assert np.all(got[..., c:] == z)
    # exact ties with s_x = 1 and z = 10: x.5 rounds to even, then + 10, clamped to 0..255
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -10.5, -11.0, 244.5, 245.5, 300.0], np.float32).reshape(1, 10, 1, 1)
    out = torch.zeros(12, dtype=torch.uint8, device=dev())
    cbs.cbs_quantize_nhwc_u8(torch.from_numpy(x).to(dev()), out, 1.0, 10, 1, 10, 1, 1, 12)
    torch.cuda.synchronize()
    assert list(out.cpu().numpy()[:10]) == [10, 12, 12, 10, 8, 0, 0, 254, 255, 255]


# ----------------------------------------------------------------- FP32 --

@pytest.mark.parametrize("workload", ["single", "ragged", "stem"])
def test_f32_workloads_bs1(workload):
    for L in W.generate(workload, n=1, seed=0):
        _check_f32_full(L)


def test_f32_yolo26n_list_bs1():
    for L in W.generate("yolo26n", n=1, seed=0):
        _check_f32_full(L)


def test_f32_yolo26n_list_bs16_full():
    """Every output of the batch-16 list against the whole-tensor oracle (FP32 bound),
    guards and padded lanes included."""
    for L in W.generate("yolo26n", n=16, seed=0):
        _check_f32_full(L)


def test_f32_ragged_and_stem_batched_full():
    for L in W.generate("ragged", n=16, seed=0) + W.generate("stem", n=2, seed=0):
        _check_f32_full(L)


def _small_cases():
    cases = [W.LayerSpec("1x1x1", 1, 1, 1, 1, 1, 1, 0), W.LayerSpec("3x3 on 1x1", 1, 1, 1, 1, 3, 1, 1),
             W.LayerSpec("odd", 5, 7, 9, 11, 3, 2, 1), W.LayerSpec("tall", 3, 16, 37, 3, 3, 1, 1),
             W.LayerSpec("wide", 24, 80, 2, 45, 1, 1, 0), W.LayerSpec("c3s2", 3, 16, 33, 34, 3, 2, 1),
             W.LayerSpec("k3p0", 20, 36, 10, 9, 3, 1, 0), W.LayerSpec("k3s2p0", 20, 36, 10, 9, 3, 2, 0),
             W.LayerSpec("k1s2", 40, 33, 13, 12, 1, 2, 0), W.LayerSpec("c48", 48, 32, 20, 20, 1, 1, 0)]
    rng = np.random.default_rng(42)
    for _ in range(8):
        spec, _ = W.random_case(rng, max_hw=23, max_c=70)
        cases.append(spec)
    return cases


def test_f32_small_and_random_shapes():
    rng = np.random.default_rng(5)
    for spec in _small_cases():
        for n in (1, 3):
            _check_f32_full(W.draw_layer(rng, spec, n))


def test_every_config_on_every_shape_f32():
    """Force each kernel configuration and several split-K factors on a set of
    shapes, so that the tile table's choice cannot hide a broken variant."""
    rng = np.random.default_rng(6)
    specs = [W.LayerSpec("r3", 32, 32, 13, 11, 3, 1, 1), W.LayerSpec("r1", 40, 80, 9, 10, 1, 1, 0),
             W.LayerSpec("s2", 12, 24, 15, 14, 3, 2, 1), W.LayerSpec("stem", 3, 16, 21, 22, 3, 2, 1),
             # <= 8 output channels, 3x3 stride 1: the column-pair halo tiles run too (odd OW: a
             # half-used last pair; 6 channels: padded rows; 3 channels: a 4-channel output pitch)
             W.LayerSpec("c8", 8, 8, 13, 11, 3, 1, 1), W.LayerSpec("c6", 12, 6, 9, 14, 3, 1, 1),
             W.LayerSpec("c3", 4, 3, 10, 9, 3, 1, 1),
             # halo tiles above 64 KiB of LDS (input window + 36 or 72 KiB of fp32 weights)
             W.LayerSpec("lds32", 32, 32, 21, 23, 3, 1, 1), W.LayerSpec("lds64s2", 32, 64, 17, 19, 3, 2, 1)]
    for spec in specs:
        L = W.draw_layer(rng, spec, 2)
        y, s = _oracle_f32(L)
        layer = create(L, cbs.CBS_F32)
        for cfg in range(cbs.cbs_num_configs()):
            for sk in (1, 2, 3, 5):
                try:
                    cbs.cbs_layer_set_config(layer, cfg, sk)
                except cbs.CbsError as e:
                    assert e.status == cbs.CBS_EUNSUPPORTED
                    continue
                r = run_f32(L, layer=layer)
                name = "%s %s" % (spec.name, r["info"]["config_name"])
                assert_f32_parity(r["y"], y, s, name)
                assert check_guards(r["host"], L, r["info"]) == 0, name


# fp32 1x1 shapes for the weight-stationary tiles (W.*): every compiled K depth,
# input channel counts that end in a partial K step (20, 22, 24, 40; 72 has no
# compiled partial depth) or have no compiled depth (80: 5 steps), channel
# counts that leave a workgroup's last
# channel blocks empty, ragged
# pixel counts, and (larger batches) runs of several 16-pixel blocks per
# workgroup, odd run lengths included.
WS_SPECS = [(W.LayerSpec("ws64", 64, 80, 9, 13, 1, 1, 0), 2), (W.LayerSpec("ws96", 96, 40, 7, 9, 1, 1, 0), 2),
            (W.LayerSpec("ws128", 128, 136, 11, 5, 1, 1, 0), 2), (W.LayerSpec("ws192", 192, 24, 5, 7, 1, 1, 0), 2),
            (W.LayerSpec("ws256", 256, 48, 6, 6, 1, 1, 0), 2), (W.LayerSpec("ws384", 384, 20, 3, 5, 1, 1, 0), 2),
            (W.LayerSpec("ws128runs", 128, 72, 49, 50, 1, 1, 0), 3),
            (W.LayerSpec("ws128long", 128, 128, 40, 40, 1, 1, 0), 8),
            (W.LayerSpec("ws16", 16, 16, 31, 29, 1, 1, 0), 3), (W.LayerSpec("ws32", 32, 24, 17, 21, 1, 1, 0), 2),
            (W.LayerSpec("ws16runs", 16, 32, 80, 80, 1, 1, 0), 4), (W.LayerSpec("ws64c80", 64, 80, 40, 40, 1, 1, 0), 4),
            (W.LayerSpec("ws128c80", 128, 80, 20, 20, 1, 1, 0), 3), (W.LayerSpec("ws48", 48, 16, 5, 5, 1, 1, 0), 1),
            (W.LayerSpec("ws24", 24, 16, 19, 17, 1, 1, 0), 3), (W.LayerSpec("ws40", 40, 32, 9, 11, 1, 1, 0), 2),
            (W.LayerSpec("ws20", 20, 24, 7, 9, 1, 1, 0), 2), (W.LayerSpec("ws22", 22, 16, 7, 7, 1, 1, 0), 1),
            (W.LayerSpec("ws80", 80, 16, 5, 5, 1, 1, 0), 1), (W.LayerSpec("ws72", 72, 16, 5, 5, 1, 1, 0), 1)]


def ws_runs(name, c_in):
    """Whether weight-stationary 1x1 configuration `name` takes a layer with c_in input
    channels: K steps (C_in rounded up to 4, over 16, rounded up) of a compiled depth,
    within the wave's register budget (24 steps with one channel block per wave, 16 with
    two, 8 with five)."""
    cb = {"c16": 1, "c32": 2, "c80": 5}[name[2:5]]
    cin_pad = -(-c_in // 4) * 4
    ks = -(-cin_pad // 16)
    return (ks in (1, 2, 3, 4, 6, 8, 12, 16, 24) and ks <= {1: 24, 2: 16, 5: 8}[cb]
            and (cin_pad % 16 == 0 or ks <= 3))  # partial last steps: depths 1-3


def test_weight_stationary_tiles_f32():
    rng = np.random.default_rng(13)
    ws = [c for c in range(cbs.cbs_num_configs()) if cbs.cbs_config_name(c).startswith("W.")]
    assert ws
    for spec, n in WS_SPECS:
        L = W.draw_layer(rng, spec, n)
        y, s = _oracle_f32(L)
        layer = create(L, cbs.CBS_F32)
        ran = []
        for cfg in ws:
            try:
                cbs.cbs_layer_set_config(layer, cfg, 1)
            except cbs.CbsError as e:
                assert e.status == cbs.CBS_EUNSUPPORTED
                continue
            r = run_f32(L, layer=layer)
            name = "%s n=%d %s" % (spec.name, n, r["info"]["config_name"])
            assert_f32_parity(r["y"], y, s, name)
            assert check_guards(r["host"], L, r["info"]) == 0, name
            ran.append(r["info"]["config_name"])
        want = sorted(cbs.cbs_config_name(c) + "/sk1" for c in ws if ws_runs(cbs.cbs_config_name(c), spec.c_in))
        assert sorted(ran) == want, (spec.name, ran, want)
        if want:
            assert "W.c16x4/sk1" in ran  # every depth runs on the 16-channel tiles
        with pytest.raises(cbs.CbsError) as e:  # no cross-workgroup split-K on these tiles
            cbs.cbs_layer_set_config(layer, ws[0], 2)
        assert e.value.status == cbs.CBS_EUNSUPPORTED


# 3x3 layers for the weight-stationary tiles with the window gather: 16 and 32
# input channels (9 and 18 K steps), stride 1 and 2, with and without padding,
# ragged rows and channel counts, several pixel blocks per run; 24 and 48 input
# channels (K steps across taps) must be refused.
WSG_SPECS = [(W.LayerSpec("g16", 16, 16, 21, 23, 3, 1, 1), 2), (W.LayerSpec("g16s2", 16, 40, 33, 29, 3, 2, 1), 2),
             (W.LayerSpec("g32", 32, 32, 17, 19, 3, 1, 1), 3), (W.LayerSpec("g32s2", 32, 64, 26, 31, 3, 2, 1), 2),
             (W.LayerSpec("g32p0", 32, 24, 11, 14, 3, 1, 0), 2), (W.LayerSpec("g16runs", 16, 32, 80, 80, 3, 1, 1), 4),
             (W.LayerSpec("g24", 24, 16, 9, 9, 3, 1, 1), 1), (W.LayerSpec("g48", 48, 16, 9, 9, 3, 1, 1), 1)]


# int8 1x1 shapes for the weight-stationary tiles (64-channel K steps): depths 1,
# 2, 4 and 6, partial last steps with 16-channel chunks (16, 32, 96 input
# channels) and with 4-channel chunks (20, 24, 72, 136; 200 has no compiled
# partial depth), runs of several blocks, channel counts that leave channel
# blocks empty.
WS_I8_SPECS = [(W.LayerSpec("wq16", 16, 16, 31, 29, 1, 1, 0), 3), (W.LayerSpec("wq32", 32, 24, 17, 21, 1, 1, 0), 2),
               (W.LayerSpec("wq64c80", 64, 80, 40, 40, 1, 1, 0), 4), (W.LayerSpec("wq96", 96, 64, 9, 11, 1, 1, 0), 2),
               (W.LayerSpec("wq128", 128, 136, 11, 5, 1, 1, 0), 2), (W.LayerSpec("wq256", 256, 48, 6, 6, 1, 1, 0), 2),
               (W.LayerSpec("wq384", 384, 20, 3, 5, 1, 1, 0), 2), (W.LayerSpec("wq64runs", 64, 32, 49, 50, 1, 1, 0), 3),
               # 4-channel chunks (C_in not a multiple of 16): one, two and three partial steps
               (W.LayerSpec("wq24", 24, 16, 29, 31, 1, 1, 0), 3), (W.LayerSpec("wq20", 20, 40, 9, 11, 1, 1, 0), 2),
               (W.LayerSpec("wq72", 72, 24, 7, 9, 1, 1, 0), 2), (W.LayerSpec("wq136", 136, 16, 6, 5, 1, 1, 0), 2),
               (W.LayerSpec("wq200", 200, 16, 5, 5, 1, 1, 0), 1)]


def test_weight_stationary_tiles_i8():
    """int8 activations on the weight-stationary 1x1 tiles: int32 accumulators bit-exact
    (raw output), dequantised output within the int8 band, guards untouched."""
    rng = np.random.default_rng(16)
    ws = [c for c in range(cbs.cbs_num_configs()) if cbs.cbs_config_name(c).startswith("W.")]
    for spec, n in WS_I8_SPECS:
        L = W.draw_layer(rng, spec, n)
        s_x = W.calibration_scale(L.x)
        ref = oracle.conv_bn_silu_i8(L.x, s_x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, spec.stride, spec.pad)
        layer = create(L, cbs.CBS_I8, s_x=s_x)
        ran = []
        for cfg in ws:
            try:
                cbs.cbs_layer_set_config(layer, cfg, 1)
            except cbs.CbsError as e:
                assert e.status == cbs.CBS_EUNSUPPORTED
                continue
            r = run_i8(L, s_x, layer=layer)
            name = "%s n=%d %s" % (spec.name, n, r["info"]["config_name"])
            assert np.array_equal(r["acc"], ref["acc"]), name
            assert_i8_parity(r["y"], ref["y"], ref["f"], ref["absacc"], name)
            assert check_guards(r["host"], L, r["info"]) == 0, name
            assert np.all(r["valid"][..., spec.c_out:] == 0), name
            ran.append(r["info"]["config_name"])
        cin_pad = -(-spec.c_in // 4) * 4
        ks = -(-cin_pad // 64)
        max_steps = {"c16": 24, "c32": 16, "c80": 8}
        want = sorted(cbs.cbs_config_name(c) + "/sk1" for c in ws
                      if ks in (1, 2, 3, 4, 6) and (cin_pad % 64 == 0 or ks <= 3)
                      and ks <= max_steps[cbs.cbs_config_name(c)[2:5]])
        assert sorted(ran) == want, (spec.name, ran, want)


def test_weight_stationary_gather_tiles_f32():
    rng = np.random.default_rng(14)
    gs = [c for c in range(cbs.cbs_num_configs()) if cbs.cbs_config_name(c).startswith("G.")]
    assert gs
    for spec, n in WSG_SPECS:
        L = W.draw_layer(rng, spec, n)
        y, s = _oracle_f32(L)
        layer = create(L, cbs.CBS_F32)
        ran = []
        for cfg in gs:
            try:
                cbs.cbs_layer_set_config(layer, cfg, 1)
            except cbs.CbsError as e:
                assert e.status == cbs.CBS_EUNSUPPORTED
                continue
            r = run_f32(L, layer=layer)
            name = "%s n=%d %s" % (spec.name, n, r["info"]["config_name"])
            assert_f32_parity(r["y"], y, s, name)
            assert check_guards(r["host"], L, r["info"]) == 0, name
            ran.append(r["info"]["config_name"])
        assert len(ran) == (len(gs) if spec.c_in in (16, 32) else 0), (spec.name, ran)
        if ran:
            with pytest.raises(cbs.CbsError) as e:  # no cross-workgroup split-K on these tiles
                cbs.cbs_layer_set_config(layer, gs[0], 2)
            assert e.value.status == cbs.CBS_EUNSUPPORTED


def test_folded_delta_kernel_gives_silu_of_input():
    """cbs_create_layer_folded with W = delta (3x3 centre), scale 1, bias 0: y = SiLU(x)."""
    rng = np.random.default_rng(7)
    c = 24
    spec = W.LayerSpec("delta", c, c, 19, 21, 3, 1, 1)
    L = W.draw_layer(rng, spec, 2)
    w = np.zeros((c, c, 3, 3), np.float32)
    for i in range(c):
        w[i, i, 1, 1] = 1.0
    d = cbs.make_desc(2, c, 19, 21, c, 3, 1, 1, cbs.CBS_F32, 21 + 64)
    layer = cbs.cbs_create_layer_folded(d, w, np.ones(c, np.float32), np.zeros(c, np.float32))
    r = run_f32(L, layer=layer)
    x = L.x.astype(np.float64)
    assert_f32_parity(r["y"], oracle.silu(x), np.abs(x), "delta")
    wf, b = cbs.cbs_get_folded(layer)
    assert np.array_equal(wf, w) and np.all(b == 0)


def test_determinism_and_streams():
    """Two runs are bitwise identical (split-K included) and a non-default stream works."""
    rng = np.random.default_rng(8)
    L = W.draw_layer(rng, W.LayerSpec("det", 128, 128, 20, 20, 3, 1, 1), 1)
    layer = create(L, cbs.CBS_F32)
    info = cbs.cbs_layer_info(layer)
    s = torch.cuda.Stream()
    outs = []
    for stream in (None, s, s):
        with torch.cuda.stream(s) if stream is s else torch.cuda.stream(torch.cuda.current_stream()):
            r = run_f32(L, layer=layer, stream=stream)
        outs.append(r["host"])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2]), info["config_name"]
    # force a split-K configuration and repeat
    for cfg in range(cbs.cbs_num_configs()):
        try:
            cbs.cbs_layer_set_config(layer, cfg, 4)
        except cbs.CbsError:
            continue
        a = run_f32(L, layer=layer)["host"]
        b = run_f32(L, layer=layer)["host"]
        assert np.array_equal(a, b), cbs.cbs_layer_info(layer)["config_name"]


def _list_case():
    """Six layers for the list and graph tests: FP32 ragged layers (one forced to a
    cross-workgroup split-K), and INT8 layers (one forced to split-K as well).
    Returns [(LayerInputs, dtype, s_x, layer, input, output buffer)] and the oracle
    answers [(y, bound)]."""
    rows, refs = [], []
    fp = W.generate("ragged", n=1, seed=3)[:4]
    i8 = W.generate("ragged", n=1, seed=4)[2:4]
    for k, (L, dt) in enumerate([(L, cbs.CBS_F32) for L in fp] + [(L, cbs.CBS_I8) for L in i8]):
        s_x = W.calibration_scale(L.x) if dt == cbs.CBS_I8 else None
        layer = create(L, dt, s_x=s_x)
        if k in (2, 4):  # the 256-channel 20x20 3x3 layers: force a split-K register-direct configuration
            for cfg in range(cbs.cbs_num_configs()):
                try:
                    cbs.cbs_layer_set_config(layer, cfg, 3)
                    break
                except cbs.CbsError:
                    continue
            assert cbs.cbs_layer_info(layer)["splitk"] == 3
        xin = pack_input(L, dt, s_x=s_x)
        buf, info = alloc_out(L, layer)
        rows.append((L, dt, s_x, layer, xin, buf))
        if dt == cbs.CBS_F32:
            y, b = _oracle_f32(L)
            refs.append((y, 1e-4 * b + 1e-6))
        else:
            r = oracle.conv_bn_silu_i8(L.x, s_x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, L.spec.stride,
                                       L.spec.pad)
            refs.append((r["y"], 1e-4 * r["f"].astype(np.float64)[None, :, None, None] * r["absacc"] + 1e-6))
    return rows, refs


def _check_list_outputs(rows, refs, what):
    for (L, dt, s_x, layer, xin, buf), (y, tol) in zip(rows, refs):
        info = cbs.cbs_layer_info(layer)
        host = buf.cpu().numpy()
        valid, _, _ = split_out(host, L, info)
        got = valid.view(np.float32)[..., : L.spec.c_out].transpose(0, 3, 1, 2)
        name = "%s %s %s" % (what, L.spec.name, info["config_name"])
        err = np.abs(got.astype(np.float64) - y)
        assert not np.isnan(got).any() and not (err > tol).any(), name + ": outside tolerance"
        assert check_guards(host, L, info) == 0, name + ": guard pixels written"


def test_layer_list_and_graph_replay():
    """cbs_run_layer_list and a captured graph, FP32 and INT8 layers with forced split-K
    among them, against the oracle; the graph is replayed several times with other
    eager work in between (every replay re-arms the split-K tickets)."""
    rows, refs = _list_case()
    layers, ins, outs = [r[3] for r in rows], [r[4] for r in rows], [r[5] for r in rows]
    eager = []
    for layer, xin, buf in zip(layers, ins, outs):
        cbs.cbs_run_layer(layer, xin, buf)
    torch.cuda.synchronize()
    _check_list_outputs(rows, refs, "eager")
    eager = [b.cpu().numpy() for b in outs]
    for b in outs:
        b.fill_(int(SENTINEL))
    cbs.cbs_run_layer_list(layers, ins, outs)
    torch.cuda.synchronize()
    _check_list_outputs(rows, refs, "list")
    for e, b in zip(eager, outs):
        assert np.array_equal(e, b.cpu().numpy())
    g = cbs.cbs_graph_create(layers, ins, outs)
    for rep in range(3):
        for b in outs:
            b.fill_(int(SENTINEL))
        torch.cuda.synchronize()
        cbs.cbs_graph_launch(g)
        torch.cuda.synchronize()
        _check_list_outputs(rows, refs, "replay %d" % rep)
        for e, b in zip(eager, outs):
            assert np.array_equal(e, b.cpu().numpy()), "replay %d" % rep
        _ = torch.randn(1000, device=dev()).sum().item()  # unrelated eager work between replays


def test_graph_keeps_splitk_workspace():
    """A graph holds its layers' split-K workspace addresses: while it lives, a
    configuration needing a larger workspace is refused (the layer is unchanged), a
    smaller one is accepted without moving the workspace, and replays still run the
    captured configuration correctly; after the graph is destroyed the larger one is
    accepted."""
    rng = np.random.default_rng(12)
    L = W.draw_layer(rng, W.LayerSpec("ws", 128, 128, 20, 20, 3, 1, 1), 1)
    y, b = _oracle_f32(L)
    tol = 1e-4 * b + 1e-6
    layer = create(L, cbs.CBS_F32)
    cfg = None
    for c in range(cbs.cbs_num_configs()):
        try:
            cbs.cbs_layer_set_config(layer, c, 2)
            cfg = c
            break
        except cbs.CbsError:
            continue
    assert cfg is not None
    xin = pack_input(L, cbs.CBS_F32)
    buf, info = alloc_out(L, layer)
    g = cbs.cbs_graph_create([layer], [xin], [buf])
    with pytest.raises(cbs.CbsError) as e:
        cbs.cbs_layer_set_config(layer, cfg, 4)  # twice the partial tiles
    assert e.value.status == cbs.CBS_EINVAL
    assert cbs.cbs_layer_info(layer)["splitk"] == 2
    cbs.cbs_layer_set_config(layer, cfg, 1)      # fits: accepted, the workspace stays
    for rep in range(3):
        buf.fill_(int(SENTINEL))
        torch.cuda.synchronize()
        cbs.cbs_graph_launch(g)                  # still the captured split-K 2
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        got = split_out(host, L, info)[0].view(np.float32)[..., : L.spec.c_out].transpose(0, 3, 1, 2)
        assert not (np.abs(got.astype(np.float64) - y) > tol).any(), "replay %d" % rep
        assert check_guards(host, L, info) == 0
        r = run_f32(L, layer=layer)              # eager split-K 1 in between
        assert_f32_parity(r["y"], y, b, "eager sk1")
    del g
    import gc
    gc.collect()
    cbs.cbs_layer_set_config(layer, cfg, 4)
    r = run_f32(L, layer=layer)
    assert_f32_parity(r["y"], y, b, "sk4 after the graph")


def test_graph_create_grouped():
    """cbs_graph_create_grouped: the grouped step gives the oracle's outputs whether a
    group is kept or not, reports its measurements, and refuses groupings that would
    reorder dependent layers."""
    rows, refs = _list_case()
    rows, refs = rows[:4], refs[:4]  # FP32 layers: one variant
    layers, ins, outs = [r[3] for r in rows], [r[4] for r in rows], [r[5] for r in rows]
    g = cbs.cbs_graph_create_grouped(layers, ins, outs, [0, 1, 0, 1])
    launches, ngroups = cbs.cbs_graph_info(g)
    assert ngroups == 2
    infos = [cbs.cbs_graph_group_info(g, i) for i in range(2)]
    assert [i["group_id"] for i in infos] == [0, 1] and all(i["members"] == 2 for i in infos)
    assert launches == 4 - sum(i["kept"] for i in infos)
    assert all(i["us_separate"] > 0 for i in infos)
    for rep in range(2):
        for b in outs:
            b.fill_(int(SENTINEL))
        torch.cuda.synchronize()
        cbs.cbs_graph_launch(g)
        torch.cuda.synchronize()
        _check_list_outputs(rows, refs, "grouped replay %d" % rep)
    # a member reading another member's output: layer 0 writes a buffer that layer 1 reads
    shared = torch.empty(max(layers[0].out_bytes, layers[1].in_bytes), dtype=torch.uint8, device=dev())
    with pytest.raises(cbs.CbsError) as e:
        cbs.cbs_graph_create_grouped(layers[:2], [ins[0], shared], [shared, outs[1]], [0, 0])
    assert e.value.status == cbs.CBS_EINVAL
    # a layer between two members reading the first member's output
    with pytest.raises(cbs.CbsError):
        cbs.cbs_graph_create_grouped(layers[:3], [ins[0], shared, ins[2]], [shared, outs[1], outs[2]], [0, -1, 0])
    # more than CBS_GROUP_MAX members, a bad id
    with pytest.raises(cbs.CbsError):
        cbs.cbs_graph_create_grouped(layers + layers[:1], ins + ins[:1], outs + outs[:1], [0] * 5)
    with pytest.raises(cbs.CbsError):
        cbs.cbs_graph_create_grouped(layers, ins, outs, [0, -2, 0, 1])


# ----------------------------------------------------------------- INT8 --

@pytest.mark.parametrize("workload", ["single", "ragged", "stem"])
def test_i8_workloads_bs1(workload):
    for L in W.generate(workload, n=1, seed=0):
        _check_i8_full(L)


def test_i8_yolo26n_list_bs1():
    for L in W.generate("yolo26n", n=1, seed=0):
        _check_i8_full(L)


def test_i8_yolo26n_list_bs16_full():
    """Every int32 accumulator of the batch-16 list bit-exact, every output within the
    INT8 bound, against the whole-tensor oracle."""
    for L in W.generate("yolo26n", n=16, seed=0):
        _check_i8_full(L)


def test_i8_small_and_random_shapes():
    rng = np.random.default_rng(9)
    for spec in _small_cases():
        for n in (1, 2):
            _check_i8_full(W.draw_layer(rng, spec, n))


def test_every_config_on_every_shape_i8():
    rng = np.random.default_rng(10)
    specs = [W.LayerSpec("r3", 64, 32, 9, 11, 3, 1, 1), W.LayerSpec("r1", 48, 80, 9, 10, 1, 1, 0),
             W.LayerSpec("c4", 12, 24, 15, 14, 3, 2, 1), W.LayerSpec("stem", 3, 16, 21, 22, 3, 2, 1),
             # column-pair halo tiles on both int8 gathers (4- and 16-channel chunks)
             W.LayerSpec("c8", 8, 8, 13, 11, 3, 1, 1), W.LayerSpec("c16to6", 16, 6, 7, 10, 3, 1, 1)]
    for spec in specs:
        L = W.draw_layer(rng, spec, 2)
        s_x = W.calibration_scale(L.x)
        ref = oracle.conv_bn_silu_i8(L.x, s_x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, spec.stride, spec.pad)
        layer = create(L, cbs.CBS_I8, s_x=s_x)
        for cfg in range(cbs.cbs_num_configs()):
            for sk in (1, 2, 3):
                try:
                    cbs.cbs_layer_set_config(layer, cfg, sk)
                except cbs.CbsError as e:
                    assert e.status == cbs.CBS_EUNSUPPORTED
                    continue
                r = run_i8(L, s_x, layer=layer)
                name = "%s %s" % (spec.name, r["info"]["config_name"])
                assert np.array_equal(r["acc"], ref["acc"]), name
                assert_i8_parity(r["y"], ref["y"], ref["f"], ref["absacc"], name)
                assert check_guards(r["host"], L, r["info"]) == 0, name

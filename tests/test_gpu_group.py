"""Grouped launches (cbs_group_*): several independent layers in one kernel.

Every member's output is checked against the oracle with the bands of the
other parity tests (test_gpu_fusion), the guard pixels and padded channels of
every member are checked after every run, and:
  * int8 and uint8 members, whose int32 sums are exact whatever the tile, give
    bit-for-bit the output of their own single-layer launch;
  * an fp32 group run with a member's own configuration gives that member's
    single-launch output bit for bit (same tile, same summation order);
  * every register-direct configuration that fits is run;
  * a group captured in a HIP graph gives the eager result on every replay.
"""
import numpy as np
import pytest
import torch

from convolution_implicit_gemm_02_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from convolution_implicit_gemm_02_amd import cbs
    from test_gpu_fusion import SENT_F32, SENT_I8, SENT_U8, Case, check, prepare, out_geometry


def dev():
    return torch.device("cuda", 0)


def spec(c_in, c_out, h, w, k, s):
    return W.LayerSpec("g", c_in, c_out, h, w, k, s, k // 2)


# the detection head's three scales (batch 1) and smaller stand-ins of mixed kinds
HEAD_3X3 = [spec(64, 64, 80, 80, 3, 1), spec(128, 64, 40, 40, 3, 1), spec(256, 64, 20, 20, 3, 1)]
HEAD_1X1 = [spec(64, 80, 80, 80, 1, 1), spec(64, 80, 40, 40, 1, 1), spec(64, 80, 20, 20, 1, 1)]
MIXED = [spec(32, 48, 17, 23, 3, 2), spec(64, 16, 9, 7, 1, 1), spec(48, 32, 12, 12, 3, 1), spec(16, 64, 30, 5, 3, 1)]


def register_direct_configs():
    return [i for i in range(cbs.cbs_num_configs()) if cbs.cbs_config_name(i).startswith("c")]


def groupable_configs():
    """Register-direct and LDS-staged tiles (halo and weight-stationary tiles have no grouped kernel)."""
    return [i for i in range(cbs.cbs_num_configs()) if not cbs.cbs_config_name(i).startswith(("H", "P", "W.", "G."))]


class Member:
    """A prepared layer with a sentinel-filled output buffer on the device."""

    def __init__(self, case):
        self.case = case
        self.prep = prepare(case)
        self.layer = self.prep["layer"]
        self.info = cbs.cbs_layer_info(self.layer)
        sp = case.spec
        ostride, _, _ = out_geometry(case, self.info)
        self.shape = (case.n * sp.oh + 1, self.info["out_row_pitch"], ostride)
        self.fill = {"f32": SENT_F32, "i8": SENT_I8, "u8": SENT_U8}[case.out]
        self.xin = torch.from_numpy(self.prep["xin"]).to(dev())
        self.obuf = torch.empty(0)
        self.reset()

    def reset(self):
        self.obuf = torch.from_numpy(np.full(self.shape, self.fill)).to(dev())

    def result(self):
        """The written NCHW region, after checking guards and padded channels."""
        case, sp = self.case, self.case.spec
        got = self.obuf.cpu().numpy()
        _, _, (c0, c1) = out_geometry(case, self.info)
        mask = np.ones(self.shape, bool)
        mask[: case.n * sp.oh, : sp.ow, c0:c1] = False
        bad = int(np.count_nonzero(got[mask] != self.fill))
        assert bad == 0, "%r: %d elements outside the output were written" % (case, bad)
        region = got[: case.n * sp.oh, : sp.ow, c0:c1].reshape(case.n, sp.oh, sp.ow, c1 - c0)
        if case.out == "f32":
            region = region.view(np.float32)
        if c1 - c0 > sp.c_out:
            assert np.all(region[..., sp.c_out:] == self.prep["z_y"]), "%r: padded channels not zero" % case
        return region[..., : sp.c_out].transpose(0, 3, 1, 2).copy()

    def single(self):
        """This layer's output from its own launch."""
        self.reset()
        cbs.cbs_run_layer(self.layer, self.xin, self.obuf)
        torch.cuda.synchronize()
        return self.result()


def run_group(group, members):
    for m in members:
        m.reset()
    cbs.cbs_group_run(group, [m.xin for m in members], [m.obuf for m in members])
    torch.cuda.synchronize()
    return [m.result() for m in members]


def make_members(specs, dtype, out, n=1, seed=80):
    return [Member(Case(sp, n=n, dtype=dtype, out=out, extra=5, seed=seed + i)) for i, sp in enumerate(specs)]


@pytest.mark.parametrize("n", [1, 16])
@pytest.mark.parametrize("dtype,out", [("f32", "f32"), ("i8", "f32"), ("i8", "i8"), ("u8", "u8")])
@pytest.mark.parametrize("which", ["head3x3", "head1x1"])
def test_detection_head_group(which, dtype, out, n):
    """The head's three scales at full size, batch 1 and 16 (the shapes the list step groups),
    with the cost model's configuration and with c64p128, which the batch-16 list picks."""
    specs = HEAD_3X3 if which == "head3x3" else HEAD_1X1
    members = make_members(specs, dtype, out, n=n)
    singles = [m.single() for m in members]
    names = [cbs.cbs_config_name(i) for i in range(cbs.cbs_num_configs())]
    for cfg in (-1, names.index("c64p128")):
        group = cbs.cbs_group_create([m.layer for m in members], cfg)
        assert cbs.cbs_config_name(cbs.cbs_group_config(group)).startswith("c")
        got = run_group(group, members)
        for m, g, s in zip(members, got, singles):
            check(m.case, m.prep, g)
            if dtype != "f32":
                assert np.array_equal(g, s), "%r: group output differs from the single launch" % m.case


@pytest.mark.parametrize("dtype", ["f32", "i8", "u8"])
def test_group_every_config(dtype):
    """Mixed shapes (3x3 s1/s2, 1x1, ragged tails, batch 2) through every register-direct and
    LDS-staged configuration."""
    out = "u8" if dtype == "u8" else "f32"
    members = make_members(MIXED, dtype, out, n=2, seed=90)
    singles = [m.single() for m in members]
    ran = 0
    for cfg in groupable_configs():
        group = cbs.cbs_group_create([m.layer for m in members], cfg)
        assert cbs.cbs_group_config(group) == cfg
        got = run_group(group, members)
        for m, g, s in zip(members, got, singles):
            check(m.case, m.prep, g)
            if dtype != "f32":
                assert np.array_equal(g, s), "%r config %s" % (m.case, cbs.cbs_config_name(cfg))
        ran += 1
    assert ran == len(groupable_configs())


def test_fp32_group_with_own_config_is_bit_identical():
    members = make_members(HEAD_3X3, "f32", "f32", seed=100)
    for m in members:
        cfg = m.info["config"]
        if cfg not in groupable_configs():
            continue
        cbs.cbs_layer_set_config(m.layer, cfg, 1)
        single = m.single()
        group = cbs.cbs_group_create([m.layer], cfg)
        (got,) = run_group(group, [m])
        assert np.array_equal(got, single)


def test_member_order_and_subsets():
    """Any order and any subset: outputs land in the caller's buffers."""
    members = make_members(MIXED, "i8", "i8", seed=110)
    singles = [m.single() for m in members]
    for order in ([3, 1, 0, 2], [2, 0], [1]):
        sub = [members[i] for i in order]
        got = run_group(cbs.cbs_group_create([m.layer for m in sub]), sub)
        for i, g in zip(order, got):
            assert np.array_equal(g, singles[i])


def test_group_in_a_graph():
    members = make_members(HEAD_3X3, "i8", "f32", seed=120)
    singles = [m.single() for m in members]
    group = cbs.cbs_group_create([m.layer for m in members])
    for m in members:
        m.reset()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cbs.cbs_group_run(group, [m.xin for m in members], [m.obuf for m in members])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cbs.cbs_group_run(group, [m.xin for m in members], [m.obuf for m in members])
    for _ in range(3):
        for m in members:
            m.obuf.fill_(0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m, single in zip(members, singles):
            got = m.obuf.cpu().numpy()
            sp = m.case.spec
            _, _, (c0, c1) = out_geometry(m.case, m.info)
            region = got[: sp.oh, : sp.ow, c0:c1].view(np.float32)[..., : sp.c_out].transpose(2, 0, 1)
            assert np.array_equal(region, single[0])


def test_group_rejections():
    f32 = make_members([MIXED[1]], "f32", "f32", seed=130)[0]
    i8 = make_members([MIXED[1]], "i8", "f32", seed=131)[0]
    i8out = make_members([MIXED[1]], "i8", "i8", seed=132)[0]
    with pytest.raises(cbs.CbsError) as e:
        cbs.cbs_group_create([f32.layer, i8.layer])
    assert e.value.status == cbs.CBS_EUNSUPPORTED
    with pytest.raises(cbs.CbsError) as e:  # plain and general epilogue variants do not mix
        cbs.cbs_group_create([i8.layer, i8out.layer])
    assert e.value.status == cbs.CBS_EUNSUPPORTED
    res = Member(Case(MIXED[1], n=1, dtype="f32", res_sl=(16, 0), extra=5, seed=133))
    with pytest.raises(cbs.CbsError) as e:
        cbs.cbs_group_create([res.layer])
    assert e.value.status == cbs.CBS_EUNSUPPORTED and "residual" in str(e.value)
    for cfg in range(cbs.cbs_num_configs()):
        if cfg in groupable_configs():
            continue
        with pytest.raises(cbs.CbsError) as e:  # halo tiles have no grouped kernel
            cbs.cbs_group_create([f32.layer], cfg)
        assert e.value.status == cbs.CBS_EUNSUPPORTED
    with pytest.raises(cbs.CbsError) as e:
        cbs.cbs_group_create([f32.layer], cbs.cbs_num_configs())
    assert e.value.status == cbs.CBS_EUNSUPPORTED
    with pytest.raises(cbs.CbsError) as e:
        cbs.cbs_group_create([f32.layer] * (cbs.CBS_GROUP_MAX + 1))
    assert e.value.status == cbs.CBS_EINVAL

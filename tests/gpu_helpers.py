"""Helpers for the GPU parity tests: run one layer through the C ABI with
guard pixels around the output, and compare against the oracle.

Output buffers carry `extra` guard pixels after every (n, oh) row (the
descriptor's out_row_pitch = OW + extra) and one whole guard row after the
tensor; every guard element is filled with a sentinel bit pattern before the
run and must still hold it afterwards (the overflow of the vision-rs page,
section "Bug fixed: TMA overflow", would show up there).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from convolution_implicit_gemm_02_amd import cbs
from convolution_implicit_gemm_02_amd import workloads as W

SENTINEL = np.int32(np.uint32(0x7FA5A5A5).view(np.int32))  # a NaN payload no kernel writes
SENTINEL_ACC = np.int32(np.uint32(0xA5A5A5A5).view(np.int32))


def dev():
    return torch.device("cuda", 0)


def create(L: W.LayerInputs, dtype: int, extra: int = 64, s_x=None, config=None, splitk=0):
    spec = L.spec
    pitch = spec.ow + extra
    desc = cbs.make_desc(L.n, spec.c_in, spec.h, spec.w, spec.c_out, spec.k, spec.stride, spec.pad, dtype,
                         pitch, float(s_x) if s_x is not None else 0.0, L.eps)
    layer = cbs.cbs_create_layer(desc, L.w, L.gamma, L.beta, L.mean, L.var)
    if config is not None:
        cbs.cbs_layer_set_config(layer, config, splitk)
    return layer


def pack_input(L: W.LayerInputs, dtype: int, s_x=None, stream=None):
    """Upload the NCHW fp32 input and convert it with the library's graph-entry kernel."""
    spec = L.spec
    cpad = -(-spec.c_in // 4) * 4
    x = torch.from_numpy(L.x).to(dev())
    n_el = L.n * spec.h * spec.w * cpad
    if dtype == cbs.CBS_F32:
        xin = torch.empty(n_el, dtype=torch.float32, device=dev())
        cbs.cbs_pack_nhwc_f32(x, xin, L.n, spec.c_in, spec.h, spec.w, cpad, stream)
    else:
        xin = torch.empty(n_el, dtype=torch.int8, device=dev())
        cbs.cbs_quantize_nhwc_i8(x, xin, s_x, L.n, spec.c_in, spec.h, spec.w, cpad, stream)
    return xin


def alloc_out(L: W.LayerInputs, layer, fill=SENTINEL):
    info = cbs.cbs_layer_info(layer)
    pitch, cpad = info["out_row_pitch"], info["c_out_pad"]
    n_el = (L.n * info["oh"] * pitch + pitch) * cpad
    buf = torch.full((n_el,), int(fill), dtype=torch.int32, device=dev())
    return buf, info


def split_out(buf_host: np.ndarray, L: W.LayerInputs, info):
    """-> (valid NHWC [n,oh,ow,cpad] view, guard-pixel elements, trailing guard row)."""
    pitch, cpad, oh, ow = info["out_row_pitch"], info["c_out_pad"], info["oh"], info["ow"]
    main = buf_host[: L.n * oh * pitch * cpad].reshape(L.n, oh, pitch, cpad)
    tail = buf_host[L.n * oh * pitch * cpad:]
    return main[:, :, :ow, :], main[:, :, ow:, :], tail


def check_guards(buf_host, L, info, fill=SENTINEL):
    _, guard, tail = split_out(buf_host, L, info)
    bad = int(np.count_nonzero(guard != fill)) + int(np.count_nonzero(tail != fill))
    return bad


def run_f32(L: W.LayerInputs, extra=64, config=None, splitk=0, stream=None, layer=None):
    """Run an FP32 layer; returns dict with y (NCHW float32 of the valid region), the raw
    output buffer (int32 view, host) and info."""
    if layer is None:
        layer = create(L, cbs.CBS_F32, extra, config=config, splitk=splitk)
    xin = pack_input(L, cbs.CBS_F32, stream=stream)
    buf, info = alloc_out(L, layer)
    cbs.cbs_run_layer(layer, xin, buf, stream)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    valid, _, _ = split_out(host, L, info)
    y = valid.view(np.float32)[..., : L.spec.c_out].transpose(0, 3, 1, 2)
    return {"y": y, "host": host, "info": info, "layer": layer, "valid": valid}


def run_i8(L: W.LayerInputs, s_x, extra=64, config=None, splitk=0, stream=None, raw=True, layer=None):
    if layer is None:
        layer = create(L, cbs.CBS_I8, extra, s_x=s_x, config=config, splitk=splitk)
    xin = pack_input(L, cbs.CBS_I8, s_x=s_x, stream=stream)
    buf, info = alloc_out(L, layer)
    cbs.cbs_run_layer(layer, xin, buf, stream)
    res = {"layer": layer, "info": info}
    if raw:
        abuf, _ = alloc_out(L, layer, fill=SENTINEL_ACC)
        cbs.cbs_run_layer_raw_acc(layer, xin, abuf, stream)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    valid, _, _ = split_out(host, L, info)
    res.update(host=host, valid=valid, y=valid.view(np.float32)[..., : L.spec.c_out].transpose(0, 3, 1, 2))
    if raw:
        ahost = abuf.cpu().numpy()
        avalid, _, _ = split_out(ahost, L, info)
        res.update(acc_host=ahost, acc_valid=avalid, acc=avalid[..., : L.spec.c_out].transpose(0, 3, 1, 2))
    return res


def f32_tolerance(sabs):
    return 1e-4 * sabs + 1e-6


def assert_f32_parity(y_gpu, y_ref, sabs, what=""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = f32_tolerance(sabs)
    bad = err > tol
    assert not np.isnan(y_gpu).any(), "%s: NaN in GPU output" % what
    assert not bad.any(), "%s: %d/%d outputs outside 1e-4*S+1e-6 (max err %.3g, worst ratio %.3g)" % (
        what, int(bad.sum()), bad.size, float(err.max()), float((err / tol).max()))


def assert_i8_parity(y_gpu, y_ref, f, absacc, what=""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = 1e-4 * f.astype(np.float64)[None, :, None, None] * absacc + 1e-6 if absacc.ndim == 4 else \
        1e-4 * absacc + 1e-6
    bad = err > tol
    assert not np.isnan(y_gpu).any(), "%s: NaN in GPU output" % what
    assert not bad.any(), "%s: %d/%d outputs outside tolerance (max err %.3g)" % (
        what, int(bad.sum()), bad.size, float(err.max()))


def sample_points(rng, n, c_out, oh, ow, count):
    """Random outputs plus the four corners and edge midpoints of every (n, co) plane sampled."""
    pts = np.stack([rng.integers(0, n, count), rng.integers(0, c_out, count), rng.integers(0, oh, count),
                    rng.integers(0, ow, count)], axis=1)
    extra = []
    for b in sorted({0, n - 1}):
        for co in sorted({0, c_out - 1, c_out // 2}):
            for i in sorted({0, oh - 1, oh // 2}):
                for j in sorted({0, ow - 1, ow // 2}):
                    extra.append((b, co, i, j))
    return np.concatenate([pts, np.array(extra)], axis=0).astype(np.int32)

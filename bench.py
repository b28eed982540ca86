"""Benchmark: the 37-layer YOLO26n-shaped fused Conv2d + BN + SiLU list on one MI355X.

One step = one pass of the whole list (every layer's fused conv + folded BN +
SiLU, inputs already resident in HBM in the library's NHWC layout), replayed
as one captured HIP graph.  The detection head's three scales are independent
of each other, so its three 3x3 layers, and its three 1x1 layers, run as one
grouped launch each (cbs_group_run) wherever that measured faster than their
separate launches (the library's cbs_graph_create_grouped measures and
decides that); the list with one launch per layer (37 launches) is reported
beside it.  The headline is FP32 at batch 1
(the configuration of the vision-rs "YOLO26N Inference Optimisation" page:
YOLO26N, FP32, batch 1, 640x640); the same line also carries INT8 and batch 16.

Printed (stdout, one JSON line): value = list FLOPs / step time (TFLOP/s),
ms_per_step, per-layer roofline of the dominant kernel (HIP events on the
launch stream), and the CPU oracle timed on the host cores as a baseline.
Per-layer details go to gpurun_out/bench_layers.json when that folder exists.

The line also carries INT8 with int8 output (the requantising epilogue) and
the 25 backbone layers chained as five downsample + C3k2 stages through
channel slices and fused residuals (chain_*).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused conv-BN-SiLU TFLOP/s + total µs for YOLO26n layer list, bs1 FP32/INT8"
# MI355X published peaks (dense): FP32 matrix 157.3 TFLOP/s, INT8 5.0 POP/s, HBM3E 8 TB/s.
PEAK_FP32 = 157.3e12
PEAK_INT8 = 5.0e15
PEAK_HBM = 8.0e12


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class ListBench:
    """Device-resident inputs/outputs and created layers for one (dtype, batch).
    out_i8: INT8 layers write int8 codes (the requantising epilogue) instead of
    fp32; the output scale is the layer's own input scale (timing does not
    depend on the value).  CBS_U8: asymmetric uint8 input codes (min/max
    calibration of each layer's input), fp32 output."""

    def __init__(self, cbs, W, torch, dtype, batch, seed=0, out_i8=False):
        self.cbs, self.torch = cbs, torch
        self.dtype = dtype
        self.batch = batch
        dev = torch.device("cuda", 0)
        self.layers, self.ins, self.outs, self.infos, self.specs = [], [], [], [], []
        for L in W.generate("yolo26n", n=batch, seed=seed):
            sp = L.spec
            cpad = -(-sp.c_in // 4) * 4
            x = torch.from_numpy(L.x).to(dev)
            if dtype == cbs.CBS_F32:
                desc = cbs.make_desc(batch, sp.c_in, sp.h, sp.w, sp.c_out, sp.k, sp.stride, sp.pad, dtype, 0, 0.0,
                                     L.eps)
                xin = torch.empty(batch * sp.h * sp.w * cpad, dtype=torch.float32, device=dev)
                cbs.cbs_pack_nhwc_f32(x, xin, batch, sp.c_in, sp.h, sp.w, cpad)
            elif dtype == cbs.CBS_U8:
                s_x, z_x = W.calibration_u8(L.x)
                desc = cbs.make_desc(batch, sp.c_in, sp.h, sp.w, sp.c_out, sp.k, sp.stride, sp.pad, dtype, 0,
                                     float(s_x), L.eps, in_zero_point=z_x)
                xin = torch.empty(batch * sp.h * sp.w * cpad, dtype=torch.uint8, device=dev)
                cbs.cbs_quantize_nhwc_u8(x, xin, s_x, z_x, batch, sp.c_in, sp.h, sp.w, cpad)
            else:
                s_x = W.calibration_scale(L.x)
                desc = cbs.make_desc(batch, sp.c_in, sp.h, sp.w, sp.c_out, sp.k, sp.stride, sp.pad, dtype, 0,
                                     float(s_x), L.eps, out_dtype=cbs.CBS_I8 if out_i8 else cbs.CBS_F32,
                                     out_scale=float(s_x) if out_i8 else 0.0)
                xin = torch.empty(batch * sp.h * sp.w * cpad, dtype=torch.int8, device=dev)
                cbs.cbs_quantize_nhwc_i8(x, xin, s_x, batch, sp.c_in, sp.h, sp.w, cpad)
            layer = cbs.cbs_create_layer(desc, L.w, L.gamma, L.beta, L.mean, L.var)
            info = cbs.cbs_layer_info(layer)
            out = torch.empty(info["out_bytes"], dtype=torch.uint8, device=dev)
            self.layers.append(layer)
            self.ins.append(xin)
            self.outs.append(out)
            self.infos.append(info)
            self.specs.append(sp)
            del x
        torch.cuda.synchronize()
        self.flops = sum(i["flops"] for i in self.infos)
        self.graph = cbs.cbs_graph_create(self.layers, self.ins, self.outs)

    def autotune(self, iters=20):
        """Create-time tuning of every layer on its own buffers (cbs_layer_autotune), then
        re-capture the graph.  Returns the number of layers whose configuration changed."""
        changed = 0
        for i, (layer, xin, out) in enumerate(zip(self.layers, self.ins, self.outs)):
            before = (self.infos[i]["config"], self.infos[i]["splitk"])
            after = self.cbs.cbs_layer_autotune(layer, xin, out, iters=iters)
            changed += after != before
            self.infos[i] = self.cbs.cbs_layer_info(layer)
        self.torch.cuda.synchronize()
        self.graph = self.cbs.cbs_graph_create(self.layers, self.ins, self.outs)
        return changed

    # the detection head's three scales are independent of each other: its 3x3
    # layers form one candidate group and its 1x1 layers another
    HEAD_GROUPS = (("head64.3x3", "head128.3x3", "head256.3x3"), ("head64.1x1", "head128.1x1", "head256.1x1"))

    def group_head(self):
        """Capture the step with the head's scales as candidate groups
        (cbs_graph_create_grouped): the library times each group's separate and
        grouped launches on these buffers and keeps a grouped launch only where
        it is faster.  Returns [(members, config name, us, us separately, kept)]."""
        cbs = self.cbs
        names = [sp.name for sp in self.specs]
        group_of = [-1] * len(names)
        for gid, members in enumerate(self.HEAD_GROUPS):
            for m in members:
                group_of[names.index(m)] = gid
        self.grouped_graph = cbs.cbs_graph_create_grouped(self.layers, self.ins, self.outs, group_of)
        self.grouped_launches, ngroups = cbs.cbs_graph_info(self.grouped_graph)
        chosen = []
        for i in range(ngroups):
            g = cbs.cbs_graph_group_info(self.grouped_graph, i)
            chosen.append((self.HEAD_GROUPS[g["group_id"]], cbs.cbs_config_name(g["config"]),
                           round(g["us_grouped"], 2), round(g["us_separate"], 2), bool(g["kept"])))
        return chosen

    def time_grouped(self, steps, warmup):
        """Time replays of the grouped step (see group_head)."""
        torch, cbs = self.torch, self.cbs
        for _ in range(warmup):
            cbs.cbs_graph_launch(self.grouped_graph)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            cbs.cbs_graph_launch(self.grouped_graph)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def time_steps(self, steps, warmup, use_graph=True):
        torch, cbs = self.torch, self.cbs
        for _ in range(warmup):
            self._step(use_graph)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self._step(use_graph)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall / steps * 1e3

    def time_prefix(self, n, steps, warmup):
        """The first n layers of the list as one captured graph (one launch per
        layer, in list order): ms per replay."""
        torch, cbs = self.torch, self.cbs
        g = cbs.cbs_graph_create(self.layers[:n], self.ins[:n], self.outs[:n])
        for _ in range(warmup):
            cbs.cbs_graph_launch(g)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            cbs.cbs_graph_launch(g)
        e1.record()
        torch.cuda.synchronize()
        cbs.cbs_graph_destroy(g)
        return e0.elapsed_time(e1) / steps

    def _step(self, use_graph):
        if use_graph:
            self.cbs.cbs_graph_launch(self.graph)
        else:
            self.cbs.cbs_run_layer_list(self.layers, self.ins, self.outs)

    def time_layers(self, min_ms=2.0, reps=5):
        """Per layer: (graph us, eager us).  graph: median over `reps` of (event pair
        around one replay of a captured graph of R back-to-back launches)/R, the way
        the list step launches its kernels; eager: the same R launches enqueued by one
        cbs_run_layer_list call (marshalled before the events).  R is chosen so that
        one repeat takes >= min_ms.  All on the stream the library launches on
        (torch's current stream)."""
        torch, cbs = self.torch, self.cbs
        graph_us, eager_us = [], []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for layer, xin, out in zip(self.layers, self.ins, self.outs):
            cbs.cbs_run_layer_list([layer] * 3, [xin] * 3, [out] * 3)
            ten = cbs.LayerList([layer] * 10, [xin] * 10, [out] * 10)
            torch.cuda.synchronize()
            e0.record()
            ten.run()
            e1.record()
            torch.cuda.synchronize()
            per = max(e0.elapsed_time(e1) / 10, 1e-4)
            r = int(min(2000, max(10, min_ms / per)))
            lst = cbs.LayerList([layer] * r, [xin] * r, [out] * r)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                lst.run()
            g.replay()
            torch.cuda.synchronize()
            tg, te = [], []
            for _ in range(reps):
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                tg.append(e0.elapsed_time(e1) / r)
                e0.record()
                lst.run()
                e1.record()
                torch.cuda.synchronize()
                te.append(e0.elapsed_time(e1) / r)
            del g
            graph_us.append(float(np.median(tg)) * 1e3)  # microseconds
            eager_us.append(float(np.median(te)) * 1e3)
        return graph_us, eager_us

    def time_layers_single(self, scratch, reps=9):
        """Per layer, one launch between two events: the median over `reps` with warm
        caches (the launch right after the same one), and the median over `reps`
        with the caches flushed first (a write of the whole `scratch` buffer,
        larger than the L2 and the 256 MB MALL, outside the events)."""
        torch, cbs = self.torch, self.cbs
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm, cold = [], []
        for layer, xin, out in zip(self.layers, self.ins, self.outs):
            tw, tc = [], []
            for _ in range(reps):
                cbs.cbs_run_layer(layer, xin, out)
                e0.record()
                cbs.cbs_run_layer(layer, xin, out)
                e1.record()
                torch.cuda.synchronize()
                tw.append(e0.elapsed_time(e1))
                scratch.fill_(1)
                torch.cuda.synchronize()
                e0.record()
                cbs.cbs_run_layer(layer, xin, out)
                e1.record()
                torch.cuda.synchronize()
                tc.append(e0.elapsed_time(e1))
            warm.append(float(np.median(tw)) * 1e3)
            cold.append(float(np.median(tc)) * 1e3)
        return warm, cold


class ChainBench:
    """The 25 backbone layers of the list chained as they run in the network: five
    stages, each a 3x3 s2 downsample and a C3k2 block (cv1 1x1; the bottleneck's
    two 3x3 convs read the second half of cv1's output in place and the second
    adds it back; cv2 1x1 reads the concatenation of cv1's output and the
    bottleneck's).  FP32 at batch 16 keeps that concatenation as two dense
    tensors in the stages of up to 64 channels, which cv2 reads as its two
    inputs; elsewhere one 1.5c-channel buffer T holds it, which cv1 (the first c
    channels) and the bottleneck (the last c/2) write slices of.
    Each stage's output is the next stage's input.  One step = 25 kernels, no
    cat / chunk / add kernel, replayed as one captured graph.  INT8: every
    tensor is int8 codes (scales: the calibration of the list layers'
    generated inputs; timing does not depend on them)."""

    def __init__(self, cbs, W, torch, int8, batch, seed=0):
        self.cbs, self.torch, self.batch = cbs, torch, batch
        dev = torch.device("cuda", 0)
        gen = W.generate("yolo26n", n=batch, seed=seed)[:25]
        DT = cbs.CBS_I8 if int8 else cbs.CBS_F32
        tdt = torch.int8 if int8 else torch.float32
        img = gen[0]
        cpad = 4
        x = torch.from_numpy(img.x).to(dev)
        cur = torch.empty(batch * img.spec.h * img.spec.w * cpad, dtype=tdt, device=dev)
        s_img = W.calibration_scale(img.x)
        s_act = W.calibration_scale(gen[1].x)  # an N(0,1) feature map
        if int8:
            cbs.cbs_quantize_nhwc_i8(x, cur, s_img, batch, img.spec.c_in, img.spec.h, img.spec.w, cpad)
        else:
            cbs.cbs_pack_nhwc_f32(x, cur, batch, img.spec.c_in, img.spec.h, img.spec.w, cpad)
        self.input = cur
        self.layers, self.steps, self.bufs, self.flops = [], [], [], 0
        s_in = s_img
        for st in range(5):
            down, cv1, b1, b2, cv2 = gen[5 * st: 5 * st + 5]
            c, h = cv1.spec.c_out, cv1.spec.h
            half = c // 2
            # FP32 at batch 16 keeps the concatenation of the large stages (up to 64
            # channels) as two dense tensors (cv1's output and b2's), which cv2 reads
            # as its two inputs; INT8, FP32 at batch 1 and the 128- and 256-channel
            # stages keep one buffer that cv1 and b2 write slices of (a second input
            # holds cv2 to the weight-stationary tiles, which lose there)
            split = not int8 and batch > 1 and c <= 64
            D = torch.empty(batch * h * h * c, dtype=tdt, device=dev)
            T = torch.empty(batch * h * h * (c if split else 3 * half), dtype=tdt, device=dev)
            T2 = torch.empty(batch * h * h * half, dtype=tdt, device=dev) if split else None
            U = torch.empty(batch * h * h * half, dtype=tdt, device=dev)
            Y = torch.empty(batch * h * h * c, dtype=tdt, device=dev)

            def mk(L, s_x, **kw):
                sp = L.spec
                d = cbs.make_desc(batch, sp.c_in, sp.h, sp.w, sp.c_out, sp.k, sp.stride, sp.pad, DT, 0,
                                  float(s_x) if int8 else 0.0, L.eps, out_dtype=DT,
                                  out_scale=float(s_act) if int8 else 0.0, **kw)
                layer = cbs.cbs_create_layer(d, L.w, L.gamma, L.beta, L.mean, L.var)
                self.layers.append(layer)
                self.flops += cbs.cbs_layer_info(layer)["flops"]
                return layer

            ld = mk(down, s_in)
            if split:
                l1 = mk(cv1, s_act)
                lb1 = mk(b1, s_act, in_c_stride=c, in_c_offset=half)
                lb2 = mk(b2, s_act, res_c_stride=c, res_c_offset=half)
                l2 = mk(cv2, s_act, in2_channels=half)
                self.steps += [(ld, cur, D), (l1, D, T), (lb1, T, U), (lb2, U, T2, T), (l2, T, Y, None, T2)]
                self.bufs += [D, T, T2, U, Y]
            else:
                l1 = mk(cv1, s_act, out_c_stride=3 * half, out_c_offset=0)
                lb1 = mk(b1, s_act, in_c_stride=3 * half, in_c_offset=half)
                lb2 = mk(b2, s_act, out_c_stride=3 * half, out_c_offset=2 * half, res_c_stride=3 * half,
                         res_c_offset=half, res_scale=float(s_act) if int8 else 0.0)
                l2 = mk(cv2, s_act)
                self.steps += [(ld, cur, D), (l1, D, T), (lb1, T, U), (lb2, U, T, T), (l2, T, Y)]
                self.bufs += [D, T, U, Y]
            cur, s_in = Y, s_act
        torch.cuda.synchronize()
        self.graph = cbs.cbs_graph_create_steps(self.steps)

    def time_layers(self, min_ms=2.0, reps=5):
        """Per chained step: the median over `reps` of (event pair around one replay
        of a captured graph of R back-to-back launches of that step)/R, in us, as
        ListBench.time_layers times the list's layers."""
        torch, cbs = self.torch, self.cbs
        out = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for st in self.steps:
            cbs.cbs_run_steps([st] * 3)
            ten = cbs.StepList([st] * 10)
            torch.cuda.synchronize()
            e0.record()
            ten.run()
            e1.record()
            torch.cuda.synchronize()
            per = max(e0.elapsed_time(e1) / 10, 1e-4)
            r = int(min(2000, max(10, min_ms / per)))
            lst = cbs.StepList([st] * r)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                lst.run()
            g.replay()
            torch.cuda.synchronize()
            t = []
            for _ in range(reps):
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                t.append(e0.elapsed_time(e1) / r)
            del g
            out.append(float(np.median(t)) * 1e3)
        return out

    def time_steps(self, steps, warmup, use_graph=True):
        torch, cbs = self.torch, self.cbs
        run = (lambda: cbs.cbs_graph_launch(self.graph)) if use_graph else (lambda: cbs.cbs_run_steps(self.steps))
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps


def warm_device(torch, seconds=0.5):
    """Keep the device busy with plain copies for a moment before the first timed
    region, so that the first configuration is not timed while clocks ramp up."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def layer_rows(bench, us, single=None, flushed=None, eager=None):
    int8 = bench.dtype != bench.cbs.CBS_F32
    peak = PEAK_INT8 if int8 else PEAK_FP32
    rows = []
    single = single or [None] * len(us)
    flushed = flushed or [None] * len(us)
    eager = eager or [None] * len(us)
    for sp, info, t, t1, tf, te in zip(bench.specs, bench.infos, us, single, flushed, eager):
        fl, by = info["flops"], info["alg_bytes"]
        t_mfma, t_hbm = fl / peak, by / PEAK_HBM
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        roof_us = max(t_mfma, t_hbm) * 1e6
        rows.append({"layer": sp.name, "c_in": sp.c_in, "c_out": sp.c_out, "h_in": sp.h, "k": sp.k, "s": sp.stride,
                     "us": round(t, 3), "tflops": round(fl / (t * 1e-6) / 1e12, 3),
                     "gbs": round(by / (t * 1e-6) / 1e9, 1), "flops": fl, "alg_bytes": by, "bound": bound,
                     "roof_us": round(roof_us, 3), "frac": round(roof_us / t, 4), "config": info["config_name"],
                     "grid": info["grid"], "us_single": None if t1 is None else round(t1, 3),
                     "us_flushed": None if tf is None else round(tf, 3),
                     "us_eager": None if te is None else round(te, 3)})
    return rows


KERNEL_SOURCES = ("convolution_implicit_gemm_02_amd/csrc/conv_kernels.h",
                  "convolution_implicit_gemm_02_amd/csrc/conv_configs.h",
                  "convolution_implicit_gemm_02_amd/csrc/cbs_variant.hip",
                  "convolution_implicit_gemm_02_amd/csrc/cbs_kernels.hip",
                  "convolution_implicit_gemm_02_amd/csrc/cbs_host.cpp",
                  "convolution_implicit_gemm_02_amd/csrc/cbs_internal.h",
                  "convolution_implicit_gemm_02_amd/csrc/tile_table.inc")


def measured_traffic(layer):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summaries (profiles/traffic_dominant.json, one entry
    per layer that can come out dominant), scaled by the counters of a plain
    copy of known size.  None when no entry covers the layer or the kernel
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_dominant.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    entry = rec.get("layers", {}).get(layer)
    if entry is None or rec.get("source_sha256") != h.hexdigest():
        return None
    return entry["traffic_bytes"]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_oracle_list(W, int8, min_seconds, max_seconds):
    """The oracle on the batch-1 list, layer by layer in list order, repeated until
    at least min_seconds of oracle time, or cut short once max_seconds is passed:
    (layers done, layers per list, FLOPs done, seconds, seconds per whole list
    extrapolated by FLOPs)."""
    import oracle
    layers = W.generate("yolo26n", n=1, seed=0)
    scales = [W.calibration_scale(L.x) for L in layers] if int8 else None
    done_flops, t_total, done = 0, 0.0, 0
    while t_total < min_seconds:
        for i, L in enumerate(layers):
            t0 = time.perf_counter()
            if int8:
                oracle.conv_bn_act_i8(L.x, scales[i], L.w, L.gamma, L.beta, L.mean, L.var, L.eps, L.spec.stride,
                                      L.spec.pad, with_bound=False)
            else:
                oracle.conv_bn_silu_f32(L.x, L.w, L.gamma, L.beta, L.mean, L.var, L.eps, L.spec.stride, L.spec.pad,
                                        with_bound=False)
            t_total += time.perf_counter() - t0
            done_flops += L.spec.flops(1)
            done += 1
            if t_total > max_seconds:
                break
        if t_total > max_seconds:
            break
    list_flops = sum(L.spec.flops(1) for L in layers)
    return done, len(layers), done_flops, t_total, t_total * list_flops / done_flops


def _sample(done, total, flops):
    if done >= total:
        return "%.1f passes of the %d-layer list (%.2f GFLOP)" % (done / total, total, flops / 1e9)
    return "%d of %d layers (%.3f GFLOP)" % (done, total, flops / 1e9)


def cpu_baseline(W, min_seconds=10.0, max_seconds=20.0):
    """The oracle as it stands (plain C, double accumulation for FP32, exact int32
    sums for INT8, OpenMP) on the batch-1 list: FP32 with every host core (the
    reported value), then FP32 with one thread and INT8 with every core.  Each
    leg repeats the list for at least `min_seconds` of oracle time and stops
    once it passes `max_seconds` (mid-list if need be; a partial list is
    extrapolated by FLOPs)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env:
        threads = min(threads, int(env))
    oracle.set_threads(threads)
    done, total, flops, sec, per_list = _time_oracle_list(W, False, min_seconds, max_seconds)
    res = {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.get_threads(), "kind": "oracle",
           "sample": "yolo26n list, batch 1, FP32, oracle conv+BN+SiLU in double: " + _sample(done, total, flops),
           "seconds": round(sec, 3), "us_per_list": round(per_list * 1e6, 1), "cpu_model": cpu_model()}
    oracle.set_threads(1)
    done, total, flops, sec, per_list = _time_oracle_list(W, False, min_seconds, max_seconds)
    res["single_thread"] = {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                            "sample": "FP32: " + _sample(done, total, flops), "seconds": round(sec, 3),
                            "us_per_list": round(per_list * 1e6, 1)}
    oracle.set_threads(threads)
    done, total, flops, sec, per_list = _time_oracle_list(W, True, min_seconds, max_seconds)
    res["int8"] = {"value": round(flops / sec / 1e12, 6), "unit": "TOP/s", "cores": oracle.get_threads(),
                   "sample": "INT8 (exact int32 sums, fp32 output): " + _sample(done, total, flops),
                   "seconds": round(sec, 3), "us_per_list": round(per_list * 1e6, 1)}
    return res


def profile_layer(cbs, W, torch, name, dtype, batch, launches, config=None, splitk=0):
    """Run only one layer of the list (or, for name "all", every layer in list
    order): 10 eager warm-up launches, then `launches` back-to-back launches
    captured as one graph, replayed twice (an untimed warm-up replay, then the
    timed one, as bench.py's per-layer figures are timed), for a profiler run
    on exactly those kernels: 10 + 2 * launches dispatches per layer.  Then a
    plain device copy of known size (the reference for scaling the
    profiler's byte counters).  Prints one JSON line per layer."""
    b = ListBench(cbs, W, torch, dtype, batch)
    names = [s.name for s in b.specs]
    for i in range(len(names)) if name == "all" else [names.index(name)]:
        layer, xin, out = b.layers[i], b.ins[i], b.outs[i]
        if config is not None:
            cbs.cbs_layer_set_config(layer, config, splitk)
            b.infos[i] = cbs.cbs_layer_info(layer)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cbs.cbs_run_layer_list([layer] * 10, [xin] * 10, [out] * 10)
        lst = cbs.LayerList([layer] * launches, [xin] * launches, [out] * launches)
        g = torch.cuda.CUDAGraph()  # the launches replayed as one graph, as bench.py times them
        with torch.cuda.graph(g):
            lst.run()
        g.replay()  # warm-up replay
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        us = e0.elapsed_time(e1) / launches * 1e3
        info = b.infos[i]
        print(json.dumps({"layer": names[i], "batch": batch, "dtype": "int8" if dtype else "f32",
                          "launches": launches, "warmup_launches": 10, "warmup_replays": 1,
                          "us_per_launch": round(us, 3),
                          "config": info["config_name"], "grid": info["grid"], "flops": info["flops"],
                          "alg_bytes": info["alg_bytes"]}), flush=True)
    copy_bytes = 256 << 20
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each": copy_bytes, "copies": 5}), flush=True)


FLOOR_FILE = os.path.join(ROOT, "bench_best.json")
FLOOR_FRACTION = 0.97


def floor_check(line, best):
    """Regression floor: each figure named in `best` (the best committed value of
    a key of the JSON line, higher is better) must reach FLOOR_FRACTION of it;
    keys this run did not measure are reported with ok None and not counted.
    Returns {key: {"best", "now", "ratio", "ok"}} and whether all measured are ok."""
    res, ok = {}, True
    for key, ref in sorted(best.items()):
        if key.startswith("_"):
            continue
        now = line.get(key)
        if isinstance(now, dict):
            now = now.get("value")
        if now is None:  # not measured in this run (e.g. --quick)
            res[key] = {"best": ref, "now": None, "ratio": None, "ok": None}
            continue
        ratio = now / ref
        res[key] = {"best": ref, "now": now, "ratio": round(ratio, 4), "ok": ratio >= FLOOR_FRACTION}
        ok &= ratio >= FLOOR_FRACTION
    return res, ok


def grouped_line(r):
    """JSON summary of a list's grouped-head step."""
    g = r["grouped_head"]
    return {"total_us": round(g["ms_per_step"] * 1e3, 2),
            "value": round(r["flops"] / (g["ms_per_step"] * 1e-3) / 1e12, 4),
            "launches": g["launches"], "groups": g["groups"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--quick", action="store_true", help="batch-1 FP32 only")
    ap.add_argument("--only-layer", default=None, help="profile mode: run only this layer of the list (\"all\": each layer in turn)")
    ap.add_argument("--dtype", default="f32", choices=["f32", "int8"], help="profile mode dtype")
    ap.add_argument("--batch", type=int, default=1, help="profile mode batch")
    ap.add_argument("--launches", type=int, default=200, help="profile mode launches")
    ap.add_argument("--config", type=int, default=None, help="profile mode: force this kernel configuration")
    ap.add_argument("--check-floor", action="store_true",
                    help="exit with status 3 when a figure of bench_best.json falls below 97%% of its best")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the batch-16 list shards over images with no "
              "exchange, see the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from convolution_implicit_gemm_02_amd import cbs
    from convolution_implicit_gemm_02_amd import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log("device: %s, %d CUs" % (props.name, props.multi_processor_count))
    if args.only_layer:
        warm_device(torch)  # as before the timed regions below: clocks up before the first timing
        profile_layer(cbs, W, torch, args.only_layer, cbs.CBS_I8 if args.dtype == "int8" else cbs.CBS_F32,
                      args.batch, args.launches, args.config)
        return

    warm_device(torch)
    # written between single launches to flush the L2s and the 256 MB MALL
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    results = {}
    combos = [("f32", cbs.CBS_F32, 1, False)]
    if not args.quick:
        combos += [("int8", cbs.CBS_I8, 1, False), ("int8out", cbs.CBS_I8, 1, True), ("uint8", cbs.CBS_U8, 1, False),
                   ("f32", cbs.CBS_F32, 16, False),
                   ("int8", cbs.CBS_I8, 16, False), ("int8out", cbs.CBS_I8, 16, True)]
    layer_tables = {}
    for name, dt, bs, out_i8 in combos:
        b = ListBench(cbs, W, torch, dt, bs, out_i8=out_i8)
        steps = args.steps if bs == 1 else max(10, args.steps // 8)
        ms_graph, wall_graph = b.time_steps(steps, args.warmup, use_graph=True)
        ms_list, _ = b.time_steps(steps, args.warmup, use_graph=False)
        us_layers, us_eager = b.time_layers()
        us_single, us_flushed = b.time_layers_single(scratch)
        rows = layer_rows(b, us_layers, us_single, us_flushed, us_eager)
        key = "%s_bs%d" % (name, bs)
        layer_tables[key] = rows
        results[key] = {"ms_per_step": ms_graph, "wall_ms_per_step": wall_graph, "ms_per_step_plain_launches": ms_list,
                        "flops": b.flops, "rows": rows, "sum_us_single_launch": round(sum(us_single), 2),
                        "sum_us_flushed": round(sum(us_flushed), 2)}
        if name in ("f32", "int8out") and not args.quick:  # the unchained twins of the chained backbone
            results[key]["us_first25_graph"] = round(b.time_prefix(25, steps, args.warmup) * 1e3, 2)
        chosen = b.group_head()
        ms_grouped = b.time_grouped(steps, args.warmup)
        launches = b.grouped_launches
        results[key]["grouped_head"] = {
            "ms_per_step": ms_grouped, "launches": launches,
            "groups": [{"layers": list(m), "config": c, "us": u, "us_separately": sep, "kept": kept}
                       for m, c, u, sep, kept in chosen]}
        log("%s: list with the head's scales grouped where faster (%d launches) %.1f us (graph); groups %s"
            % (key, launches, ms_grouped * 1e3,
               ", ".join("%s %s %.2f us vs %.2f us separately (%s)" % ("+".join(m), c, u, sep, "kept" if k else "not kept")
                         for m, c, u, sep, k in chosen)))
        log("%s: list %.1f us (graph), %.1f us (plain launches), %.2f T(FL)OP/s, sum of per-layer %.1f us "
            "(single launches %.1f warm, %.1f flushed), roofline sum %.1f us"
            % (key, ms_graph * 1e3, ms_list * 1e3, b.flops / (ms_graph * 1e-3) / 1e12, sum(us_layers), sum(us_single),
               sum(us_flushed), sum(r["roof_us"] for r in rows)))
        for r in rows:
            log("  %-13s %4d->%-4d %4d k%d s%d  %8.2f us (eager %6.2f, single %6.2f, flushed %6.2f)  %7.2f TF/s  "
                "%7.1f GB/s  roof %6.2f us (%s)  frac %.3f  %s"
                % (r["layer"], r["c_in"], r["c_out"], r["h_in"], r["k"], r["s"], r["us"], r["us_eager"],
                   r["us_single"], r["us_flushed"], r["tflops"], r["gbs"], r["roof_us"], r["bound"], r["frac"],
                   r["config"]))
        del b
        torch.cuda.empty_cache()

    # create-time tuning (cbs_layer_autotune) against the compiled-in table, batch 1
    tuned = {}
    for name, dt in ([] if args.quick else [("f32", cbs.CBS_F32), ("int8", cbs.CBS_I8)]):
        b = ListBench(cbs, W, torch, dt, 1)
        t0 = time.perf_counter()
        changed = b.autotune()
        t_tune = time.perf_counter() - t0
        steps = args.steps
        ms_graph, _ = b.time_steps(steps, args.warmup, use_graph=True)
        key = "%s_bs1_autotuned" % name
        tuned[key] = {"value": round(b.flops / (ms_graph * 1e-3) / 1e12, 4),
                      "unit": "TOP/s" if dt == cbs.CBS_I8 else "TFLOP/s", "total_us": round(ms_graph * 1e3, 2),
                      "layers_changed": changed, "tune_seconds": round(t_tune, 2)}
        log("%s: list %.1f us (graph) after create-time tuning (%d of %d layers changed configuration, %.1f s)"
            % (key, ms_graph * 1e3, changed, len(b.layers), t_tune))
        del b
        torch.cuda.empty_cache()

    # the 25 backbone layers chained through channel slices and fused residuals
    chains = {}
    for name, int8, bs in ([] if args.quick else [("f32", False, 1), ("int8", True, 1), ("f32", False, 16),
                                                  ("int8", True, 16)]):
        c = ChainBench(cbs, W, torch, int8, bs)
        steps = args.steps if bs == 1 else max(10, args.steps // 8)
        ms_graph = c.time_steps(steps, args.warmup, use_graph=True)
        ms_plain = c.time_steps(steps, args.warmup, use_graph=False)
        us_steps = c.time_layers()
        lst = results.get("%s_bs%d" % ("int8out" if int8 else "f32", bs))
        indep = round(sum(r["us"] for r in lst["rows"][:25]), 2) if lst else None
        indep_graph = lst.get("us_first25_graph") if lst else None
        key = "chain_%s_bs%d" % (name, bs)
        chains[key] = {"value": round(c.flops / (ms_graph * 1e-3) / 1e12, 4), "unit": "TOP/s" if int8 else "TFLOP/s",
                       "total_us": round(ms_graph * 1e3, 2), "total_us_plain_launches": round(ms_plain * 1e3, 2),
                       "layers": len(c.layers), "sum_us_chained_steps": round(sum(us_steps), 2),
                       "total_us_same_layers_unchained_graph": indep_graph,
                       "sum_us_same_layers_unchained": indep}
        log("%s: 25 chained backbone layers %.1f us (graph), %.1f us (plain), sum of per-step %.1f us; the same "
            "layers unchained: %s us as one graph, sum of per-layer %s us"
            % (key, ms_graph * 1e3, ms_plain * 1e3, sum(us_steps), indep_graph, indep))
        if lst:
            for r, u, st in zip(lst["rows"][:25], us_steps, c.steps):
                log("  %-13s chained %8.2f us (%s)  unchained %8.2f us (%s)"
                    % (r["layer"], u, cbs.cbs_layer_info(st[0])["config_name"], r["us"], r["config"]))
        del c
        torch.cuda.empty_cache()

    head = results["f32_bs1"]
    rows = head["rows"]
    dom = max(rows, key=lambda r: r["us"])
    if dom["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": round(dom["alg_bytes"] / (dom["us"] * 1e-6) / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(dom["flops"] / (dom["us"] * 1e-6) / 1e12, 3),
                "peak": PEAK_FP32 / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom["layer"])
    roof["kernel"] = "conv_igemm %s (%s)" % (dom["layer"], dom["config"])
    roof["layer"] = dom["layer"]
    roof["us_per_launch"] = dom["us"]

    gh = head["grouped_head"]
    line = {"metric": METRIC, "value": round(head["flops"] / (gh["ms_per_step"] * 1e-3) / 1e12, 4),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(gh["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "yolo26n 37-layer fused conv+BN+SiLU list, 640x640 input, batch 1, FP32, "
                                   "one hipGraph replay per step; the detection head's three independent scales "
                                   "run as grouped launches where measured faster (%d launches)" % gh["launches"],
                       "batch": 1, "layers": len(rows), "launches": gh["launches"],
                       "gflop_per_step": round(head["flops"] / 1e9, 4)},
            "total_us": round(gh["ms_per_step"] * 1e3, 2),
            "total_us_one_launch_per_layer": round(head["ms_per_step"] * 1e3, 2),
            "total_us_plain_launches": round(head["ms_per_step_plain_launches"] * 1e3, 2),
            "sum_us_single_launch": head["sum_us_single_launch"], "sum_us_flushed": head["sum_us_flushed"],
            "grouped_head": grouped_line(head),
            "roofline": roof}
    for key, r in results.items():
        if key == "f32_bs1":
            continue
        int8 = key.startswith("int8") or key.startswith("uint8")
        g = r["grouped_head"]["ms_per_step"]
        line[key] = {"value": round(r["flops"] / (g * 1e-3) / 1e12, 4),
                     "unit": "TOP/s" if int8 else "TFLOP/s", "total_us": round(g * 1e3, 2),
                     "total_us_one_launch_per_layer": round(r["ms_per_step"] * 1e3, 2),
                     "total_us_plain_launches": round(r["ms_per_step_plain_launches"] * 1e3, 2),
                     "sum_us_single_launch": r["sum_us_single_launch"], "sum_us_flushed": r["sum_us_flushed"],
                     "grouped_head": grouped_line(r)}
    line.update(tuned)
    line.update(chains)
    floor_ok = True
    if os.path.exists(FLOOR_FILE):
        line["floor"], floor_ok = floor_check(line, json.load(open(FLOOR_FILE)))
        if not floor_ok:
            log("bench floor: below %.0f%% of the committed best: %s" % (100 * FLOOR_FRACTION, line["floor"]))
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(W)
    outdir = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(outdir):
        with open(os.path.join(outdir, "bench_layers.json"), "w") as f:
            json.dump({"device": props.name, "results": results}, f, indent=1)
    print(json.dumps(line), flush=True)
    if args.check_floor and not floor_ok:
        sys.exit(3)


if __name__ == "__main__":
    main()

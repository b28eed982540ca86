"""Offline per-shape tile sweep: time every kernel configuration on every layer
shape of the workloads, on the device, and write the winners to
csrc/tile_table.inc (rebuild libcbs afterwards).

The vision-rs "YOLO26N Inference Optimisation" page ranks per-shape tile
autotuning first among its improvements (section "Improvements", #1): one
fixed tile spans 5 to 556 us across the call sites.  This is that step, done
once per device generation, offline, with the result compiled into the library.

usage: python -m convolution_implicit_gemm_02_amd.tile_sweep [--out PATH] [--json PATH] [--quick]
                                                            [--merge NAME_PREFIX]

--merge times, per shape, only the configuration the current table (or the
cost model) picks and the configurations whose names start with NAME_PREFIX,
and keeps the faster: a way to fold a new kernel family into the table without
re-timing every configuration.  In both modes below a change of configuration
is kept only when the new one beats the current one by 2% in at least two of
three interleaved, longer timings of both.

--classes keeps the fp32 and int8 entries of the current table and sweeps
every configuration for three more table classes per shape: int8 input with
int8 output codes and fp32 with a residual (the general epilogue), and uint8
input with fp32 output.  An entry is written for such a class only where its
best configuration differs from, and beats by 2%, the entry of its input type
the class would fall back to.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

# Table classes (TileEntry::dtype; see table_class in csrc/cbs_host.cpp).
CLS_F32, CLS_I8, CLS_U8, CLS_I8_X, CLS_F32_X = 0, 1, 2, 3, 4
CLASS_NAMES = ["f32", "int8", "uint8", "int8->int8", "f32+res"]

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
DEFAULT_OUT = os.path.join(PKG_DIR, "csrc", "tile_table.inc")

HEADER = """// tile_table.inc -- per-shape kernel configuration chosen by measurement.
// Written by convolution_implicit_gemm_02_amd/tile_sweep.py from a sweep of
// every configuration (split-K 1, and 2-4 for grids below 256 workgroups) on %s;
// shapes not listed fall back to the cost model in cbs_host.cpp.
// Key: (n, c_in, c_out, h, w, k, stride, class) -> (config, splitk); class 0
// fp32, 1 int8 (plain epilogue), 2 uint8 input, 3 int8 input with int8 output,
// 4 fp32 with the general epilogue (a residual).
struct TileEntry {
  int n, c_in, c_out, h, w, k, s, dtype, config, splitk;
};
static const TileEntry kTileTable[] = {
"""


def sweep_shapes(W):
    shapes = []
    for name in ("single", "ragged", "stem", "yolo26n"):
        for spec in W.WORKLOADS[name]():
            for n in ((1, 16) if name in ("yolo26n", "ragged") else (1,)):
                shapes.append((spec, n))
    seen, out = set(), []
    for spec, n in shapes:
        key = (n, spec.c_in, spec.c_out, spec.h, spec.w, spec.k, spec.stride)
        if key not in seen:
            seen.add(key)
            out.append((spec, n))
    return out


def time_layer(cbs, torch, layer, xin, out, min_ms=1.0, reps=3, res=None):
    """Median over `reps` of (event pair around one replay of a captured graph of R
    back-to-back launches) / R, in us: the way a list step launches its kernels
    (an eager launch costs the GPU ~3 us of its own, which would hide the
    differences between configurations of the small layers)."""
    def many(r):
        if res is None:
            return cbs.LayerList([layer] * r, [xin] * r, [out] * r)
        return cbs.StepList([(layer, xin, out, res)] * r)
    many(3).run()
    ten = many(10)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ten.run()
    e1.record()
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / 10, 1e-3)
    r = int(min(1000, max(10, min_ms / per)))
    lst = many(r)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lst.run()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / r * 1e3)
    del g
    return float(np.median(ts))


def other_class_entries(path):
    """Entry lines of classes 2-4 in the table at `path` (a full sweep or a merge
    times classes 0 and 1 only and keeps these as they are)."""
    import re
    keep = []
    if not os.path.exists(path):
        return keep
    for line in open(path):
        m = re.match(r"\s*\{\s*(-?\d+(?:,\s*-?\d+){9})\}", line)
        if m and int(m.group(1).split(",")[0]) != 0 and int(m.group(1).split(",")[7]) in (CLS_U8, CLS_I8_X, CLS_F32_X):
            keep.append(line if line.endswith("\n") else line + "\n")
    return keep


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=DEFAULT_OUT)
    ap.add_argument("--json", default=None)
    ap.add_argument("--quick", action="store_true", help="batch-1 shapes only")
    ap.add_argument("--merge", default=None, metavar="NAME_PREFIX",
                    help="time only the current choice and the configurations named NAME_PREFIX* "
                         "(several prefixes separated by commas)")
    ap.add_argument("--classes", action="store_true",
                    help="keep the fp32/int8 entries; sweep the int8-output and uint8 classes")
    args = ap.parse_args()

    import torch
    from convolution_implicit_gemm_02_amd import cbs
    from convolution_implicit_gemm_02_amd import workloads as W
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    props = torch.cuda.get_device_properties(0)
    name = "%s (%s)" % (props.name, getattr(props, "gcnArchName", "?").split(":")[0])
    rng = np.random.default_rng(0)
    entries, report = [], []
    shapes = sweep_shapes(W)
    if args.quick:
        shapes = [s for s in shapes if s[1] == 1]
    t_start = time.time()
    for si, (spec, n) in enumerate(shapes):
        w = (rng.standard_normal((spec.c_out, spec.c_in, spec.k, spec.k)) / np.sqrt(spec.c_in * spec.k * spec.k)
             ).astype(np.float32)
        ones, zeros = np.ones(spec.c_out, np.float32), np.zeros(spec.c_out, np.float32)
        classes = (CLS_F32, CLS_I8, CLS_I8_X, CLS_U8, CLS_F32_X) if args.classes else (CLS_F32, CLS_I8)
        for cls in classes:
            dtype = {CLS_F32: cbs.CBS_F32, CLS_I8: cbs.CBS_I8, CLS_I8_X: cbs.CBS_I8, CLS_U8: cbs.CBS_U8,
                     CLS_F32_X: cbs.CBS_F32}[cls]
            extra = {}
            if cls == CLS_I8_X:
                extra = dict(out_dtype=cbs.CBS_I8, out_scale=0.05)
            elif cls == CLS_U8:
                extra = dict(in_zero_point=128)
            elif cls == CLS_F32_X:  # a dense residual, as the second conv of a bottleneck adds
                extra = dict(res_c_stride=-(-spec.c_out // 4) * 4)
            desc = cbs.make_desc(n, spec.c_in, spec.h, spec.w, spec.c_out, spec.k, spec.stride, spec.pad, dtype, 0,
                                 0.05, W.BN_EPS, **extra)
            layer = cbs.cbs_create_layer(desc, w, ones, zeros, zeros, ones)
            info = cbs.cbs_layer_info(layer)
            xin = torch.zeros(info["in_bytes"], dtype=torch.int8, device=dev)
            out = torch.empty(max(1, info["out_bytes"] // 4), dtype=torch.float32, device=dev)
            res = torch.zeros(info["res_bytes"], dtype=torch.int8, device=dev) if info["res_bytes"] else None
            tl = lambda **kw: time_layer(cbs, torch, layer, xin, out, res=res, **kw)
            results = []
            candidates = range(cbs.cbs_num_configs())
            current = None
            if args.merge is not None or (args.classes and cls in (CLS_F32, CLS_I8)):
                cur = (info["config"], info["splitk"])
                current = (tl(), cur[0], cur[1])
                results.append(current)
                candidates = [] if args.classes else [c for c in candidates
                                                      if cbs.cbs_config_name(c).startswith(tuple(args.merge.split(",")))]
            elif args.classes:
                # the layer's current choice (its own class entry, else the int8 one) is the one to beat
                current = (tl(), info["config"], info["splitk"])
            for cfg in candidates:
                for sk in (1, 2, 3, 4):
                    if sk > 1 and info["grid"] >= 256:
                        continue
                    try:
                        cbs.cbs_layer_set_config(layer, cfg, sk)
                    except cbs.CbsError:
                        continue
                    results.append((tl(), cfg, sk))
            results.sort()
            best_us, best_cfg, best_sk = results[0]
            if current is not None and best_us > 0.98 * current[0]:
                best_us, best_cfg, best_sk = current  # within noise of the current choice: keep it
            elif current is not None and (best_cfg, best_sk) != current[1:]:
                # a change: confirm it with longer, interleaved timings of both
                # choices (one short run can be off by several percent)
                wins, t_new = 0, []
                for _ in range(3):
                    cbs.cbs_layer_set_config(layer, best_cfg, best_sk)
                    tn = tl(min_ms=3.0, reps=5)
                    cbs.cbs_layer_set_config(layer, current[1], current[2])
                    tc = tl(min_ms=3.0, reps=5)
                    wins += tn < 0.98 * tc
                    t_new.append(tn)
                if wins < 2:
                    best_us, best_cfg, best_sk = current
                else:
                    best_us = float(np.median(t_new))
            if cls == CLS_I8:
                i8_choice = (best_cfg, best_sk)
            if cls == CLS_F32:
                f32_choice = (best_cfg, best_sk)
            # classes 2 and 3 fall back to the int8 entry, class 4 to the fp32 one: write them only
            # where they differ from it
            if cls in (CLS_F32, CLS_I8) or (best_cfg, best_sk) != (f32_choice if cls == CLS_F32_X else i8_choice):
                entries.append((n, spec.c_in, spec.c_out, spec.h, spec.w, spec.k, spec.stride, cls, best_cfg, best_sk,
                                best_us, spec.name))
            report.append({"layer": spec.name, "n": n, "dtype": CLASS_NAMES[cls],
                           "best_us": best_us, "config": cbs.cbs_config_name(best_cfg), "splitk": best_sk,
                           "all": [(round(t, 3), cbs.cbs_config_name(c), s) for t, c, s in results[:6]]})
            del layer, xin, out, res
        print("[%3d/%d] %-14s n=%-2d %s  (%.0f s)" % (
            si + 1, len(shapes), spec.name, n, " | ".join("%s %s/%d %.2f us" % (r["dtype"], r["config"], r["splitk"],
                                                                                r["best_us"])
                                                           for r in report[-len(classes):]),
            time.time() - t_start), flush=True)

    kept = [] if args.classes else other_class_entries(DEFAULT_OUT)
    with open(args.out, "w") as f:
        f.write(HEADER % name)
        for e in entries:
            f.write("    {%d, %d, %d, %d, %d, %d, %d, %d, %d, %d},  // %s %s %.2f us\n" % (
                e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7], e[8], e[9], e[11], CLASS_NAMES[e[7]], e[10]))
        for line in kept:  # classes this mode does not sweep: the current table's entries, unchanged
            f.write(line)
        f.write("    {0, 0, 0, 0, 0, 0, 0, 0, 0, 1},  // sentinel: n == 0 never matches\n};\n")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(report, f, indent=1)
    print("wrote %s (%d entries)" % (args.out, len(entries)), flush=True)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(PKG_DIR))
    main()

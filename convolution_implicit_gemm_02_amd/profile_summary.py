"""Summaries of rocprofv3 runs of bench.py's profile mode, written to profiles/.

Two kinds, each from runs whose commands the summary itself records:

  python -m convolution_implicit_gemm_02_amd.profile_summary dominant OUT_DIR
      for each layer L of DOMINANT_LAYERS (the batch-1 FP32 layers whose
      per-launch times tie at the top of the list): OUT_DIR/prof_dom_L
      (--kernel-trace --stats, with the program's output in prof_dom_L.log),
      OUT_DIR/pmc_fetch_L and OUT_DIR/pmc_write_L (--pmc FETCH_SIZE,
      --pmc WRITE_SIZE) of `bench.py --only-layer L`, plus OUT_DIR/bench.log
      and bench_layers.json (a default bench run of the same tree):
      profiles/conv_igemm_L_f32_bs1.md and profiles/traffic_dominant.json
      (per-layer traffic that bench.py reports while the kernel sources hash
      to the profiled ones).

  python -m convolution_implicit_gemm_02_amd.profile_summary layers OUT_DIR DTYPE BATCH
      OUT_DIR/lp_<dtype>_bs<batch>/{trace,mfma,fetch,write} of
      `bench.py --only-layer all` and its log OUT_DIR/lp_<dtype>_bs<batch>.trace.log:
      profiles/list_layers_<dtype>_bs<batch>.md.

Byte counters are scaled by what they read for the 256 MiB device copies the
profile mode ends with (on this device FETCH_SIZE reads about half the bytes a
copy moves and WRITE_SIZE all of them).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_KIB = 262144.0


def _rows(path):
    return list(csv.DictReader(open(glob.glob(path)[0])))


def _copy_factor(rows, counter):
    v = [float(r["Counter_Value"]) for r in rows
         if r["Kernel_Name"] == "__amd_rocclr_copyBuffer" and r["Counter_Name"] == counter
         and float(r["Counter_Value"]) > 100000]
    return COPY_KIB / (sum(v) / len(v)), sum(v) / len(v)


DOMINANT_LAYERS = ("neck256.3x3", "neck64.3x3", "head64.3x3")


def _source_hash():
    sys.path.insert(0, ROOT)
    import bench
    h = hashlib.sha256()
    for f in bench.KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def _dominant_one(out_dir, layer, bench_line):
    sub = lambda kind: os.path.join(out_dir, "%s_%s" % (kind, layer))
    stats = _rows(os.path.join(sub("prof_dom"), "*kernel_stats.csv"))
    kern = [s for s in stats if s["Name"].startswith("void cbs::conv")][0]
    kname = kern["Name"]
    trace = sorted((r for r in _rows(os.path.join(sub("prof_dom"), "*kernel_trace.csv")) if r["Kernel_Name"] == kname),
                   key=lambda r: int(r["Dispatch_Id"]))
    timed = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace[-200:]]
    timed_avg = sum(timed) / len(timed)
    fr = _rows(os.path.join(sub("pmc_fetch"), "*counter_collection.csv"))
    wr = _rows(os.path.join(sub("pmc_write"), "*counter_collection.csv"))
    info = [json.loads(line) for line in open(sub("prof_dom") + ".log") if line.startswith('{"layer"')][0]
    noprof = None  # the same program without the profiler (OUT_DIR/noprof_L.log), if it was run
    npath = os.path.join(out_dir, "noprof_%s.log" % layer)
    if os.path.exists(npath):
        noprof = [json.loads(line) for line in open(npath) if line.startswith('{"layer"')][0]["us_per_launch"]

    def avg(rows):
        v = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] == kname]
        return sum(v) / len(v)

    fk, wk = avg(fr), avg(wr)
    ff, fcopy = _copy_factor(fr, "FETCH_SIZE")
    wf, wcopy = _copy_factor(wr, "WRITE_SIZE")
    traffic = int(round((fk * ff + wk * wf) * 1024))
    alg = int(info["alg_bytes"])
    rec = {"kernel": kname, "config": info["config"], "grid": info["grid"], "fetch_kib": fk, "write_kib": wk,
           "fetch_factor": ff, "write_factor": wf, "traffic_bytes": traffic, "alg_bytes": alg,
           "rocprof_avg_ns": float(kern["AverageNs"]), "rocprof_timed_replay_avg_us": round(timed_avg, 3),
           "graph_us_per_launch": info["us_per_launch"],
           "graph_us_per_launch_without_profiler": noprof,
           "summary": "profiles/conv_igemm_%s_f32_bs1.md" % layer}
    tbl = "\n".join("| `%s` | %s | %.1f | %s | %s |" % (s["Name"][:90], s["Calls"], float(s["AverageNs"]), s["MinNs"],
                                                         s["MaxNs"]) for s in stats)
    bench_row = None
    if bench_line is not None:
        bench_row = [r for r in bench_line.get("_rows", []) if r["layer"] == layer]
    ev = ("`bench.py` (default run of the same tree) reports %.3f us per launch for this layer in the "
          "list's per-layer table" % bench_row[0]["us"]) if bench_row else ""
    dom_note = ""
    if bench_line is not None:
        roof = bench_line["roofline"]
        dom_note = ("In that run the dominant layer was %s (%.3f us per launch)." %
                    (roof["layer"], roof["us_per_launch"]))
    nop = ("The same program without the profiler (`python bench.py --only-layer %s --launches 200`, same call): "
           "%.3f us per launch, so the profiler slows these launches by %.0f%%. " % (layer, noprof,
                                                                                     100 * (info["us_per_launch"] / noprof - 1))
           if noprof else "")
    md = f"""# rocprofv3 summary: {kname}, layer {layer} (batch 1, FP32)

One of the three layers of the batch-1 FP32 YOLO26n list step whose per-launch times lie within a few
tenths of a microsecond of each other at the top of the list (neck256.3x3, neck64.3x3, head64.3x3);
`bench.py` reports the one that measures largest in its run as the dominant kernel. {dom_note}

## Kernel trace (`--kernel-trace --stats`)

Command (from the repository root on the GPU box):

```
rocprofv3 --kernel-trace --stats --output-format csv -d $PWD/gpurun_out/prof_dom_{layer} -o dom -- python bench.py --only-layer {layer} --launches 200
```

The program launches the layer 10 times eagerly, then captures 200 launches as one graph and
replays it twice (an untimed warm-up replay, then the timed one, the way the list step runs its kernels
and bench.py times them), then five 256 MiB device copies.

| Kernel | Calls | Average ns | Min ns | Max ns |
|---|---|---|---|---|
{tbl}

Kernel duration in the trace, averaged over the 200 dispatches of the timed replay: {timed_avg:.3f} us
(the table above averages all 410 dispatches). Event timing of the timed replay inside the profiled
program: {info['us_per_launch']:.3f} us per launch. {nop}{ev}.

## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, separate runs)

```
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $PWD/gpurun_out/pmc_fetch_{layer} -o fetch -- python bench.py --only-layer {layer} --launches 20
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $PWD/gpurun_out/pmc_write_{layer} -o write -- python bench.py --only-layer {layer} --launches 20
```

Reference: the same runs end with device copies of 256 MiB (`__amd_rocclr_copyBuffer`); their counters read
FETCH_SIZE = {fcopy:.0f} KiB and WRITE_SIZE = {wcopy:.0f} KiB per copy against 262144 KiB moved, so the scale
factors are {ff:.3f} (fetch) and {wf:.3f} (write).

| Kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled bytes/dispatch |
|---|---|---|---|
| `{kname}` | {fk:.2f} | {wk:.2f} | {traffic} |

Algorithmic bytes per launch: {alg:,} (input + weights + output + folded bias and scale, each once).
The counted L2-miss traffic is {traffic / alg:.2f}x that; misses may be served by the 256 MB MALL
rather than HBM, and every XCD's L2 fetches its own copy of what its workgroups read.

Summarised by `python -m convolution_implicit_gemm_02_amd.profile_summary dominant gpurun_out`.
"""
    with open(os.path.join(ROOT, "profiles", "conv_igemm_%s_f32_bs1.md" % layer), "w") as f:
        f.write(md)
    return rec


def dominant(out_dir, layers=DOMINANT_LAYERS):
    """Per-layer traffic of the candidates for the dominant kernel, from
    OUT_DIR/{prof_dom,pmc_fetch,pmc_write}_<layer>, and OUT_DIR/bench.log."""
    bench_line = None
    blog = os.path.join(out_dir, "bench.log")
    if os.path.exists(blog):
        bench_line = json.loads(open(blog).read().strip().split("\n")[-1])
        bl = os.path.join(out_dir, "bench_layers.json")
        if os.path.exists(bl):
            bench_line["_rows"] = json.load(open(bl))["results"]["f32_bs1"]["rows"]
    rec = {"dtype": "f32", "batch": 1, "source_sha256": _source_hash(),
           "layers": {layer: _dominant_one(out_dir, layer, bench_line) for layer in layers}}
    with open(os.path.join(ROOT, "profiles", "traffic_dominant.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def layers(out_dir, dtype, batch):
    base = os.path.join(out_dir, "lp_%s_bs%d" % (dtype, batch))
    i8 = dtype == "int8"
    info = [json.loads(line) for line in open(base + ".trace.log") if line.startswith('{"layer"')]

    def conv_rows(sub):
        rs = [r for r in _rows(os.path.join(base, sub, "*%s.csv" % ("kernel_trace" if sub == "trace"
                                                                     else "counter_collection")))
              if r["Kernel_Name"].startswith("void cbs::conv")]
        rs.sort(key=lambda r: int(r["Dispatch_Id"]))
        return rs

    def per_layer(rs, launches, key):
        # per layer: 10 eager warm-up launches, a warm-up replay and the timed replay
        per = 10 + 2 * launches
        assert len(rs) == per * len(info), (len(rs), per, len(info))
        return [[key(r) for r in rs[(i + 1) * per - launches:(i + 1) * per]] for i in range(len(info))]

    tr = per_layer(conv_rows("trace"), 20, lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def pmc(sub, counter):
        rs = [r for r in conv_rows(sub) if r["Counter_Name"] == counter]
        return per_layer(rs, 10, lambda r: float(r["Counter_Value"]))

    mf = pmc("mfma", "SQ_VALU_MFMA_BUSY_CYCLES")
    fe, wr = pmc("fetch", "FETCH_SIZE"), pmc("write", "WRITE_SIZE")
    ff, _ = _copy_factor(_rows(os.path.join(base, "fetch", "*counter_collection.csv")), "FETCH_SIZE")
    wf, _ = _copy_factor(_rows(os.path.join(base, "write", "*counter_collection.csv")), "WRITE_SIZE")
    peak = 5.0e15 if i8 else 157.3e12
    cyc_per_flop = 16.0 / 32768 if i8 else 32.0 / 2048
    avg = lambda v: sum(v) / len(v)
    lines, tsum, rsum = [], 0.0, 0.0
    for i, L in enumerate(info):
        us, busy = avg(tr[i]), avg(mf[i])
        fmb, wmb = avg(fe[i]) * 1024 * ff / 1e6, avg(wr[i]) * 1024 * wf / 1e6
        t_c, t_m = L["flops"] / peak * 1e6, L["alg_bytes"] / 8e12 * 1e6
        roof = max(t_c, t_m)
        tsum += us
        rsum += roof
        lines.append("| %d | %s | %s | %d | %.2f | %.2f | %.1f%% | %.2f | %.2f | %.2f | %.0f | %s | %.2f |" % (
            i + 1, L["layer"], L["config"], L["grid"], us, busy / (L["flops"] * cyc_per_flop),
            100 * busy / (us * 2400 * 1024), fmb, wmb, L["alg_bytes"] / 1e6, (fmb + wmb) / us * 1e3,
            "mfma" if t_c > t_m else "hbm", roof / us))
    title = "INT8 (fp32 output)" if i8 else "FP32"
    pk = "5.0 POP/s INT8" if i8 else "157.3 TFLOP/s FP32"
    mfma_note = "16 busy cycles per 32768-FLOP MFMA" if i8 else "32 busy cycles per 2048-FLOP MFMA"
    D, B = dtype, batch
    md = f"""# rocprofv3 per-layer summary: YOLO26n-shaped list, {title}, batch {B}

Every layer of the 37-layer list, in list order, each launched 10 times to warm up and then repeatedly back to back as a captured graph, replayed once untimed and once timed (`bench.py --only-layer all`). Four runs of the same program, from the repository root on the GPU box:

```
rocprofv3 --kernel-trace --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/trace -o t -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 20
rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/mfma -o m -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 10
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/fetch -o f -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 10
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/write -o w -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 10
```

The second run also collected `SQ_BUSY_CU_CYCLES` and `GRBM_GUI_ACTIVE`; the table does not use them.

Columns:
- `us`: mean kernel duration over the timed replay of 20 launches in the kernel-trace run (after 10 eager launches and a warm-up replay);
- `MFMA busy / alg.`: `SQ_VALU_MFMA_BUSY_CYCLES` over the cycles the layer's algorithmic FLOPs need ({mfma_note}); above 1 means padded work;
- `MFMA util`: the busy cycles over `us` x 2.4 GHz x 1024 SIMDs;
- `fetch MB`, `write MB`: `FETCH_SIZE` and `WRITE_SIZE` per dispatch, scaled by what they read for a 256 MiB device copy in the same runs (factors {ff:.3f} and {wf:.3f}); these count L2 misses, which the 256 MB MALL may serve;
- `alg MB`: the layer's algorithmic bytes; `GB/s`: (fetch + write) / `us`;
- `frac`: roofline time max(FLOPs / peak, alg bytes / 8 TB/s) over `us` (peak {pk}).

| # | layer | config | grid | us | MFMA busy / alg. | MFMA util | fetch MB | write MB | alg MB | GB/s | bound | frac |
|---|---|---|---|---|---|---|---|---|---|---|---|---|
""" + "\n".join(lines) + f"""

Sum of kernel durations: {tsum:.1f} us; sum of rooflines: {rsum:.1f} us.

Summarised by `python -m convolution_implicit_gemm_02_amd.profile_summary layers gpurun_out {D} {B}`.
"""
    with open(os.path.join(ROOT, "profiles", "list_layers_%s_bs%d.md" % (D, B)), "w") as f:
        f.write(md)
    return tsum, rsum


def main():
    if len(sys.argv) >= 3 and sys.argv[1] == "dominant":
        print(dominant(sys.argv[2]))
    elif len(sys.argv) == 5 and sys.argv[1] == "layers":
        print(layers(sys.argv[2], sys.argv[3], int(sys.argv[4])))
    else:
        print(__doc__)
        sys.exit(2)


if __name__ == "__main__":
    main()

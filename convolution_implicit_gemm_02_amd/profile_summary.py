"""Summaries of rocprofv3 runs of bench.py's profile mode, written to profiles/.

Two kinds, each from runs whose commands the summary itself records:

  python -m convolution_implicit_gemm_02_amd.profile_summary dominant OUT_DIR
      OUT_DIR/prof_dom (--kernel-trace --stats), OUT_DIR/pmc_fetch and
      OUT_DIR/pmc_write (--pmc FETCH_SIZE, --pmc WRITE_SIZE) of
      `bench.py --only-layer neck256.3x3`, plus OUT_DIR/bench.log (a default
      bench run of the same tree): profiles/conv_igemm_<layer>_f32_bs1.md and
      profiles/traffic_dominant.json (the traffic figure bench.py reports while
      the kernel sources hash to the profiled ones).

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


def dominant(out_dir, layer="neck256.3x3"):
    sys.path.insert(0, ROOT)
    import bench
    stats = _rows(os.path.join(out_dir, "prof_dom", "*kernel_stats.csv"))
    kern = [s for s in stats if s["Name"].startswith("void cbs::conv")][0]
    kname = kern["Name"]
    fr = _rows(os.path.join(out_dir, "pmc_fetch", "*counter_collection.csv"))
    wr = _rows(os.path.join(out_dir, "pmc_write", "*counter_collection.csv"))

    def avg(rows):
        v = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] == kname]
        return sum(v) / len(v)

    fk, wk = avg(fr), avg(wr)
    ff, fcopy = _copy_factor(fr, "FETCH_SIZE")
    wf, wcopy = _copy_factor(wr, "WRITE_SIZE")
    traffic = int(round((fk * ff + wk * wf) * 1024))
    h = hashlib.sha256()
    for f in bench.KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    line = json.loads(open(os.path.join(out_dir, "bench.log")).read().strip().split("\n")[-1])
    ev = line["roofline"]["us_per_launch"]
    rec = {"layer": layer, "dtype": "f32", "batch": 1, "kernel": kname, "source_sha256": h.hexdigest(),
           "fetch_kib": fk, "write_kib": wk, "fetch_factor": ff, "write_factor": wf, "traffic_bytes": traffic,
           "rocprof_avg_ns": float(kern["AverageNs"]), "summary": "profiles/conv_igemm_%s_f32_bs1.md" % layer}
    with open(os.path.join(ROOT, "profiles", "traffic_dominant.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    tbl = "\n".join("| `%s` | %s | %.1f | %s | %s |" % (s["Name"][:90], s["Calls"], float(s["AverageNs"]), s["MinNs"],
                                                         s["MaxNs"]) for s in stats)
    md = f"""# rocprofv3 summary: {kname}, layer {layer} (batch 1, FP32)

Dominant kernel of the batch-1 FP32 YOLO26n list step (largest per-launch time in `bench.py`).

## Kernel trace (`--kernel-trace --stats`)

Command (from the repository root on the GPU box):

```
rocprofv3 --kernel-trace --stats --output-format csv -d $PWD/gpurun_out/prof_dom -o dom -- python bench.py --only-layer {layer} --launches 200
```

| Kernel | Calls | Average ns | Min ns | Max ns |
|---|---|---|---|---|
{tbl}

`bench.py` event timing in the default run of the same tree: {ev:.3f} us per launch (rocprofv3 average {float(kern['AverageNs']) / 1000:.3f} us).

## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, separate runs)

```
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $PWD/gpurun_out/pmc_fetch -o fetch -- python bench.py --only-layer {layer} --launches 20
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $PWD/gpurun_out/pmc_write -o write -- python bench.py --only-layer {layer} --launches 20
```

Reference: the same runs end with device copies of 256 MiB (`__amd_rocclr_copyBuffer`); their counters read FETCH_SIZE = {fcopy:.0f} KiB and WRITE_SIZE = {wcopy:.0f} KiB per copy against 262144 KiB moved, so the scale factors are {ff:.3f} (fetch) and {wf:.3f} (write).

| Kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled bytes/dispatch |
|---|---|---|---|
| `{kname}` | {fk:.2f} | {wk:.2f} | {traffic} |

Algorithmic bytes per launch: 3,180,544 (input 409,600 + weights 2,359,296 + output 409,600 + folded bias and scale 2,048). The L2-miss traffic is {traffic / 3180544:.2f}x that: each of the eight XCDs fetches the whole input and its share of the weights.

Summarised by `python -m convolution_implicit_gemm_02_amd.profile_summary dominant gpurun_out`.
"""
    with open(os.path.join(ROOT, "profiles", "conv_igemm_%s_f32_bs1.md" % layer), "w") as f:
        f.write(md)
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
        per = 10 + launches
        assert len(rs) == per * len(info), (len(rs), per, len(info))
        return [[key(r) for r in rs[i * per + 10:(i + 1) * per]] for i in range(len(info))]

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

Every layer of the 37-layer list, in list order, each launched 10 times to warm up and then repeatedly back to back (`bench.py --only-layer all`). Four runs of the same program, from the repository root on the GPU box:

```
rocprofv3 --kernel-trace --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/trace -o t -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 20
rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/mfma -o m -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 10
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/fetch -o f -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 10
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $PWD/gpurun_out/lp_{D}_bs{B}/write -o w -- python bench.py --only-layer all --dtype {D} --batch {B} --launches 10
```

The second run also collected `SQ_BUSY_CU_CYCLES` and `GRBM_GUI_ACTIVE`; the table does not use them.

Columns:
- `us`: mean kernel duration over the last 20 launches of the kernel-trace run;
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

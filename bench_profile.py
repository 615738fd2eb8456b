"""Turn rocprofv3 outputs of bench.py runs into the short summaries kept under profiles/.

  python bench_profile.py trace   <kernel_trace.csv> <out.txt> "<command>"
  python bench_profile.py traffic <fetch_counter_collection.csv> <write_counter_collection.csv>
                                  <copy_bytes> <config> <out.json> "<command>"
  python bench_profile.py mfma    <counter_collection.csv> <out.json> "<command>"

`traffic` scales the per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each csa kernel by what the same
counters read for the plain device copy of `copy_bytes` bytes that bench.py --calibrate-copy runs
(each copy reads and writes copy_bytes), and records the indexer kernel source hash so bench.py can
tell whether the figure still describes the current kernel.

`mfma` averages every counter of each csa kernel over its dispatches and derives matrix-core use:
GRBM_GUI_ACTIVE sums the eight XCDs' busy cycles, SQ_VALU_MFMA_BUSY_CYCLES the busy cycles of all
1,024 SIMDs, so busy / (1024 * GRBM_GUI_ACTIVE / 8) is the share of SIMD time the matrix cores
worked; SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 is the bf16 FLOP count of the dispatch.
"""
import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def _short(name):
    return name.split("(")[0].replace("void ", "").strip()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("indexer.hip", "indexer_score.h", "csa_device.h"):
        h.update(open(os.path.join(ROOT, "long_context_sparse_csa_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def trace(path, out, cmd):
    rows = list(csv.DictReader(open(path)))
    st = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        n = _short(r["Kernel_Name"])
        st.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"command: {cmd}", "", f"{'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for n, v in st.items():
        s = sorted(v)
        lines.append(f"{n[:58]:58s} {len(v):6d} {sum(v)/len(v):9.2f} {s[len(s)//2]:9.2f} {s[0]:9.2f} {s[-1]:9.2f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(path, counter):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def _last_copies(path, counter, n=3):
    rows = [r for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    vals = [float(r["Counter_Value"]) for r in rows[-n:]]
    return sum(vals) / len(vals)


def traffic(fetch_csv, write_csv, copy_bytes, config, out, cmd):
    copy_bytes = int(copy_bytes)
    f = _counter(fetch_csv, "FETCH_SIZE")
    w = _counter(write_csv, "WRITE_SIZE")
    # the calibration copies are the last three copy dispatches of the run (bench.py issues them after
    # all timed work; the workload's own input copies, some larger, come before)
    fc = _last_copies(fetch_csv, "FETCH_SIZE")
    wc = _last_copies(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (fc * 1024.0)
    w_scale = copy_bytes / (wc * 1024.0)
    res = {"command": cmd, "config": config, "copy_bytes": copy_bytes,
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
    for k in f:
        if "csa::" not in k:
            continue
        fb = sum(f[k]) / len(f[k]) * 1024.0 * f_scale
        wb = sum(w.get(k, [0.0])) / max(1, len(w.get(k, []))) * 1024.0 * w_scale
        res["kernels"][k] = {"fetch_bytes": int(fb), "write_bytes": int(wb), "dispatches": len(f[k])}
    # the decode indexer the fused step runs (the roofline kernel of the decode workloads)
    idx = [k for k in res["kernels"] if ("indexer_fp8" in k or "indexer_fp4" in k) and "prefill" not in k]
    if idx:
        k = idx[-1]
        res["bytes_per_launch"] = res["kernels"][k]["fetch_bytes"] + res["kernels"][k]["write_bytes"]
        res["kernel"] = k
    res["kernel_source_sha256_16"] = kernel_source_hash()
    open(out, "w").write(json.dumps(res, indent=1) + "\n")
    print(json.dumps(res, indent=1))


def mfma(csv_path, out, cmd, xcds=8, simds=1024):
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        k = _short(r["Kernel_Name"])
        if "csa::" in k:
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    res = {"command": cmd, "kernels": {}}
    for k, d in vals.items():
        avg = {c: sum(v) / len(v) for c, v in d.items()}
        e = {"dispatches": max(len(v) for v in d.values()),
             "counters": {c: int(round(v)) for c, v in avg.items()}}
        if "GRBM_GUI_ACTIVE" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg["GRBM_GUI_ACTIVE"] > 0:
            e["mfma_busy_frac"] = round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * avg["GRBM_GUI_ACTIVE"] / xcds), 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
            e["bf16_gflop"] = round(avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9, 2)
        if "SQ_INSTS_VALU" in avg and avg.get("SQ_INSTS_MFMA"):
            e["valu_per_mfma"] = round(avg["SQ_INSTS_VALU"] / avg["SQ_INSTS_MFMA"], 2)
        res["kernels"][k] = e
    open(out, "w").write(json.dumps(res, indent=1) + "\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:8])
    elif sys.argv[1] == "mfma":
        mfma(*sys.argv[2:5])
    else:
        sys.exit(__doc__)

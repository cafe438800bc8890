"""Summary of a rocprofv3 --pmc run of bench.py --no-graph with SQ_INSTS_VALU_MFMA_MOPS_BF16 and
SQ_INSTS_VALU_MFMA_MOPS_F32 (among others): per Q4_1 GEMM class of the verify passes (classed by
their place in each layer: q|k|v, o, gate|up, down), the MFMA work each launch executes (512 flops
per MOPS unit, as rocprofv3's MfmaFlops metric counts it), the rate over the dispatches' own
durations, and that rate as a fraction of MI355X's dense bf16 MFMA peak (2.5 PFLOP/s).

usage: python summarize_mfma_util.py <rocprofv3 output dir>"""
import collections
import csv
import glob
import sys

PEAK_BF16 = 2.5e15
d = sys.argv[1]
f = glob.glob(f"{d}/**/*counter_collection.csv", recursive=True)[0]
by = collections.OrderedDict()
for r in sorted(csv.DictReader(open(f)), key=lambda r: int(r["Dispatch_Id"])):
    e = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
    e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
seq = list(by.values())
# the GEMMs of a layer: q|k|v (store epilogue, followed by attention), o (residual, before
# gate|up), gate|up (SwiGLU epilogue), down (residual, right after gate|up)
cls = collections.defaultdict(list)
for i, e in enumerate(seq):
    n = e["name"]
    if "k_gemm<0, 2," in n:
        cls["gate|up"].append(e)
        if i + 1 < len(seq) and "k_gemm<0, 1," in seq[i + 1]["name"]:
            cls["down"].append(seq[i + 1])
        if i >= 1 and "k_gemm<0, 1," in seq[i - 1]["name"]:
            cls["o"].append(seq[i - 1])
    elif "k_gemm<0, 0," in n and i + 1 < len(seq) and "k_attention" in seq[i + 1]["name"]:
        cls["q|k|v"].append(e)
print(f"{'class':8s} {'dispatches':>10s} {'MFMA GFLOP/launch':>18s} {'TFLOP/s':>9s} {'% of bf16 peak':>15s}")
for c in ("q|k|v", "o", "gate|up", "down"):
    v = cls[c]
    if not v:
        continue
    fl = sum((e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + e["SQ_INSTS_VALU_MFMA_MOPS_F32"]) * 512 for e in v)
    ns = sum(e["ns"] for e in v)
    print(f"{c:8s} {len(v):10d} {fl / len(v) / 1e9:18.3f} {fl / ns / 1e3:9.1f} {100 * fl / (ns * 1e-9) / PEAK_BF16:15.2f}")

"""Summaries of rocprofv3 runs of bench.py, as committed under profiles/ (measurement tooling; the
library never imports this file).

usage (from the repository root):
  python profile_summaries.py kernel-trace <rocprofv3 output dir> [kernels per pass, default 256]
  python profile_summaries.py pmc-traffic <fetch dir> <write dir> <probe MiB> <q|k|v bytes> <o bytes> <gate|up bytes> <down bytes>
  python profile_summaries.py mfma <rocprofv3 output dir>
  python profile_summaries.py attn-traffic <fetch dir> <write dir> <probe MiB> <one-chunk K/V bytes> <two-stage K/V bytes>

kernel-trace: the per-kernel statistics of a --kernel-trace --stats csv run, then the median of the
  first 7 verify passes (embed ... accept) with every kernel labelled by its place in the layer (the
  statistics alone where the run holds no verify pass, as a prefill run does).
pmc-traffic: two --pmc runs (FETCH_SIZE, then WRITE_SIZE) of bench.py --no-graph --copy-probe-mib N;
  each counter is scaled by what it reads for the copy probe (torch neg over N MiB: N MiB read, N MiB
  written); the Q4_1 GEMM dispatches of the verify passes are classed by their place in each layer
  (the byte arguments: each class's algorithmic bytes per launch, bench.py's gemm_alg_bytes), and
  the whole Q4_1 stream of a pass (one launch of each class per layer) is summed from the classes.
attn-traffic: two --pmc runs (FETCH_SIZE, then WRITE_SIZE) of bench.py --no-graph --copy-probe-mib N
  restricted to the attention kernels and the copy probe; each counter scaled by the copy probe as in
  pmc-traffic; per attention form (one sub-chunk per workgroup, two-stage) and for the combine, the
  bytes per dispatch against the K/V bytes a launch of that form reads (the byte arguments: rows read
  x 2 x KV width x element size, one layer of each form at the run's context).
mfma: a --pmc run with SQ_INSTS_VALU_MFMA_MOPS_BF16 and SQ_INSTS_VALU_MFMA_MOPS_F32 (of bench.py, or
  of bench.py --prefill N for the 64-row chunks): per Q4_1 GEMM class, the MFMA work per launch (512 flops per MOPS unit, as rocprofv3's MfmaFlops metric counts
  it), its rate over the dispatches' durations and the fraction of the 2.5 PFLOP/s dense bf16 peak.
"""
import collections
import csv
import glob
import hashlib
import sys


def kernel_trace(ARGV):
    d = ARGV[1]
    stats = glob.glob(f"{d}/**/*kernel_stats.csv", recursive=True)
    trace = glob.glob(f"{d}/**/*kernel_trace.csv", recursive=True)
    rows = list(csv.DictReader(open(stats[0])))
    def short(n):
        n = n.replace('void ', '')
        for pre in ('bvf::(anonymous namespace)::', 'bvf::'):
            n = n.replace(pre, '')
        i = n.find('(')
        return n[:i] if i > 0 else n
    print(f"{'kernel':48s} {'calls':>7s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'share %':>8s}")
    for r in rows:
        print(f"{short(r['Name'])[:48]:48s} {int(r['Calls']):7d} {float(r['AverageNs'])/1e3:9.2f} {float(r['MinNs'])/1e3:9.2f} {float(r['MaxNs'])/1e3:9.2f} {float(r['Percentage']):8.2f}")
    tr = list(csv.DictReader(open(trace[0])))
    tr.sort(key=lambda r: int(r['Start_Timestamp']))
    names = [r['Kernel_Name'] for r in tr]
    # last pass: from the last k_embed that is followed by a k_accept before the next k_embed
    emb = [i for i, n in enumerate(names) if 'k_embed' in n]
    passes = []
    for j, i in enumerate(emb):
        end = emb[j + 1] if j + 1 < len(emb) else len(names)
        acc = [q for q in range(i, end) if 'k_accept' in names[q]]
        if acc:
            passes.append((i, acc[0]))
    want = int(ARGV[2]) if len(ARGV) > 2 else 256
    cands = [p for p in passes if p[1] - p[0] + 1 == want][:7]
    if not cands:
        print(f"\nno verify pass of {want} kernels in this trace (a prefill run has none)")
        return
    dur = lambda p: int(tr[p[1]]['End_Timestamp']) - int(tr[p[0]]['Start_Timestamp'])
    i0, i1 = sorted(cands, key=dur)[len(cands) // 2]   # the median of the k = 8 graph passes
    seg = tr[i0:i1 + 1]
    t = (int(seg[-1]['End_Timestamp']) - int(seg[0]['Start_Timestamp'])) / 1e3
    busy = sum(int(r['End_Timestamp']) - int(r['Start_Timestamp']) for r in seg) / 1e3
    print(f"\none pass from the trace: {t:.1f} us, {len(seg)} kernels, gaps between kernels {t - busy:.1f} us in total")
    agg = collections.OrderedDict()
    roles = ['q|k|v GEMM', 'attention', 'attention combine', 'o GEMM', 'gate|up GEMM', 'down GEMM']
    for idx, r in enumerate(seg):
        k = short(r['Kernel_Name'])
        if 1 <= idx <= 6 * 42:
            k = f"{k} ({roles[(idx - 1) % 6]})"
        agg.setdefault(k, []).append((int(r['End_Timestamp']) - int(r['Start_Timestamp'])) / 1e3)
    print(f"{'kernel':52s} {'n':>4s} {'total us':>9s} {'mean us':>8s}")
    for k, v in agg.items():
        print(f"{k[:52]:52s} {len(v):4d} {sum(v):9.1f} {sum(v)/len(v):8.2f}")


def pmc_traffic(ARGV):
    fetch_dir, write_dir, probe_mib = ARGV[1], ARGV[2], int(ARGV[3])
    # algorithmic bytes per launch (class average)
    alg = {"qkv": float(ARGV[4]), "o": float(ARGV[5]), "gate_up": float(ARGV[6]), "down": float(ARGV[7])}
    def load(d, counter):
        f = glob.glob(f"{d}/**/*counter_collection.csv", recursive=True)[0]
        rows = [r for r in csv.DictReader(open(f)) if r['Counter_Name'] == counter]
        by = collections.OrderedDict()
        for r in sorted(rows, key=lambda r: int(r['Dispatch_Id'])):
            did = int(r['Dispatch_Id'])
            if did in by: by[did][1] += float(r['Counter_Value'])
            else: by[did] = [r['Kernel_Name'], float(r['Counter_Value'])]
        return by
    def classify(by):
        # q|k|v: the store-epilogue GEMM right before an attention; o: the residual GEMM right
        # before a gate|up; gate|up: the SwiGLU-epilogue GEMM; down: the residual GEMM right after it
        seq = list(by.items())
        cls = collections.defaultdict(list)
        probe = []
        for i, (did, (name, v)) in enumerate(seq):
            nxt = seq[i + 1][1][0] if i + 1 < len(seq) else ''
            prev = seq[i - 1][1][0] if i > 0 else ''
            if 'elementwise' in name and 'neg' in name.lower() and len(probe) < 3:
                probe.append(v)
            if 'k_gemm<0, 2,' in name:
                cls['gate_up'].append(v)
            elif 'k_gemm<0, 1,' in name and 'k_gemm<0, 2,' in prev:
                cls['down'].append(v)
            elif 'k_gemm<0, 1,' in name and 'k_gemm<0, 2,' in nxt:
                cls['o'].append(v)
            elif 'k_gemm<0, 0,' in name and 'k_attention' in nxt:
                cls['qkv'].append(v)
        return probe, cls
    out = []
    sh = hashlib.sha256(open('block_verify_forward_amd/csrc/gemm.hip', 'rb').read()).hexdigest()
    res = {}
    for d, counter, ideal in [(fetch_dir, 'FETCH_SIZE', probe_mib * 1024), (write_dir, 'WRITE_SIZE', probe_mib * 1024)]:
        probe, cls = classify(load(d, counter))
        p = sum(probe) / len(probe)
        scale = ideal / p
        out.append(f"{counter}: copy probe {p:.1f} KiB per dispatch ({len(probe)} dispatches) -> scale {scale:.4f}")
        for c, v in cls.items():
            kib = sum(v) / len(v)
            res.setdefault(c, {})[counter] = (len(v), kib, kib * scale * 1024)
    pass_traffic = pass_alg = 0.0
    for c in ("qkv", "o", "gate_up", "down"):
        f, w = res[c]['FETCH_SIZE'], res[c]['WRITE_SIZE']
        tot = f[2] + w[2]
        pass_traffic += tot
        pass_alg += alg[c]
        out.append(f"\n{c} dispatches: {f[0]}")
        out.append(f"  FETCH_SIZE {f[1]:.1f} KiB per dispatch -> {f[2]/1e6:.2f} MB")
        out.append(f"  WRITE_SIZE {w[1]:.1f} KiB per dispatch -> {w[2]/1e6:.2f} MB")
        out.append(f"  algorithmic bytes per launch (class average of the Q4_1 image, 0.625 B per weight): {alg[c]/1e6:.2f} MB")
        out.append(f"  traffic / algorithmic: {tot/alg[c]:.3f}")
        out.append(f"traffic_bytes_per_launch.{c}: {int(tot)}")
    out.append("\nwhole Q4_1 stream (one launch of each class per layer, averaged over the 4 launches):")
    out.append(f"  traffic / algorithmic: {pass_traffic / pass_alg:.3f}")
    out.append(f"traffic_bytes_per_launch.all: {int(pass_traffic / 4)}")
    out.append(f"\ngemm_hip_sha256: {sh}")
    print("\n".join(out))


def mfma(ARGV):
    PEAK_BF16 = 2.5e15
    d = ARGV[1]
    f = glob.glob(f"{d}/**/*counter_collection.csv", recursive=True)[0]
    by = collections.OrderedDict()
    for r in sorted(csv.DictReader(open(f)), key=lambda r: int(r["Dispatch_Id"])):
        e = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    allseq = list(by.values())
    # the GEMMs of a layer: q|k|v (store epilogue, followed by attention), o (residual, before
    # gate|up), gate|up (SwiGLU epilogue), down (residual, right after gate|up). Wide launches
    # (prefill chunks) are each followed by their split-sum kernel (k_splitk_epilogue): it is
    # skipped when looking at neighbours, and its duration is reported beside the GEMM's. Such chunks
    # also run their RMSNorms as k_rmsnorm before q|k|v and gate|up: skipped the same way.
    seq = [e for e in allseq if "k_splitk_epilogue" not in e["name"] and "k_rmsnorm" not in e["name"]]
    follow = {}
    for i, e in enumerate(allseq):
        if "k_gemm" in e["name"] and i + 1 < len(allseq) and "k_splitk_epilogue" in allseq[i + 1]["name"]:
            follow[id(e)] = allseq[i + 1]["ns"]
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
    print(f"{'class':8s} {'dispatches':>10s} {'MFMA GFLOP/launch':>18s} {'GEMM us':>8s} {'sum us':>7s} {'TFLOP/s':>9s} {'% of bf16 peak':>15s}")
    for c in ("q|k|v", "o", "gate|up", "down"):
        v = cls[c]
        if not v:
            continue
        fl = sum((e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + e["SQ_INSTS_VALU_MFMA_MOPS_F32"]) * 512 for e in v)
        ns = sum(e["ns"] for e in v)
        ns_sum = sum(follow.get(id(e), 0) for e in v)
        print(f"{c:8s} {len(v):10d} {fl / len(v) / 1e9:18.3f} {ns / len(v) / 1e3:8.2f} {ns_sum / len(v) / 1e3:7.2f} "
              f"{fl / ns / 1e3:9.1f} {100 * fl / (ns * 1e-9) / PEAK_BF16:15.2f}")
    print("(TFLOP/s: the MFMA work over the GEMM kernel's own duration; 'sum us': the split-sum kernel that follows a wide")
    print(" launch, 0 where there is none)")


def attn_traffic(ARGV):
    fetch_dir, write_dir, probe_mib = ARGV[1], ARGV[2], int(ARGV[3])
    alg = {"one sub-chunk": float(ARGV[4]), "two-stage": float(ARGV[5])}
    def load(d, counter):
        f = glob.glob(f"{d}/**/*counter_collection.csv", recursive=True)[0]
        by = collections.OrderedDict()
        for r in csv.DictReader(open(f)):
            if r['Counter_Name'] != counter:
                continue
            did = int(r['Dispatch_Id'])
            if did in by: by[did][1] += float(r['Counter_Value'])
            else: by[did] = [r['Kernel_Name'], float(r['Counter_Value'])]
        return by
    def form(name):
        if 'k_attn_combine' in name: return 'combine'
        if 'k_attention<' in name: return 'two-stage' if name.split('>')[0].endswith('true') else 'one sub-chunk'
        return None
    res = {}
    for d, counter in [(fetch_dir, 'FETCH_SIZE'), (write_dir, 'WRITE_SIZE')]:
        by = load(d, counter)
        probe = [v for n, v in by.values() if 'elementwise' in n and 'neg' in n.lower()][:3]
        scale = probe_mib * 1024 / (sum(probe) / len(probe))
        print(f"{counter}: copy probe {sum(probe) / len(probe):.1f} KiB per dispatch ({len(probe)} dispatches) -> scale {scale:.4f}")
        for n, v in by.values():
            f = form(n)
            if f: res.setdefault(f, {}).setdefault(counter, []).append(v * scale * 1024)
    for f in ('one sub-chunk', 'two-stage', 'combine'):
        if f not in res: continue
        fe, wr = res[f]['FETCH_SIZE'], res[f]['WRITE_SIZE']
        fm, wm = sorted(fe)[len(fe) // 2], sorted(wr)[len(wr) // 2]
        print(f"\n{f}: {len(fe)} dispatches (median of each counter)")
        print(f"  FETCH_SIZE -> {fm / 1e6:.2f} MB, WRITE_SIZE -> {wm / 1e6:.2f} MB per dispatch")
        if f in alg:
            print(f"  K/V bytes a launch reads: {alg[f] / 1e6:.2f} MB; fetched / K/V: {fm / alg[f]:.3f}")
    sh = hashlib.sha256(open('block_verify_forward_amd/csrc/layer_ops.hip', 'rb').read()).hexdigest()
    print(f"\nlayer_ops_hip_sha256: {sh}")


if __name__ == "__main__":
    cmds = {"kernel-trace": kernel_trace, "pmc-traffic": pmc_traffic, "mfma": mfma, "attn-traffic": attn_traffic}
    if len(sys.argv) < 3 or sys.argv[1] not in cmds:
        sys.exit(__doc__)
    cmds[sys.argv[1]](sys.argv[1:])

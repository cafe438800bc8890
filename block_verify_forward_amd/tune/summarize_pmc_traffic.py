"""Summary of two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
bench.py --no-graph --copy-probe-mib N: each counter is scaled by what it reads for the copy probe
(torch neg over N MiB: N MiB read, N MiB written), and the Q4_1 GEMM dispatches of the verify
passes are classed by their place in each layer (gate|up = the SwiGLU-epilogue GEMM, down = the
residual GEMM right after it). Prints HBM bytes per launch and the GEMM source hash that bench.py
checks before it reports the traffic.

usage: python summarize_pmc_traffic.py <fetch dir> <write dir> <probe MiB> <gate|up algorithmic
       bytes per launch> <down algorithmic bytes per launch>   (run from the repository root)"""
import csv, glob, sys, hashlib, collections
fetch_dir, write_dir, probe_mib = sys.argv[1], sys.argv[2], int(sys.argv[3])
alg = {"gate_up": float(sys.argv[4]), "down": float(sys.argv[5])}   # algorithmic bytes per launch (class average)
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
    seq = list(by.items())
    cls = collections.defaultdict(list)
    probe = []
    prev = None
    for did, (name, v) in seq:
        if 'elementwise' in name and 'neg' in name.lower() and len(probe) < 3:
            probe.append(v)
        if 'k_gemm<0, 2,' in name:
            cls['gate_up'].append(v)
        elif 'k_gemm<0, 1,' in name and prev is not None and 'k_gemm<0, 2,' in prev:
            cls['down'].append(v)
        prev = name
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
for c in ("gate_up", "down"):
    f, w = res[c]['FETCH_SIZE'], res[c]['WRITE_SIZE']
    tot = f[2] + w[2]
    out.append(f"\n{c} dispatches: {f[0]}")
    out.append(f"  FETCH_SIZE {f[1]:.1f} KiB per dispatch -> {f[2]/1e6:.2f} MB")
    out.append(f"  WRITE_SIZE {w[1]:.1f} KiB per dispatch -> {w[2]/1e6:.2f} MB")
    out.append(f"  algorithmic bytes per launch (class average of the Q4_1 image, 0.625 B per weight): {alg[c]/1e6:.2f} MB")
    out.append(f"  traffic / algorithmic: {tot/alg[c]:.3f}")
    out.append(f"traffic_bytes_per_launch.{c}: {int(tot)}")
out.append(f"\ngemm_hip_sha256: {sh}")
print("\n".join(out))

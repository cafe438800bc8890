"""Summary of a rocprofv3 --kernel-trace --stats csv run of bench.py: the per-kernel statistics,
then the median of the first 7 verify passes (embed ... accept, `want` kernels each) with every
kernel labelled by its place in the layer (q|k|v, attention, combine, o, gate|up, down).

usage: python summarize_kernel_trace.py <rocprofv3 output dir> [kernels per pass, default 256]"""
import csv, glob, sys, collections
d = sys.argv[1]
stats = glob.glob(f"{d}/**/*kernel_stats.csv", recursive=True)
trace = glob.glob(f"{d}/**/*kernel_trace.csv", recursive=True)
rows = list(csv.DictReader(open(stats[0])))
print(f"{'kernel':40s} {'calls':>7s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'share %':>8s}")
for r in rows:
    print(f"{r['Name'][:40]:40s} {int(r['Calls']):7d} {float(r['AverageNs'])/1e3:9.2f} {float(r['MinNs'])/1e3:9.2f} {float(r['MaxNs'])/1e3:9.2f} {float(r['Percentage']):8.2f}")
tr = list(csv.DictReader(open(trace[0])))
tr.sort(key=lambda r: int(r['Start_Timestamp']))
names = [r['Kernel_Name'] for r in tr]
def short(n):
    n = n.replace('void ', '')
    for pre in ('bvf::(anonymous namespace)::', 'bvf::'):
        n = n.replace(pre, '')
    i = n.find('(')
    return n[:i] if i > 0 else n
# last pass: from the last k_embed that is followed by a k_accept before the next k_embed
emb = [i for i, n in enumerate(names) if 'k_embed' in n]
passes = []
for j, i in enumerate(emb):
    end = emb[j + 1] if j + 1 < len(emb) else len(names)
    acc = [q for q in range(i, end) if 'k_accept' in names[q]]
    if acc:
        passes.append((i, acc[0]))
want = int(sys.argv[2]) if len(sys.argv) > 2 else 256
cands = [p for p in passes if p[1] - p[0] + 1 == want][:7]
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

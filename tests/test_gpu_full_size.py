"""GPU parity at the benchmark's full size: the target-shaped verify (42 layers, hidden 2560, Q4_1,
tied bf16 head 262144 x 2560, 1024 cached positions; k = 8 and k = 1), run the way the benchmark
runs it (the captured graph), against the CPU oracle on the same seeded inputs; full-size Q4_1
GEMMs of every matrix kind; the greedy accept over a 262144-entry vocabulary; commit and
snapshot/restore at full size."""
import dataclasses
import os

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import GEMM_TOL, compare_taps, dev, embed_rows, host, logits_bar, run_verify
from tests.util import rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P = 1024
THREADS = min(16, os.cpu_count() or 8)
MAT = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}


@pytest.fixture(scope="module")
def full():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m = synth.target_model(max_ctx=P + 64)
    w = synth.make_weights(m, 0, threads=THREADS)
    kv = synth.make_kv(m, P, 0)
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, P)
    g.set_graph_mode(True)
    yield m, w, kv, g
    torch.cuda.synchronize()


@pytest.mark.parametrize("layer", [0, 5, 30, 41])
def test_full_size_gemms(full, layer):
    """Own sliding (0), own full (5), shared sliding (30) and shared full (41) layers: every matrix
    at its real shape, 8 rows, rel-L1 per row within fp32 accumulation order."""
    m, w, kv, g = full
    for key, (n_out, n_in) in synth.layer_matrix_shapes(m, layer).items():
        x = synth.bf16_normal(0, f"full.gemm.{layer}.{key}", (8, n_in))
        y = torch.empty((8, n_out), dtype=torch.float32, device="cuda")
        g.q4_1_gemm(layer, MAT[key], dev(x), 8, y)
        ref = oracle.q4_1_matmul(w["layers"][layer][key], n_out, n_in, x)
        err = rel_l1(host(y), ref)
        print(f"layer {layer} {key} {n_out}x{n_in}: rel-L1 {err:.2e}")
        assert err < GEMM_TOL


@pytest.mark.parametrize("rows", [3, 13, 16])
@pytest.mark.parametrize("layer", [0, 30])
def test_full_size_gemms_ragged_rows(full, layer, rows):
    """The gate|up and down matrices of an own (0) and a shared (30) layer at row counts that are
    not 8 (the planner's split-K and wide-tile plans at ragged M), rel-L1 per row."""
    m, w, kv, g = full
    shapes = synth.layer_matrix_shapes(m, layer)
    for key in ("gate", "up", "down"):
        n_out, n_in = shapes[key]
        x = synth.bf16_normal(0, f"full.gemm.ragged.{layer}.{key}.{rows}", (rows, n_in))
        y = torch.empty((rows, n_out), dtype=torch.float32, device="cuda")
        g.q4_1_gemm(layer, MAT[key], dev(x), rows, y)
        ref = oracle.q4_1_matmul(w["layers"][layer][key], n_out, n_in, x)
        err = rel_l1(host(y), ref)
        print(f"layer {layer} {key} {n_out}x{n_in}, {rows} rows: rel-L1 {err:.2e}")
        assert err < GEMM_TOL


@pytest.mark.parametrize("rows", [40, 64])
@pytest.mark.parametrize("layer", [0, 5, 30])
def test_full_size_gemms_wide_rows(full, layer, rows):
    """Prefill chunk widths (40 rows: four row tiles, the last partly empty; 64: four full tiles):
    every matrix of an own sliding (0), own full (5) and shared (30) layer at its real shape, rel-L1
    per row within fp32 accumulation order."""
    m, w, kv, g = full
    for key, (n_out, n_in) in synth.layer_matrix_shapes(m, layer).items():
        x = synth.bf16_normal(0, f"full.gemm.wide.{layer}.{key}.{rows}", (rows, n_in))
        y = torch.empty((rows, n_out), dtype=torch.float32, device="cuda")
        g.q4_1_gemm(layer, MAT[key], dev(x), rows, y)
        ref = oracle.q4_1_matmul(w["layers"][layer][key], n_out, n_in, x)
        err = rel_l1(host(y), ref)
        print(f"layer {layer} {key} {n_out}x{n_in}, {rows} rows: rel-L1 {err:.2e}")
        assert err < GEMM_TOL


def test_full_size_prefill_64(full):
    """One 64-row prefill chunk at full size on the 1024 cached positions: counts exact, the last
    row's logits within the fixed 2e-3 bar of the oracle's batched rows, the appended K/V rows of
    layer 0 to the GEMM's accumulation order and of the other own layers within the logits bar."""
    m, w, kv, g = full
    n = 64
    snap = g.snapshot_take()
    toks = synth.tokens(0, "full.prefill", n, m.vocab)
    last = torch.empty(m.vocab, dtype=torch.float32, device="cuda")
    print(f"[full prefill] {n} rows at {P} cached positions", flush=True)
    g.prefill(dev(toks), last)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    rlg = o.verify_batch(toks)
    o.commit_verify_rows(n)
    assert g.positions_held() == o.held() == P + n
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    err = rel_l1(host(last)[None, :], rlg[-1:])
    tol = logits_bar(err, m, None, None, "full-size prefill of 64 rows: last row")
    assert err < tol
    for l in range(m.n_layers):
        if not m.own(l):
            continue
        gp, op = g.get_kv(l, P + n).astype(np.float64), o.plane(l, P + n).astype(np.float64)
        assert np.array_equal(gp[:P], op[:P]), f"layer {l}: cached rows changed"
        kv_err = rel_l1(gp[P:].reshape(2 * n, -1), op[P:].reshape(2 * n, -1))
        bar = GEMM_TOL if l == 0 else tol
        assert kv_err < bar, f"layer {l}: {kv_err:.2e}"
    g.restore(snap)
    assert g.positions_held() == P


@pytest.mark.parametrize("k", [8, 1, 5, 13])
def test_full_size_verify(full, k):
    """The benchmark's step at full size (k = 8, 1) and at ragged row counts (5, 13): logits of every
    row within the stack bar, the taps, the greedy tokens where the top-2 margin is clear, the
    accept decision bit-exact, KV counts."""
    m, w, kv, g = full
    toks = synth.tokens(0, "bench.tokens", max(8, k), m.vocab)[:k]   # the benchmark's rows first
    lg, taps = run_verify(g, m, toks)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P)
        return x.verify_embedded(arrs[0])

    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, run_oracle, [embed_rows(w, toks)] + kv, f"full-size verify k={k}")
    assert err < tol
    compare_taps(taps, rtaps, tol)
    assert g.positions_held() == o.held() == P + k
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    # the fp32 K/V rows this verify appended, element by element against the oracle's planes: the
    # cached rows untouched, layer 0's rows to the GEMM's accumulation order (its input rows are
    # the embedding rows on both sides), deeper layers within the logits bar (their inputs carry
    # the stack's rounding differences); K and V rows compared separately
    for l in range(m.n_layers):
        if not m.own(l):
            continue
        gp, op = g.get_kv(l, P + k).astype(np.float64), o.plane(l, P + k).astype(np.float64)
        assert np.array_equal(gp[:P], op[:P]), f"layer {l}: cached rows changed"
        kv_err = rel_l1(gp[P:].reshape(2 * k, -1), op[P:].reshape(2 * k, -1))
        bar = GEMM_TOL if l == 0 else tol
        print(f"layer {l}: appended K/V rows rel-L1 {kv_err:.2e} (bar {bar:.1e})")
        assert kv_err < bar, f"layer {l}"
    for i in range(k):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert lg[i].argmax() == rlg[i].argmax(), f"row {i}"
    # the accept kernel over V = 262144 decides exactly as the oracle's accept on the same logits
    lg_dev = dev(lg)
    out = torch.zeros(k, dtype=torch.int32, device="cuda")
    n_acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.accept_greedy(lg_dev, dev(toks.astype(np.int32)), out, n_acc)
    a, emitted = oracle.accept_greedy(lg, toks)
    assert int(host(n_acc)[0]) == a
    assert np.array_equal(host(out)[: a + 1], emitted)
    g.commit_verify_rows(0)
    assert g.positions_held() == P


def test_full_size_commit_snapshot_restore(full):
    """commit_verify_rows(n) for every n of a k = 8 verify at full size, and snapshot/restore of the
    per-layer planes (K and V rows of 256 / 512 floats per position, shared planes empty): the
    counts against the oracle for n = 0, 3, 8 and against their closed form for every n."""
    m, w, kv, g = full
    toks = synth.tokens(0, "full.commit", 8, m.vocab)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    snap = g.snapshot_take()
    osnap = o.snapshot()
    assert np.array_equal(snap.floats(), osnap.floats())
    widths = g.kv_widths()
    assert np.array_equal(widths, o.kv_widths())
    own = np.array([L.kv_owner < 0 for L in m.layers])
    lg = torch.empty((8, m.vocab), dtype=torch.float32, device="cuda")
    for n in range(9):
        g.verify_batch(dev(toks), lg, None)
        g.commit_verify_rows(n)
        assert g.positions_held() == P + n
        assert np.array_equal(g.plane_floats(), np.where(own, (P + n) * 2 * widths, 0))
        if n in (0, 3, 8):
            o.verify_batch(toks)
            o.commit_verify_rows(n)
            assert o.held() == P + n
            assert np.array_equal(g.plane_floats(), o.plane_floats())
            o.restore(osnap)
        g.restore(snap)
        assert g.positions_held() == P
        assert np.array_equal(g.plane_floats(), np.where(own, P * 2 * widths, 0))
    # K (= V) floats per position: 2 x 256 on sliding layers, 2 x 512 on full layers
    assert set(int(x) for x in widths[:24]) == {256, 512}
    assert all(int(f) == 0 for f in g.plane_floats()[24:])


@pytest.mark.parametrize("n_new", [1, 8])
def test_full_size_draft_block(full, n_new):
    """The draft block forward at its real size: 5 layers of hidden 2560 (32 query / 8 KV heads of
    128, FFN 5120, window 1024), fc over 5 taps of 2560, 1024 cached context rows plus n_new rows
    appended from taps, a block of 8 and the target's tied head over 262144 entries: logits of
    rows 1..7 and the proposals, against the oracle."""
    m, w, kv, g = full
    dm = synth.draft_model(max_ctx=P + 64)
    dmg = dataclasses.replace(dm, vocab=m.vocab)   # the draft's logits scratch takes the target's vocab
    dw = synth.make_weights(dm, 0, threads=THREADS)
    kvd = synth.make_kv(dm, P, 0, threads=THREADS)
    taps = synth.bf16_normal(0, "full.draft.taps", (n_new, len(dm.tap_layers), dm.hidden))
    D = bvf.Model(dmg)
    D.load_weights(dw)
    D.set_context(kvd, P)
    block = 8
    props = torch.zeros(block - 1, dtype=torch.int32, device="cuda")
    lg = torch.empty((block - 1, m.vocab), dtype=torch.float32, device="cuda")
    D.draft_block_forward(g, dev(taps), n_new, dev(np.array([17], dtype=np.int32)), block, 1.0, m.vocab - 1, props, lg)
    assert D.positions_held() == P + n_new
    To = oracle.Model(m, w)
    x0 = embed_rows(w, [17] + [m.vocab - 1] * (block - 1))

    def run_oracle(arrs):
        Do = oracle.Model(dm, dw)
        Do.set_kv(arrs[1:], P)
        Do.draft_append(taps)
        return oracle.draft_block_embedded(Do, To, arrs[0])

    rp, rlg = run_oracle([x0] + kvd)
    glg = host(lg)
    err = rel_l1(glg, rlg)
    tol = logits_bar(err, dm, lambda a: run_oracle(a)[1], [x0] + kvd, f"full-size draft block n_new={n_new}")
    print(f"full-size draft n_new={n_new}: logits rel-L1 {err:.2e} (bar {tol:.2e})")
    assert err < tol
    gp = host(props)
    for i in range(block - 1):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert gp[i] == rp[i], f"proposal {i}"

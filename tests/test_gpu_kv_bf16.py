"""GPU parity of the bf16 K/V planes (a memory variant of the per-layer planes of [PR2303], "What
changes" item 1: every stored K/V value, whether set as cached context, appended by a verify pass
or a draft context append, or written by a draft block's own rows, is the fp32 value rounded to
bf16, nearest even) against the oracle run with the same option.

Bars: cached rows read back bit-exact (the host rounding of bvf_set_kv against the oracle's);
appended rows bf16-representable; at the first layer (the same input rows on both sides) 99% of
them identical to the oracle's and the rest within one bf16 unit plus the fp32 accumulation error;
rel-L1 inside the logits bar at every layer; logits and proposals as in the fp32-plane tests."""
import dataclasses
import os

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import compare_taps, dev, embed_rows, host, logits_bar, ragged_model, run_verify
from tests.util import rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 8)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    bvf.lib()
    yield
    torch.cuda.synchronize()


def bf16_model(m):
    return dataclasses.replace(m, kv_bf16=1)


def build_pair(m, P, seed=0, threads=1):
    w = synth.make_weights(m, seed, threads=threads)
    kv = synth.make_kv(m, P, seed, threads=threads)
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, P)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    return g, o, w, kv


def is_bf16(a: np.ndarray) -> bool:
    return not np.any(np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) & 0xFFFF)


def close_bf16_rows(g: np.ndarray, o: np.ndarray) -> bool:
    """Two bf16 roundings of the same rows computed in fp32 and in fp64: at least 99% identical, and
    every value within one bf16 unit in the last place of the larger magnitude (7 stored fraction
    bits) plus 2^-10 of the row's rms (the fp32 accumulation and bf16-input differences before the
    rounding, which a value near zero cannot absorb in its own unit). Rounding by truncation instead
    of to nearest would leave about half the values off by one unit."""
    g = g.astype(np.float64)
    o = o.astype(np.float64)
    same = np.mean(g == o)
    mag = np.maximum(np.abs(g), np.abs(o))
    ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    worst = np.max(np.abs(g - o) - ulp - rms / 1024.0)
    print(f"identical {same:.4f}, worst excess over the bound {worst:.2e}")
    return bool(same >= 0.99 and worst <= 0)


def own_layers(m):
    return [l for l in range(m.n_layers) if m.layers[l].kv_owner < 0]


def check_planes(g, o, m, P, n_new, tol):
    """Rows 0..P-1 bit-exact; rows P..P+n_new-1 bf16 values close to the oracle's."""
    for l in own_layers(m):
        gp = g.get_kv(l, P + n_new)
        op = o.plane(l, P + n_new)
        assert is_bf16(gp), f"layer {l}: a stored value is not a bf16 value"
        assert np.array_equal(gp[:P].astype(np.float64), op[:P]), f"layer {l}: cached rows"
        if n_new:
            a, b = gp[P:].reshape(n_new, -1), op[P:].reshape(n_new, -1)
            err = rel_l1(a, b)
            print(f"layer {l}: appended rows rel-L1 {err:.2e}")
            assert err < tol, f"layer {l}"
            if l == 0:
                assert close_bf16_rows(a, b), "layer 0: appended rows differ beyond the rounding"


# ------------------------------------------------------------------------------------------
# planes in and out
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("kv_bf16", [0, 1])
def test_set_get_kv_round_trip(kv_bf16):
    """fp32 planes read back the floats set; bf16 planes read back the oracle's rounding of them."""
    m = dataclasses.replace(synth.tiny_two_width_model(), kv_bf16=kv_bf16)
    g, o, w, kv = build_pair(m, 33)
    for l in own_layers(m):
        got = g.get_kv(l, 33)
        if kv_bf16:
            assert is_bf16(got)
            assert np.array_equal(got.astype(np.float64), o.plane(l, 33))
            assert not np.array_equal(got, kv[l])          # the rounding did happen
        else:
            assert np.array_equal(got, kv[l])
    with pytest.raises(bvf.BvfError) as e:
        g.get_kv(4, 1)                                      # a shared layer holds no plane
    assert e.value.status == bvf.BVF_E_INVALID


def test_set_kv_rounds_ties_to_even():
    """Values on and beside bf16 rounding ties, through bvf_set_kv and back."""
    m = bf16_model(synth.tiny_model(max_ctx=8))
    g = bvf.Model(m)
    g.load_weights(synth.make_weights(m))
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8),
                     2.0 ** -130, 3.0e38, 0.0, -0.0], dtype=np.float32)
    want = np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0], dtype=np.float64)
    kv = np.zeros((1, 2, 64), dtype=np.float32)
    kv[0, 0, :8] = vals
    g.set_kv(0, kv, 1)
    g.set_positions(1)
    got = g.get_kv(0, 1)[0, 0, :8]
    assert np.array_equal(got[:4].astype(np.float64), want)
    assert is_bf16(got)
    assert np.signbit(got[7]) and got[6] == 0


# ------------------------------------------------------------------------------------------
# the verify pass, commit and snapshot
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("mk, P, k", [(synth.tiny_two_width_model, 40, 8), (ragged_model, 30, 16),
                                      (synth.tiny_two_width_model, 0, 5), (synth.tiny_model, 64, 1)])
def test_verify_parity_kv_bf16(mk, P, k):
    m = bf16_model(mk())
    g, o, w, kv = build_pair(m, P)
    toks = synth.tokens(0, f"kvb.verify.{m.name}", k, m.vocab)
    lg, taps = run_verify(g, m, toks)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P)
        return x.verify_embedded(arrs[0])

    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, run_oracle, [embed_rows(w, toks)] + kv, f"bf16 planes verify P={P} k={k}")
    assert err < tol
    if m.tap_layers:
        compare_taps(taps, rtaps, tol)
    assert g.positions_held() == o.held() == P + k
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    check_planes(g, o, m, P, k, tol)
    for i in range(k):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert lg[i].argmax() == rlg[i].argmax()


@pytest.mark.parametrize("n", [0, 3, 8])
def test_commit_then_next_pass_kv_bf16(n):
    """commit_verify_rows(n) keeps the first n appended rows; the next pass sees exactly those."""
    m = bf16_model(synth.tiny_two_width_model())
    g, o, w, kv = build_pair(m, 24)
    toks = synth.tokens(0, "kvb.commit.toks", 8, m.vocab)
    run_verify(g, m, toks, with_taps=False)
    rows = [g.get_kv(l, 32) for l in own_layers(m)]
    g.commit_verify_rows(n)
    assert g.positions_held() == 24 + n
    assert np.array_equal(g.plane_floats(), [(24 + n) * 2 * m.kv_width(l) if m.own(l) else 0
                                             for l in range(m.n_layers)])
    nxt = synth.tokens(2, "kvb.commit.next", 4, m.vocab)
    lg, _ = run_verify(g, m, nxt, with_taps=False)
    for l, before in zip(own_layers(m), rows):          # committed rows untouched by the next pass
        assert np.array_equal(g.get_kv(l, 24 + n), before[:24 + n])

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], 24)
        for t in toks[:n]:
            x.step(int(t))
        return x.verify_embedded(arrs[0])

    arrs = [embed_rows(w, nxt)] + kv
    err = rel_l1(lg, run_oracle(arrs))
    assert err < logits_bar(err, m, run_oracle, arrs, f"bf16 planes commit({n}), next pass")


def test_snapshot_restore_kv_bf16():
    """A snapshot of bf16 planes restores them bit-exactly; a snapshot of fp32 planes of the same
    geometry is refused by a bf16 model (and the reverse), leaving its state unchanged."""
    m = bf16_model(synth.tiny_two_width_model())
    g, o, w, kv = build_pair(m, 18)
    snap = g.snapshot_take()
    assert snap.floats().tolist() == [18 * 2 * m.kv_width(l) if m.own(l) else 0 for l in range(m.n_layers)]
    before = [g.get_kv(l, 18) for l in own_layers(m)]
    run_verify(g, m, synth.tokens(0, "kvb.snap.a", 6, m.vocab), with_taps=False)
    g.commit_verify_rows(6)
    g.restore(snap)
    assert g.positions_held() == 18
    for l, b in zip(own_layers(m), before):
        assert np.array_equal(g.get_kv(l, 18), b)
    toks = synth.tokens(0, "kvb.snap.b", 5, m.vocab)
    lg, _ = run_verify(g, m, toks, with_taps=False)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], 18)
        return x.verify_embedded(arrs[0])

    arrs = [embed_rows(w, toks)] + kv
    err = rel_l1(lg, run_oracle(arrs))
    assert err < logits_bar(err, m, run_oracle, arrs, "bf16 planes, after snapshot restore")
    g.commit_verify_rows(0)
    m32 = dataclasses.replace(m, kv_bf16=0)
    g32, _, _, _ = build_pair(m32, 18)
    with pytest.raises(bvf.BvfError) as e:
        g32.restore(snap)
    assert e.value.status == bvf.BVF_E_INVALID
    assert g32.positions_held() == 18
    with pytest.raises(bvf.BvfError) as e:
        g.restore(g32.snapshot_take())
    assert e.value.status == bvf.BVF_E_INVALID
    assert g.positions_held() == 18


# ------------------------------------------------------------------------------------------
# DFlash draft block with bf16 planes
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window, n_ctx, n_new, block", [(0, 12, 4, 8), (6, 20, 3, 8), (0, 0, 8, 8)])
def test_draft_block_kv_bf16(window, n_ctx, n_new, block):
    tm = synth.tiny_model(max_ctx=64)
    tw = synth.make_weights(tm)
    dm = bf16_model(synth.tiny_draft_model(max_ctx=64, window=window))
    dmg = dataclasses.replace(dm, vocab=tm.vocab)
    dw = synth.make_weights(dm)
    kvd = synth.make_kv(dm, n_ctx)
    taps = synth.bf16_normal(0, "kvb.draft.taps", (n_new, len(dm.tap_layers), dm.hidden))
    T = bvf.Model(tm)
    T.load_weights(tw)
    D = bvf.Model(dmg)
    D.load_weights(dw)
    D.set_context(kvd, n_ctx)
    To = oracle.Model(tm, tw)
    props = torch.zeros(block - 1, dtype=torch.int32, device="cuda")
    lg = torch.empty((block - 1, tm.vocab), dtype=torch.float32, device="cuda")
    D.draft_block_forward(T, dev(taps) if n_new else None, n_new, dev(np.array([17], dtype=np.int32)), block, 1.0,
                          tm.vocab - 1, props, lg)
    assert D.positions_held() == n_ctx + n_new
    x0 = embed_rows(tw, [17] + [tm.vocab - 1] * (block - 1))

    def run_oracle(arrs, keep=None):
        Do = oracle.Model(dm, dw)
        Do.set_kv(arrs[1:], n_ctx)
        if n_new:
            Do.draft_append(taps)
        r = oracle.draft_block_embedded(Do, To, arrs[0])
        if keep is not None:
            keep.append(Do)
        return r

    held = []
    rp, rlg = run_oracle([x0] + kvd, held)
    glg = host(lg)
    err = rel_l1(glg, rlg)
    tol = logits_bar(err, dm, lambda a: run_oracle(a)[1], [x0] + kvd, f"bf16 planes draft w={window} ctx={n_ctx} new={n_new} B={block}")
    assert err < tol
    check_planes(D, held[0], dm, n_ctx, n_new, tol)
    gp = host(props)
    for i in range(block - 1):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert gp[i] == rp[i]


# ------------------------------------------------------------------------------------------
# the target and draft at full size (head dims 256 and 128)
# ------------------------------------------------------------------------------------------
def test_full_size_verify_kv_bf16():
    """The target-shaped verify (42 layers, hidden 2560, head dim 256, KV widths 256 and 512, shared
    layers) over 4096 cached positions with k = 8, as the benchmark runs it (captured graph)."""
    P, k = 4096, 8
    m = bf16_model(synth.target_model(max_ctx=P + 64))
    g, o, w, kv = build_pair(m, P, threads=THREADS)
    g.set_graph_mode(True)
    toks = synth.tokens(0, "kvb.full", k, m.vocab)
    lg, taps = run_verify(g, m, toks)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P)
        return x.verify_embedded(arrs[0])

    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, run_oracle, [embed_rows(w, toks)] + kv, "full-size verify, bf16 planes")
    assert err < tol
    compare_taps(taps, rtaps, tol)
    check_planes(g, o, m, P, k, tol)
    for i in range(k):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert lg[i].argmax() == rlg[i].argmax(), f"row {i}"
    g.commit_verify_rows(3)
    assert g.positions_held() == P + 3


def test_full_size_draft_block_kv_bf16():
    """The draft at its real size (5 layers, 8 KV heads of 128, window 1024) with bf16 planes: 1024
    cached rows, 8 rows appended from taps, a block of 8 against the target's head."""
    P, n_new, block = 1024, 8, 8
    tm = synth.target_model(max_ctx=P + 64, n_layers=1)
    tw = synth.make_weights(tm, 0, threads=THREADS)
    T = bvf.Model(tm)
    T.load_weights(tw)
    dm = bf16_model(synth.draft_model(max_ctx=P + 64))
    dmg = dataclasses.replace(dm, vocab=tm.vocab)
    dw = synth.make_weights(dm, 0, threads=THREADS)
    kvd = synth.make_kv(dm, P, 0, threads=THREADS)
    taps = synth.bf16_normal(0, "kvb.full.draft.taps", (n_new, len(dm.tap_layers), dm.hidden))
    D = bvf.Model(dmg)
    D.load_weights(dw)
    D.set_context(kvd, P)
    props = torch.zeros(block - 1, dtype=torch.int32, device="cuda")
    lg = torch.empty((block - 1, tm.vocab), dtype=torch.float32, device="cuda")
    D.draft_block_forward(T, dev(taps), n_new, dev(np.array([17], dtype=np.int32)), block, 1.0, tm.vocab - 1,
                          props, lg)
    To = oracle.Model(tm, tw)
    x0 = embed_rows(tw, [17] + [tm.vocab - 1] * (block - 1))

    def run_oracle(arrs, keep=None):
        Do = oracle.Model(dm, dw)
        Do.set_kv(arrs[1:], P)
        Do.draft_append(taps)
        r = oracle.draft_block_embedded(Do, To, arrs[0])
        if keep is not None:
            keep.append(Do)
        return r

    held = []
    rp, rlg = run_oracle([x0] + kvd, held)
    err = rel_l1(host(lg), rlg)
    tol = logits_bar(err, dm, lambda a: run_oracle(a)[1], [x0] + kvd, "full-size draft block, bf16 planes")
    assert err < tol
    check_planes(D, held[0], dm, P, n_new, tol)
    gp = host(props)
    for i in range(block - 1):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert gp[i] == rp[i], f"proposal {i}"

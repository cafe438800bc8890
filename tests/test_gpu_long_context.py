"""GPU parity at long contexts: the target-shaped verify (42 layers, hidden 2560, Q4_1, bf16 head
262144 x 2560) over 4096 and 16384 cached positions with k = 1, 4, 8 and 16 rows, against the CPU
oracle on the same seeded inputs; commit_verify_rows(n) for every n of a k = 16 verify and a
snapshot/restore of the planes at that size."""
import dataclasses
import os

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import compare_taps, dev, embed_rows, host, logits_bar, run_verify
from tests.util import rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 8)


@pytest.fixture(scope="module", params=[4096, 16384])
def ctx(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    P = request.param
    m = synth.target_model(max_ctx=P + 64)
    w = synth.make_weights(m, 0, threads=THREADS)
    kv = synth.make_kv(m, P, 0, threads=THREADS)
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, P)
    g.set_graph_mode(True)
    yield P, m, w, kv, g
    torch.cuda.synchronize()


@pytest.mark.parametrize("k", [1, 4, 8, 16])
def test_long_context_verify(ctx, k):
    P, m, w, kv, g = ctx
    toks = synth.tokens(0, f"long.{P}", 16, m.vocab)[:k]
    lg, taps = run_verify(g, m, toks)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P)
        return x.verify_embedded(arrs[0])

    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, run_oracle, [embed_rows(w, toks)] + kv, f"target P={P} k={k}")
    assert err < tol
    compare_taps(taps, rtaps, tol)
    assert g.positions_held() == o.held() == P + k
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    for i in range(k):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert lg[i].argmax() == rlg[i].argmax(), f"row {i}"
    g.commit_verify_rows(0)
    assert g.positions_held() == P


def test_long_context_commit_sweep(ctx):
    """A k = 16 verify, then commit_verify_rows(n) for n = 0 .. 16 (restoring the snapshot in
    between): positions held P + n and floats (P + n) * 2 * w_l on own planes, 0 on shared ones."""
    P, m, w, kv, g = ctx
    toks = synth.tokens(0, f"long.commit.{P}", 16, m.vocab)
    widths = g.kv_widths()
    own = np.array([L.kv_owner < 0 for L in m.layers])
    snap = g.snapshot_take()
    assert np.array_equal(snap.floats(), np.where(own, P * 2 * widths, 0))
    lg = torch.empty((16, m.vocab), dtype=torch.float32, device="cuda")
    for n in range(17):
        g.verify_batch(dev(toks), lg, None)
        assert g.positions_held() == P + 16
        g.commit_verify_rows(n)
        assert g.positions_held() == P + n
        assert np.array_equal(g.plane_floats(), np.where(own, (P + n) * 2 * widths, 0))
        g.restore(snap)
        assert g.positions_held() == P
        assert np.array_equal(g.plane_floats(), np.where(own, P * 2 * widths, 0))
    torch.cuda.synchronize()
    assert np.isfinite(host(lg)).all()


# ------------------------------------------------------------------------------------------
# workgroups that take several sub-chunks (the two-stage K/V pipeline) at every head dim
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("kv_bf16", [0, 1])
def test_long_context_tiny_stack(kv_bf16):
    """The 6-layer miniature (head dim 64, widths 64 and 128, shared layers) over 26000 cached
    positions: enough keys that each attention workgroup takes several sub-chunks."""
    P, k = 26000, 8
    m = dataclasses.replace(synth.tiny_two_width_model(max_ctx=P + 16), kv_bf16=kv_bf16)
    w = synth.make_weights(m, 0)
    kv = synth.make_kv(m, P, 0)
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, P)
    toks = synth.tokens(0, "long.tiny", k, m.vocab)
    lg, taps = run_verify(g, m, toks)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P)
        return x.verify_embedded(arrs[0])

    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, run_oracle, [embed_rows(w, toks)] + kv, f"tiny stack at {P}, bf16 planes {kv_bf16}")
    assert err < tol
    compare_taps(taps, rtaps, tol)
    assert g.positions_held() == o.held() == P + k


@pytest.mark.parametrize("kv_bf16", [0, 1])
def test_long_context_draft_block(kv_bf16):
    """The draft at its real size (head dim 128, 8 KV heads) with an unlimited window over 16384
    cached context rows plus 8 appended from taps, a block of 8 against a one-layer target's head."""
    P, n_new, block = 16384, 8, 8
    tm = synth.target_model(max_ctx=P + 64, n_layers=1)
    tw = synth.make_weights(tm, 0, threads=THREADS)
    T = bvf.Model(tm)
    T.load_weights(tw)
    dm = dataclasses.replace(synth.draft_model(max_ctx=P + 64, window=0), kv_bf16=kv_bf16)
    dmg = dataclasses.replace(dm, vocab=tm.vocab)
    dw = synth.make_weights(dm, 0, threads=THREADS)
    kvd = synth.make_kv(dm, P, 0, threads=THREADS)
    taps = synth.bf16_normal(0, "long.draft.taps", (n_new, len(dm.tap_layers), dm.hidden))
    D = bvf.Model(dmg)
    D.load_weights(dw)
    D.set_context(kvd, P)
    props = torch.zeros(block - 1, dtype=torch.int32, device="cuda")
    lg = torch.empty((block - 1, tm.vocab), dtype=torch.float32, device="cuda")
    D.draft_block_forward(T, dev(taps), n_new, dev(np.array([17], dtype=np.int32)), block, 1.0, tm.vocab - 1,
                          props, lg)
    assert D.positions_held() == P + n_new
    To = oracle.Model(tm, tw)
    x0 = embed_rows(tw, [17] + [tm.vocab - 1] * (block - 1))

    def run_oracle(arrs):
        Do = oracle.Model(dm, dw)
        Do.set_kv(arrs[1:], P)
        Do.draft_append(taps)
        return oracle.draft_block_embedded(Do, To, arrs[0])

    rp, rlg = run_oracle([x0] + kvd)
    err = rel_l1(host(lg), rlg)
    tol = logits_bar(err, dm, lambda a: run_oracle(a)[1], [x0] + kvd, f"draft over {P} context rows, bf16 planes {kv_bf16}")
    assert err < tol
    gp = host(props)
    for i in range(block - 1):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert gp[i] == rp[i], f"proposal {i}"

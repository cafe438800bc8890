"""GPU ring planes (kv_ring): every own sliding layer keeps window + 16 position slots. Through the C
ABI the ring model must give bit-identical logits to the linear-plane model (the same kernels read
the same values, only at other addresses), count and snapshot the last min(held, window) positions
of a ring plane, and agree with the oracle's ring planes (engine PR #2303, "What changes" item 1:
per-layer cuts)."""
import dataclasses

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import build_pair, dev, host, logits_bar, run_verify
from tests.util import rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _keep(m, l, held):
    L = m.layers[l]
    if not m.own(l):
        return 0
    ring = getattr(m, "kv_ring", 0) and L.attn == synth.ATTN_SLIDING and L.window > 0 and L.window + 16 < m.max_ctx
    return min(held, L.window) if ring else held


@pytest.mark.parametrize("kv_bf16", [0, 1])
def test_ring_equals_linear_over_a_state_sequence(kv_bf16):
    """Two-width miniature (sliding window 16: rings of 32 slots): verifies of 8, 5, 16 and 4 rows
    with commits of 3, 5, 0 and 4, an extend_context of 7 rows, a snapshot and a restore. Every
    verify's logits are bit-identical to the linear model's, counts and snapshot floats follow
    min(held, window) on ring planes, the rows a ring holds equal the oracle ring's (cached and
    extended rows bit-exact), and the oracle's ring logits are within the stack bar."""
    base = dataclasses.replace(synth.tiny_two_width_model(), kv_bf16=kv_bf16)
    ring = dataclasses.replace(base, kv_ring=1)
    P = 45
    gl, ol, w, kv = build_pair(base, P)
    gr, orr, _, _ = build_pair(ring, P)
    kv_new = synth.make_kv(base, 7, 1)
    assert bvf.arena_bytes(ring) < bvf.arena_bytes(base)

    def step(k, n, tag):
        toks = synth.tokens(0, f"ring.gpu.{tag}", k, base.vocab)
        ll, _ = run_verify(gl, base, toks, with_taps=False)
        lr, _ = run_verify(gr, ring, toks, with_taps=False)
        assert np.array_equal(ll, lr), tag
        ro = orr.verify_batch(toks)
        err = rel_l1(lr, ro)
        print(f"[ring {tag}] logits rel-L1 vs oracle ring {err:.2e}")
        gl.commit_verify_rows(n); gr.commit_verify_rows(n)
        assert orr.commit_verify_rows(n) == 0
        h = gr.positions_held()
        assert h == gl.positions_held() == orr.held()
        want = [_keep(ring, l, h) * 2 * ring.kv_width(l) for l in range(ring.n_layers)]
        assert gr.plane_floats().tolist() == orr.plane_floats().tolist() == want
        return err

    errs = [step(8, 3, "a"), step(5, 5, "b")]
    gl.extend_context(kv_new, 7); gr.extend_context(kv_new, 7)
    assert orr.extend_context(kv_new, 7) == 0
    h = gr.positions_held()
    for l in range(ring.n_layers):
        if ring.own(l):
            keep = _keep(ring, l, h)
            got, ref = gr.get_kv(l, h), orr.plane(l, h)
            assert np.all(np.isnan(got[:h - keep]))
            assert np.array_equal(got[h - 7:], ref[h - 7:]), f"layer {l}: extended rows"
    snap = gr.snapshot_take()
    assert snap.floats().tolist() == [_keep(ring, l, h) * 2 * ring.kv_width(l) for l in range(ring.n_layers)]
    snap_l = gl.snapshot_take()
    snap_o = orr.snapshot()
    errs.append(step(16, 0, "c"))
    gl.restore(snap_l); gr.restore(snap)
    assert orr.restore(snap_o) == 0
    errs.append(step(4, 4, "d"))
    with pytest.raises(bvf.BvfError) as e:     # a ring snapshot does not fit a linear model
        gl.restore(snap)
    assert e.value.status == bvf.BVF_E_INVALID

    def run(arrs):
        x = oracle.Model(ring, w)
        x.set_kv(arrs, P)
        return x.verify_batch(synth.tokens(0, "ring.gpu.a", 8, base.vocab))

    assert errs[0] < logits_bar(errs[0], ring, run, kv, f"ring planes bf16={kv_bf16}, first verify")
    assert max(errs) < 0.1


def test_ring_full_size_4096_equals_linear():
    """Target-shaped stack at 4096 cached positions: ring planes (window 512: 528 slots on the 20
    own sliding layers) against linear planes, k = 8 and k = 16, logits bit-identical, commit counts
    per layer, and the arena smaller by the planes' difference. Then a prefill of 72 tokens (a
    64-row chunk, whose attention walks several sub-chunks per workgroup through two LDS stages,
    and an 8-row chunk) on both: last-token logits bit-identical and the window's rows of a ring
    plane equal to the linear plane's."""
    P = 4096
    base = synth.target_model(max_ctx=P + 128)
    ring = dataclasses.replace(base, kv_ring=1)
    w = synth.make_weights(base, 0, threads=16)
    kv = synth.make_kv(base, P, 0, threads=16)
    gl, gr = bvf.Model(base), bvf.Model(ring)
    for g in (gl, gr):
        g.load_weights(w)
        g.set_context(kv, P)
    print(f"[ring full size] arena linear {bvf.arena_bytes(base) / 2**30:.2f} GiB, ring {bvf.arena_bytes(ring) / 2**30:.2f} GiB",
          flush=True)
    assert bvf.arena_bytes(ring) < bvf.arena_bytes(base) - 20 * (P - 528) * 2 * 256 * 4
    for k in (8, 16):
        toks = synth.tokens(0, f"ring.full.{k}", k, base.vocab)
        ll, tl = run_verify(gl, base, toks)
        lr, tr = run_verify(gr, ring, toks)
        assert np.array_equal(ll, lr) and np.array_equal(tl, tr), f"k={k}"
        gl.commit_verify_rows(0)
        gr.commit_verify_rows(k // 2)
        want = [_keep(ring, l, P + k // 2) * 2 * ring.kv_width(l) for l in range(ring.n_layers)]
        assert gr.plane_floats().tolist() == want
        gr.set_positions(P)
    gl.set_positions(P)
    n = 72
    toks = torch.from_numpy(synth.tokens(0, "ring.full.prefill", n, base.vocab)).cuda()
    outs = []
    for g in (gl, gr):
        last = torch.empty(base.vocab, dtype=torch.float32, device="cuda")
        g.prefill(toks, last)
        torch.cuda.synchronize()
        outs.append(last.cpu().numpy())
        assert g.positions_held() == P + n
    assert np.array_equal(outs[0], outs[1]), "prefill logits"
    l_ring = next(l for l in range(ring.n_layers) if ring.own(l) and ring.layers[l].attn == synth.ATTN_SLIDING)
    a, b = gl.get_kv(l_ring, P + n), gr.get_kv(l_ring, P + n)
    win = ring.layers[l_ring].window
    assert np.array_equal(a[P + n - win:], b[P + n - win:]), "ring rows after the prefill"


def test_ring_refused_on_a_draft():
    dm = dataclasses.replace(synth.tiny_draft_model(), kv_ring=1)
    with pytest.raises(bvf.BvfError) as e:
        bvf.arena_bytes(dm)
    assert e.value.status == bvf.BVF_E_INVALID

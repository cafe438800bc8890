"""Chunked prefill on the GPU against the oracle, and snapshot/restore as a prefix cache.

The prefill runs the batched body in chunks of up to 64 rows (37: one chunk of three row tiles
and a ragged fourth; 100 and 150: full 64-row chunks and a ragged tail; 72: a 64-row chunk, whose
RMSNorms run as their own kernel, then an 8-row chunk, whose RMSNorms fold into the GEMMs'
staging) and keeps every row; the oracle runs
the same rows as one batched verify plus commit (its batched verify equals sequential steps bit for
bit). Compared: positions held and plane floats exactly; the last row's logits and the logits of a
verify that follows, within the stack bar (2e-3, or three times the oracle's own spread under
fp32-level perturbation of its inputs, as for the verify)."""
import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import dev, embed_rows, host, logits_bar
from tests.util import rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P0 = 24


@pytest.fixture(scope="module")
def setup():
    m = synth.tiny_two_width_model(max_ctx=256)
    w = synth.make_weights(m)
    kv = synth.make_kv(m, P0)
    return m, w, kv


def gpu_model(m, w, kv):
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, P0)
    return g


@pytest.mark.parametrize("n", [1, 16, 37, 64, 72, 100, 150])
def test_prefill_matches_oracle(setup, n):
    m, w, kv = setup
    g = gpu_model(m, w, kv)
    toks = synth.tokens(0, f"prefill.{n}", n, m.vocab)
    last = torch.empty(m.vocab, dtype=torch.float32, device="cuda")
    g.prefill(dev(toks), last)
    o = oracle.Model(m, w)
    o.set_kv(kv, P0)
    rlg = o.verify_batch(toks)
    o.commit_verify_rows(n)
    assert g.positions_held() == o.held() == P0 + n
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    err = rel_l1(host(last)[None, :], rlg[-1:])

    def run_prefill_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P0)
        return x.verify_embedded(arrs[0])[-1:]

    tol = logits_bar(err, m, run_prefill_oracle, [embed_rows(w, toks)] + kv, f"prefill {n}: last row")
    assert err < tol
    # the context the prefill left: a verify of 8 rows on top of it
    vt = synth.tokens(1, f"prefill.next.{n}", 8, m.vocab)
    lg = torch.empty((8, m.vocab), dtype=torch.float32, device="cuda")
    g.verify_batch(dev(vt), lg, None)
    rv = o.verify_batch(vt)
    err = rel_l1(host(lg), rv)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P0)
        x.verify_batch(toks)
        x.commit_verify_rows(n)
        return x.verify_embedded(arrs[0])

    tol = logits_bar(err, m, run_oracle, [embed_rows(w, vt)] + kv, f"prefill {n}: next verify")
    assert err < tol


def test_prefill_as_prefix_cache(setup):
    """Prefill a 40-token prefix once, snapshot; per continuation: restore, prefill the suffix,
    verify. Each equals a model that prefilled prefix + suffix from the start within the stack bar
    (the two chunkings group rows differently, so the GEMM plans differ), and the counts are exact."""
    m, w, kv = setup
    prefix = synth.tokens(0, "prefix", 40, m.vocab)
    cache = gpu_model(m, w, kv)
    cache.prefill(dev(prefix))
    snap = cache.snapshot_take()
    held0 = cache.positions_held()
    lg = torch.empty((4, m.vocab), dtype=torch.float32, device="cuda")
    lg2 = torch.empty((4, m.vocab), dtype=torch.float32, device="cuda")
    for j, ns in enumerate([5, 19, 33]):
        suffix = synth.tokens(j, "suffix", ns, m.vocab)
        cache.restore(snap)
        assert cache.positions_held() == held0 == P0 + 40
        cache.prefill(dev(suffix))
        vt = synth.tokens(j, "cont", 4, m.vocab)
        cache.verify_batch(dev(vt), lg, None)
        cold = gpu_model(m, w, kv)
        cold.prefill(dev(np.concatenate([prefix, suffix]).astype(np.int32)))
        cold.verify_batch(dev(vt), lg2, None)
        assert cache.positions_held() == cold.positions_held() == P0 + 40 + ns + 4
        assert np.array_equal(cache.plane_floats(), cold.plane_floats())
        err = rel_l1(host(lg), host(lg2))

        def run_oracle(arrs, suffix=suffix):
            x = oracle.Model(m, w)
            x.set_kv(arrs[1:], P0)
            x.verify_batch(np.concatenate([prefix, suffix]).astype(np.int32))
            x.commit_verify_rows(40 + len(suffix))
            return x.verify_embedded(arrs[0])

        tol = logits_bar(err, m, run_oracle, [embed_rows(w, vt)] + kv, f"prefix cache vs cold, suffix {ns}")
        assert err < tol
        cache.commit_verify_rows(0)


def test_prefill_refusals(setup):
    m, w, kv = setup
    g = gpu_model(m, w, kv)
    toks = synth.tokens(0, "prefill.refuse", 8, m.vocab)
    lg = torch.empty((8, m.vocab), dtype=torch.float32, device="cuda")
    g.verify_batch(dev(toks), lg, None)
    with pytest.raises(bvf.BvfError):          # a verify is pending
        g.prefill(dev(toks))
    g.commit_verify_rows(8)
    big = np.zeros(m.max_ctx, dtype=np.int32)
    with pytest.raises(bvf.BvfError):          # beyond max_ctx
        g.prefill(dev(big))
    assert g.positions_held() == P0 + 8       # refusals change nothing


def test_snapshot_update_reuses_the_snapshot(setup):
    """bvf_snapshot_update refreshes a snapshot in place: take one at 24 + 60 positions, prefill 20
    more, update it at 24 + 80 positions -- refused (more rows than it was taken with, snapshot
    unchanged) --, restore it, cut back by a verify and commit(0) to a smaller state, update it
    there, prefill something else, restore: the planes and the next verify equal those of a model
    that reached the same state directly (bit for bit), counts follow the update; refused while a
    verify is pending; on ring planes as well."""
    import dataclasses
    for ring in (0, 1):
        m, w, kv = setup
        m = dataclasses.replace(m, kv_ring=ring)
        g = gpu_model(m, w, kv)
        pre = synth.tokens(0, "upd.pre", 60, m.vocab)
        g.prefill(dev(pre))
        snap = g.snapshot_take()
        f60 = snap.floats().copy()
        g.prefill(dev(synth.tokens(1, "upd.more", 20, m.vocab)))
        with pytest.raises(bvf.BvfError) as e:            # the full layers' planes outgrew the snapshot
            g.snapshot_update(snap)
        assert e.value.status == bvf.BVF_E_CAPACITY
        assert np.array_equal(snap.floats(), f60)
        g.restore(snap)
        assert g.positions_held() == P0 + 60
        # a smaller committed state: 24 + 45 via a fresh model's prefill of the first 45 tokens
        ref = gpu_model(m, w, kv)
        ref.prefill(dev(pre[:45]))
        small = gpu_model(m, w, kv)
        small.prefill(dev(pre[:45]))
        small.snapshot_update(snap)                        # taken by another model of the same shape
        assert np.array_equal(snap.floats(), small.plane_floats())
        lg = torch.empty((8, m.vocab), dtype=torch.float32, device="cuda")
        small.verify_batch(dev(synth.tokens(2, "upd.v", 8, m.vocab)), lg, None)
        with pytest.raises(bvf.BvfError) as e:             # a verify is pending
            small.snapshot_update(snap)
        assert e.value.status == bvf.BVF_E_STATE
        small.commit_verify_rows(0)
        g.prefill(dev(synth.tokens(3, "upd.other", 5, m.vocab)))
        g.restore(snap)
        assert g.positions_held() == ref.positions_held() == P0 + 45
        assert np.array_equal(g.plane_floats(), ref.plane_floats())
        for l in range(m.n_layers):
            if m.own(l):
                assert np.array_equal(g.get_kv(l, P0 + 45), ref.get_kv(l, P0 + 45), equal_nan=True), f"ring {ring} layer {l}"
        vt = synth.tokens(4, "upd.next", 8, m.vocab)
        a, b = (torch.empty((8, m.vocab), dtype=torch.float32, device="cuda") for _ in range(2))
        g.verify_batch(dev(vt), a, None)
        ref.verify_batch(dev(vt), b, None)
        assert np.array_equal(host(a), host(b))

"""GPU parity of the verify pass on models with per-layer embeddings (PLE), through the C ABI: the
per-row per-layer inputs gathered by token id, the PLE gate and projection as M-row GEMMs and the
layer scalar (engine PR #2303, "What changes"), against the CPU oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import GEMM_TOL, build_pair, compare_taps, dev, host, logits_bar, run_verify
from tests.util import rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def ple_tiny(n_layers=1):
    return dataclasses.replace(synth.tiny_model(n_layers=n_layers), ple_dim=128, name="tinyple",
                               tap_layers=tuple(range(n_layers)))


def ple_two_width():
    return dataclasses.replace(synth.tiny_two_width_model(), ple_dim=128, name="tiny2wple")


def _oracle_on_tokens(m, w, kv, P, toks):
    """run(arrs) for the stack bar: the oracle's verify of toks on perturbed cached K/V (PLE models
    take token ids, so only the cached rows are perturbed)."""
    def run(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs, P)
        return x.verify_batch(toks)
    return run


@pytest.mark.parametrize("mk, P, k", [(ple_tiny, 64, 8), (ple_tiny, 7, 5), (ple_two_width, 40, 8), (ple_two_width, 3, 16)])
def test_ple_verify_parity(mk, P, k):
    m = mk()
    g, o, w, kv = build_pair(m, P)
    toks = synth.tokens(0, f"ple.verify.{m.name}.{k}", k, m.vocab)
    lg, taps = run_verify(g, m, toks)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)
    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, _oracle_on_tokens(m, w, kv, P, toks), kv, f"PLE verify P={P} k={k}")
    assert err < tol
    compare_taps(taps, rtaps, tol)
    assert g.positions_held() == o.held() == P + k
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    for i in range(k):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert lg[i].argmax() == rlg[i].argmax()


def test_ple_graph_replay_and_prefill():
    """The captured pass of a PLE model replays bit-identically to direct launches; a chunked
    prefill of 21 tokens (one chunk of two row tiles, its RMSNorms as their own kernel) leaves the
    context the oracle leaves."""
    m = ple_two_width()
    g, o, w, kv = build_pair(m, 12)
    toks = synth.tokens(0, "ple.graph", 8, m.vocab)
    lg_direct, _ = run_verify(g, m, toks, with_taps=False)
    g.commit_verify_rows(0)
    g.set_graph_mode(True)
    for _ in range(3):
        lg_graph, _ = run_verify(g, m, toks, with_taps=False)
        g.commit_verify_rows(0)
        assert np.array_equal(lg_graph, lg_direct)
    g.set_graph_mode(False)
    pt = synth.tokens(0, "ple.prefill", 21, m.vocab)
    g.prefill(dev(pt))
    o.verify_batch(pt)
    o.commit_verify_rows(21)
    assert g.positions_held() == o.held() == 33
    vt = synth.tokens(1, "ple.prefill.next", 4, m.vocab)
    lg, _ = run_verify(g, m, vt, with_taps=False)
    rv = o.verify_batch(vt)

    def run(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs, 12)
        x.verify_batch(pt)
        x.commit_verify_rows(21)
        return x.verify_batch(vt)

    err = rel_l1(lg, rv)
    assert err < logits_bar(err, m, run, kv, "PLE prefill 21, next verify")


def test_ple_refusals():
    """Injected rows are refused on a PLE model (the per-layer inputs need token ids); PLE tensors
    are refused on a model without per-layer embeddings; a pass before the PLE weights are loaded
    is refused; each refusal leaves the state unchanged."""
    m = ple_tiny()
    g = bvf.Model(m)
    w = synth.make_weights(m, 0)
    lg = torch.empty((2, m.vocab), dtype=torch.float32, device="cuda")
    t = dev(np.array([1, 2], dtype=np.int32))
    g.set_positions(0)
    with pytest.raises(bvf.BvfError) as e:
        g.verify_batch(t, lg)
    assert e.value.status == bvf.BVF_E_STATE
    g.load_weights(w)
    x = torch.zeros((2, m.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(bvf.BvfError) as e:
        g.layer_forward(0, x, 2)
    assert e.value.status == bvf.BVF_E_INVALID
    assert g.positions_held() == 0
    plain = bvf.Model(synth.tiny_model())
    with pytest.raises(bvf.BvfError) as e:
        plain.load_q4_1(0, bvf.PLE_GATE, w["layers"][0]["ple_gate"])
    assert e.value.status == bvf.BVF_E_INVALID
    with pytest.raises(bvf.BvfError) as e:
        plain.load_bf16(bvf.PLE_TABLE, 0, w["ple_table"])
    assert e.value.status == bvf.BVF_E_INVALID


def test_ple_gemms_bit_level():
    """The PLE gate and projection matrices through the kernel-level GEMM entry point, at 8 and 3
    rows, against the oracle's Q4_1 product (fp32 accumulation order)."""
    m = ple_two_width()
    g, o, w, kv = build_pair(m, 4)
    for l in (0, 5):
        for key in ("ple_gate", "ple_proj"):
            n_out, n_in = synth.layer_matrix_shapes(m, l)[key]
            for rows in (8, 3):
                x = synth.bf16_normal(rows, f"ple.gemm.{l}.{key}", (rows, n_in))
                y = torch.empty((rows, n_out), dtype=torch.float32, device="cuda")
                g.q4_1_gemm(l, bvf.MATRIX_IDS[key], dev(x), rows, y)
                ref = oracle.q4_1_matmul(w["layers"][l][key], n_out, n_in, x)
                assert rel_l1(host(y), ref) < GEMM_TOL


def test_ple_full_size_target():
    """The target-shaped stack (42 layers, hidden 2560, 1024 cached positions) with per-layer
    embeddings of width 256 (Gemma4-E4B's per-layer width) and a 16384-entry vocabulary (the
    per-layer table is vocab x 42 x 256 bf16): k = 8 verify against the oracle, fixed 2e-3 bar."""
    P = 1024
    m = dataclasses.replace(synth.target_model(max_ctx=P + 64, vocab=16384), ple_dim=256)
    w = synth.make_weights(m, 0, threads=16)
    kv = synth.make_kv(m, P, 0, threads=16)
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, P)
    toks = synth.tokens(0, "ple.full", 8, m.vocab)
    print("[ple full size] target 42 layers, ple_dim 256, vocab 16384, k=8", flush=True)
    lg, taps = run_verify(g, m, toks)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)
    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, None, None, "full-size target with PLE, k=8")
    assert err < tol
    compare_taps(taps, rtaps, tol)

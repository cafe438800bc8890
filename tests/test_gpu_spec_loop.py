"""The speculative loop (draft block -> batched verify -> greedy accept -> commit) on the GPU against
the oracle running the same rounds, on a small target with two attention widths and KV-shared
layers plus its small draft; and, without steering, the loop's output against plain greedy decoding
(one row per step) on the GPU."""
import dataclasses

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from block_verify_forward_amd.loop import SpecLoop
from tests.test_gpu_parity import dev, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

P0 = 24
BLOCK = 8
BONUS = 1.0e4


def models():
    tm = synth.tiny_two_width_model(max_ctx=160)
    dm = synth.tiny_draft_model(max_ctx=160, n_taps=len(tm.tap_layers), window=32)
    tw = synth.make_weights(tm)
    dw = synth.make_weights(dm)
    kv = synth.make_kv(tm, P0)
    kvd = synth.make_kv(dm, P0)
    return tm, dm, tw, dw, kv, kvd


def gpu_pair(tm, dm, tw, dw, kv, kvd):
    T = bvf.Model(tm)
    T.load_weights(tw)
    T.set_context(kv, P0)
    D = bvf.Model(dataclasses.replace(dm, vocab=tm.vocab))
    D.load_weights(dw)
    D.set_context(kvd, P0)
    return T, D


def margin_clear(row):
    """The row's top-2 margin is clear (the near-tie reading: more than 0.02 of the row's rms)."""
    top2 = np.sort(row)[-2:]
    return top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(row.astype(np.float64) ** 2))


def test_spec_loop_matches_oracle_with_steering():
    """Ten steered rounds. The oracle is teacher-forced with the GPU's tokens each round (so one
    near-tie cannot make the two runs diverge) and every decision is compared where its margin is
    clear: the draft's proposals, the accepted length (exact: steered), the emitted tokens."""
    tm, dm, tw, dw, kv, kvd = models()
    T, D = gpu_pair(tm, dm, tw, dw, kv, kvd)
    To = oracle.Model(tm, tw)
    To.set_kv(kv, P0)
    Do = oracle.Model(dm, dw)
    Do.set_kv(kvd, P0)
    steer = synth.accept_lengths(0, 10, max_a=BLOCK - 1)
    loop = SpecLoop(T, D, BLOCK, steer_bonus=BONUS)
    last = 17
    loop.start(last)
    taps_rows = None
    compared = 0
    for r, a_want in enumerate(steer):
        a_want = int(a_want)
        a, emitted = loop.round(a_want)
        gtoks = host(loop.toks)                      # [last, GPU proposals]
        if taps_rows is not None:
            Do.draft_append(taps_rows)
        rprops, dlg = Do.draft_block(To, BLOCK, last, 1.0, tm.vocab - 1, with_logits=True)
        for i in range(BLOCK - 1):
            if margin_clear(dlg[i]):
                assert gtoks[i + 1] == rprops[i], f"round {r} proposal {i}"
                compared += 1
        toks = np.concatenate([[last], gtoks[1:]]).astype(np.int32)
        lg, taps = To.verify_batch(toks, with_taps=True)
        for m in range(a_want):
            lg[m, toks[m + 1]] += BONUS
        if a_want < BLOCK - 1:
            lg[a_want, toks[a_want + 1]] -= BONUS
        ra, remitted = oracle.accept_greedy(lg, toks)
        assert a == ra == a_want, f"round {r}"
        assert emitted[:a] == toks[1:a + 1].tolist()
        if margin_clear(lg[a]):
            assert emitted[a] == remitted[a], f"round {r}: the target's own token"
            compared += 1
        To.commit_verify_rows(a + 1)
        assert T.positions_held() == To.held()
        taps_rows = taps[: a + 1]
        last = emitted[a]
    assert compared >= 40
    assert T.positions_held() == P0 + int(np.sum(steer)) + len(steer)
    assert D.positions_held() == P0 + int(np.sum(steer[:-1])) + len(steer) - 1


def test_spec_loop_equals_greedy_decoding():
    """Without steering the speculative output is the target's own greedy continuation, whatever
    the draft proposes: each of the loop's first 24 tokens is the greedy token of a plain one-row
    step fed the loop's previous tokens (compared where the step's margin is clear)."""
    tm, dm, tw, dw, kv, kvd = models()
    T, D = gpu_pair(tm, dm, tw, dw, kv, kvd)
    loop = SpecLoop(T, D, BLOCK)
    loop.start(17)
    spec = loop.run(24)[:24]

    T2, _ = gpu_pair(tm, dm, tw, dw, kv, kvd)
    tok = dev(np.array([17], dtype=np.int32))
    lg = torch.empty((1, tm.vocab), dtype=torch.float32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    To = oracle.Model(tm, tw)
    To.set_kv(kv, P0)
    compared = 0
    prev = 17
    for i in range(24):
        T2.verify_batch(tok, lg, None)
        T2.accept_greedy(lg, tok, out, n_acc)
        T2.commit_verify_rows(1)
        lgo = To.verify_batch(np.array([prev], dtype=np.int32))
        To.commit_verify_rows(1)
        if margin_clear(lgo[0]):
            assert int(host(out)[0]) == spec[i] == int(np.argmax(lgo[0])), f"step {i}"
            compared += 1
        prev = spec[i]
        tok.copy_(dev(np.array([prev], dtype=np.int32)))
    assert compared >= 12


def test_spec_loop_sampled_matches_oracle():
    """Eight rounds at temperature 0.8 without steering. Per round the oracle, teacher-forced with the
    rows the GPU verified ([last token, the GPU draft's proposals]), computes the logits and draws
    with the same key and counter offset (the round number). Each row's draw is compared where the
    oracle's perturbed-score margin clears the logits' rounding differences; the accepted length and
    the emitted tokens where every draw they depend on was compared."""
    T_, SEED = 0.8, 31337
    tm, dm, tw, dw, kv, kvd = models()
    T, D = gpu_pair(tm, dm, tw, dw, kv, kvd)
    To = oracle.Model(tm, tw)
    To.set_kv(kv, P0)
    loop = SpecLoop(T, D, BLOCK, temperature=T_, seed=SEED)
    last = 17
    loop.start(last)
    compared_draws = compared_a = 0
    for r in range(8):
        a, emitted = loop.round()
        rows = np.concatenate([[last], host(loop.toks)[1:]]).astype(np.int32)
        draws = host(loop.draws)
        lg = To.verify_batch(rows)
        ra, remitted, rdraws = oracle.accept_sampled(lg, rows, T_, SEED, r)
        clear = []
        for i in range(BLOCK):
            sc = oracle.sample_scores(lg[i], T_, SEED, r, i)
            top = np.sort(sc)[-2:]
            bar = 0.02 * np.sqrt(np.mean(lg[i].astype(np.float64) ** 2)) / T_
            clear.append(bool(top[1] - top[0] > bar))
            if clear[-1]:
                assert draws[i] == rdraws[i], f"round {r} row {i}"
                compared_draws += 1
        if all(clear[: max(a, ra) + 1]):
            assert a == ra and emitted == remitted.tolist(), f"round {r}"
            compared_a += 1
        To.commit_verify_rows(a + 1)
        assert T.positions_held() == To.held()
        last = emitted[a]
    assert compared_draws >= 40 and compared_a >= 4


def test_spec_loop_graphs_equal_direct_launches():
    """Twelve steered rounds with both models replayed from graphs (the verify pass and the draft
    block) give the same proposals, accepted lengths and emitted tokens as direct launches, bit for
    bit, and the draft takes one capture per context-row count it met."""
    tm, dm, tw, dw, kv, kvd = models()
    steer = synth.accept_lengths(1, 12, max_a=BLOCK - 1)
    runs = []
    for graph in (False, True):
        T, D = gpu_pair(tm, dm, tw, dw, kv, kvd)
        T.set_graph_mode(graph)
        D.set_graph_mode(graph)
        loop = SpecLoop(T, D, BLOCK, steer_bonus=BONUS)
        loop.start(17)
        rounds = []
        for a_want in steer:
            a, emitted = loop.round(int(a_want))
            rounds.append((a, emitted, host(loop.toks).tolist(), host(loop.logits)))
        runs.append((rounds, D.graph_captures(), T.positions_held(), D.positions_held()))
    (rd, cd, td, dd), (rg, cg, tg_, dg) = runs
    for r, (x, y) in enumerate(zip(rd, rg)):
        assert x[0] == y[0] and x[1] == y[1] and x[2] == y[2], f"round {r}"
        assert np.array_equal(x[3], y[3]), f"round {r} verify logits"
    assert (td, dd) == (tg_, dg)
    n_news = {0} | {int(a) + 1 for a in steer[:-1]}
    print(f"[loop graphs] draft captures {cg} for context-row counts {sorted(n_news)}", flush=True)
    assert cd == 0 and cg == len(n_news)

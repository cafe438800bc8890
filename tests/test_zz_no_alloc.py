"""The allocation-free greedy accept (bvf_accept_greedy_static) against the model entry point
bvf_accept_greedy and the oracle's accept, through the C ABI: two calls in a row on the same GPU,
the second with fewer rows and a smaller vocabulary (the array keeps the first call's contents),
then the refusals."""
import dataclasses

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _logits_and_drafts(k, V, accept, seed):
    """Random logits [k][V] and drafts that match the argmax of rows 0..accept-1, then mismatch."""
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((k, V)).astype(np.float32)
    y = lg.argmax(axis=1)
    toks = rng.integers(0, V, size=k).astype(np.int32)
    for m in range(1, k):
        toks[m] = y[m - 1] if m <= accept else (y[m - 1] + 1) % V
    return lg, toks


def _model_accept(vocab, lg, toks):
    m = dataclasses.replace(synth.tiny_model(max_ctx=8), vocab=vocab)
    g = bvf.Model(m)
    out = torch.zeros(len(toks), dtype=torch.int32, device="cuda")
    na = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.accept_greedy(torch.from_numpy(lg).cuda(), torch.from_numpy(toks).cuda(), out, na)
    torch.cuda.synchronize()
    a = int(na.cpu()[0])
    return a, out.cpu().numpy()[: a + 1]


def _static_accept(lg, toks):
    out = torch.full((len(toks),), -7, dtype=torch.int32, device="cuda")
    na = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    bvf.accept_greedy_static(torch.from_numpy(lg).cuda(), torch.from_numpy(toks).cuda(), out, na)
    torch.cuda.synchronize()
    a = int(na.cpu()[0])
    return a, out.cpu().numpy()[: a + 1]


def test_static_accept_matches_model_accept_on_two_calls():
    assert torch.cuda.is_available()
    cases = [(16, 262144, 9, 0), (3, 1040, 1, 1)]      # the second call: fewer rows, smaller vocabulary
    for k, V, accept, seed in cases:
        print(f"[no-alloc accept] k={k} vocab={V} constructed accept={accept}", flush=True)
        lg, toks = _logits_and_drafts(k, V, accept, seed)
        got = _static_accept(lg, toks)
        ref = _model_accept(V, lg, toks)
        ora, oemit = oracle.accept_greedy(lg, toks)
        assert got[0] == ref[0] == ora == accept
        assert np.array_equal(got[1], ref[1]) and np.array_equal(got[1], oemit)


def test_static_accept_refusals():
    lg = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    toks = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = torch.zeros(2, dtype=torch.int32, device="cuda")
    na = torch.zeros(1, dtype=torch.int32, device="cuda")
    big = torch.zeros((17, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(bvf.BvfError) as e:
        bvf.accept_greedy_static(big, torch.zeros(17, dtype=torch.int32, device="cuda"), out, na)
    assert e.value.status == bvf.BVF_E_INVALID
    with pytest.raises(bvf.BvfError) as e:     # refused before anything is enqueued
        bvf._check(bvf.lib().bvf_accept_greedy_static(lg.data_ptr(), 2, (1 << 20) + 16, toks.data_ptr(),
                                                       out.data_ptr(), na.data_ptr(), None))
    assert e.value.status == bvf.BVF_E_CAPACITY

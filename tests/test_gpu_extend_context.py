"""GPU parity of extend_context through the C ABI ([PR2303] "What changes" item 1: the KV count of
extend_context is per layer): n new positions are appended to every own plane at the held count at
that layer's own width, shared planes stay empty, and a model extended from 5 to 8 positions is the
model that cached all 8 from the start (planes bit-exact, the next verify bit-identical, and within
the stack bar of the oracle's extend path). Refusals leave the state unchanged."""
import dataclasses

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import dev, host, logits_bar, embed_rows
from tests.util import rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _model(kv_bf16: int):
    m = synth.tiny_two_width_model()
    return dataclasses.replace(m, kv_bf16=kv_bf16) if kv_bf16 else m


@pytest.mark.parametrize("kv_bf16", [0, 1])
def test_extend_context_equals_cached_context(kv_bf16):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m = _model(kv_bf16)
    w = synth.make_weights(m, 0)
    kv8 = synth.make_kv(m, 8, 0)
    new = [None if kv is None else kv[5:8] for kv in kv8]
    A = bvf.Model(m); A.load_weights(w); A.set_context(kv8, 5)
    A.extend_context(new, 3)
    B = bvf.Model(m); B.load_weights(w); B.set_context(kv8, 8)
    o = oracle.Model(m, w); o.set_kv(kv8, 5)
    assert o.extend_context(new, 3) == 0
    assert A.positions_held() == B.positions_held() == o.held() == 8
    assert np.array_equal(A.plane_floats(), o.plane_floats())
    for l in range(m.n_layers):
        if m.layers[l].kv_owner < 0:
            got = A.get_kv(l, 8)
            assert np.array_equal(got, B.get_kv(l, 8)), f"plane {l}"
            if not kv_bf16:
                assert np.array_equal(got, kv8[l][:8]), f"plane {l}"
    # the next verify: bit-identical to the model that cached 8 positions, and the oracle's
    toks = synth.tokens(0, "extend.toks", 4, m.vocab)
    lgA = torch.empty((4, m.vocab), dtype=torch.float32, device="cuda")
    lgB = torch.empty_like(lgA)
    A.verify_batch(dev(toks), lgA, None)
    B.verify_batch(dev(toks), lgB, None)
    a, b = host(lgA), host(lgB)
    assert np.array_equal(a, b)
    ref = o.verify_batch(toks)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], 8)
        return x.verify_embedded(arrs[0])

    err = rel_l1(a, ref)
    tol = logits_bar(err, m, run_oracle, [embed_rows(w, toks)] + kv8, f"extend_context kv_bf16={kv_bf16}")
    assert err < tol, f"rel-L1 {err:.2e} >= {tol:.2e}"
    A.commit_verify_rows(2)
    assert A.positions_held() == 10


def test_extend_context_refusals_leave_state():
    m = _model(0)
    w = synth.make_weights(m, 0)
    kv8 = synth.make_kv(m, 8, 0)
    new = [None if kv is None else kv[5:8] for kv in kv8]
    A = bvf.Model(m); A.load_weights(w); A.set_context(kv8, 5)
    toks = synth.tokens(0, "extend.refuse", 2, m.vocab)
    lg = torch.empty((2, m.vocab), dtype=torch.float32, device="cuda")
    A.verify_batch(dev(toks), lg, None)
    planes = {l: A.get_kv(l, 7) for l in range(m.n_layers) if m.layers[l].kv_owner < 0}
    with pytest.raises(bvf.BvfError) as e:
        A.extend_context(new, 3)                       # a verify is pending
    assert e.value.status == bvf.BVF_E_STATE
    assert A.positions_held() == 7
    for l, p in planes.items():
        assert np.array_equal(A.get_kv(l, 7), p)
    A.commit_verify_rows(0)
    big = [None if kv is None else np.zeros((m.max_ctx, 2, kv.shape[2]), np.float32) for kv in kv8]
    with pytest.raises(bvf.BvfError) as e:
        A.extend_context(big, m.max_ctx - 4)           # past max_ctx
    assert e.value.status == bvf.BVF_E_CAPACITY
    assert A.positions_held() == 5
    A.extend_context(new, 0)                           # nothing to append
    assert A.positions_held() == 5

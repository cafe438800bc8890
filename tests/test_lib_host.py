"""Host-side checks of the HIP library (no GPU needed): it loads, exports every symbol the header
declares, and its host-only rules (descriptor checks, per-plane cut arithmetic) hold."""
import dataclasses
import os
import re

import pytest

from block_verify_forward_amd import bvf, synth
from tests.util import golden

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "bvf.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bvf_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = bvf.lib()
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), f"{n} declared in bvf.h but not exported"
    assert set(names) == set(bvf.SIGNATURES), "binding signatures and header disagree"


def test_cut_floats_rule():
    g = golden("cut_arithmetic")
    assert bvf.cut_floats([g["width"]], 0, g["positions"]) == g["floats"]
    per = [256, 512, 128]
    for plane in range(5):
        assert bvf.cut_floats(per, plane, 9) == 9 * 2 * per[min(plane, 2)]
    assert bvf.lib().bvf_cut_floats(None, 0, 0, 5) == -1


def test_arena_bytes_for_the_configs():
    for m in (synth.tiny_model(), synth.tiny_two_width_model(), synth.target_model(max_ctx=1100),
              synth.draft_model()):
        assert bvf.arena_bytes(m) > 0, bvf.last_error()
    # the target's arena holds at least its packed weights, head and planes
    m = synth.target_model(max_ctx=1100)
    planes = sum(m.max_ctx * 2 * m.kv_width(l) * 4 for l in range(m.n_layers) if m.own(l))
    assert bvf.arena_bytes(m) > synth.q4_1_bytes(m) + m.vocab * m.hidden * 2 + planes


@pytest.mark.parametrize("change, msg", [
    (dict(hidden=200), "hidden"),
    (dict(vocab=1000), "vocab"),
    (dict(max_ctx=0), "max_ctx"),
    (dict(tap_layers=(7,)), "tap layer"),
])
def test_descriptor_refusals(change, msg):
    m = dataclasses.replace(synth.tiny_model(), **change)
    with pytest.raises(bvf.BvfError) as e:
        bvf.arena_bytes(m)
    assert msg in str(e.value)


def test_layer_refusals():
    base = synth.tiny_two_width_model()
    bad_owner = list(base.layers)
    bad_owner[4] = dataclasses.replace(bad_owner[4], kv_owner=2)     # sliding layer owned by a full one
    with pytest.raises(bvf.BvfError, match="another attention type"):
        bvf.arena_bytes(dataclasses.replace(base, layers=tuple(bad_owner)))
    fwd = list(base.layers)
    fwd[1] = dataclasses.replace(fwd[1], kv_owner=3)
    with pytest.raises(bvf.BvfError, match="not an earlier layer"):
        bvf.arena_bytes(dataclasses.replace(base, layers=tuple(fwd)))
    hd = list(base.layers)
    hd[0] = dataclasses.replace(hd[0], head_dim=96)
    with pytest.raises(bvf.BvfError, match="head_dim"):
        bvf.arena_bytes(dataclasses.replace(base, layers=tuple(hd)))


def test_arena_bytes_for_the_variants():
    """Every model shape the tests and the benchmark build: per-layer embeddings, ring planes, bf16
    planes, the ragged model, the tiny draft; the ring arena is smaller than the linear one."""
    from tests.test_gpu_parity import ragged_model
    tgt = synth.target_model(max_ctx=16384 + 64)
    models = [dataclasses.replace(synth.tiny_model(), ple_dim=128), dataclasses.replace(tgt, ple_dim=256, vocab=16384),
              dataclasses.replace(tgt, kv_ring=1), dataclasses.replace(tgt, kv_bf16=1),
              dataclasses.replace(synth.tiny_two_width_model(), kv_ring=1, kv_bf16=1), ragged_model(),
              synth.tiny_draft_model(), dataclasses.replace(synth.draft_model(), kv_bf16=1)]
    for m in models:
        assert bvf.arena_bytes(m) > 0, (m.name, bvf.last_error())
    assert bvf.arena_bytes(dataclasses.replace(tgt, kv_ring=1)) < bvf.arena_bytes(tgt)
    assert bvf.arena_bytes(dataclasses.replace(tgt, kv_bf16=1)) < bvf.arena_bytes(tgt)


@pytest.mark.parametrize("change, msg", [
    (dict(ple_dim=100), "ple_dim"),
    (dict(ple_dim=8192), "ple_dim"),
    (dict(kv_ring=2), "kv_ring"),
    (dict(kv_bf16=3), "kv_bf16"),
    (dict(max_ctx=(1 << 24) + 1), "max_ctx"),
    (dict(rope_base=0.0), "rope_base"),
])
def test_descriptor_refusals_more(change, msg):
    m = dataclasses.replace(synth.tiny_model(), **change)
    with pytest.raises(bvf.BvfError) as e:
        bvf.arena_bytes(m)
    assert msg in str(e.value)


def test_kv_heads_must_divide_the_query_heads():
    m = synth.tiny_model()
    m = dataclasses.replace(m, n_q_heads=6, layers=(dataclasses.replace(m.layers[0], n_kv_heads=4),))
    with pytest.raises(bvf.BvfError, match="does not divide"):
        bvf.arena_bytes(m)


def test_draft_refusals():
    d = synth.tiny_draft_model()
    for change, msg in [(dict(ple_dim=128), "verify model only"), (dict(kv_ring=1), "verify model only"),
                        (dict(tap_layers=()), "n_taps")]:
        with pytest.raises(bvf.BvfError) as e:
            bvf.arena_bytes(dataclasses.replace(d, **change))
        assert msg in str(e.value)
    shared = list(d.layers)
    shared[1] = dataclasses.replace(shared[1], kv_owner=0)
    with pytest.raises(bvf.BvfError, match="cannot share"):
        bvf.arena_bytes(dataclasses.replace(d, layers=tuple(shared)))

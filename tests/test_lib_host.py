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

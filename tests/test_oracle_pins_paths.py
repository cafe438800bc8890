"""Pins of the oracle's q/k path and of the draft forward by hand cases with closed forms, and the
agreement of the oracle with an independent numpy float64 twin. No GPU; no HIP library.

Each hand case is built so that a plausible mistake changes a checked value:
  - q/k path: swapped q/k norm gains, a missing per-head RMSNorm, queries or keys rotated at the
    wrong position;
  - draft context append: the tap concatenation order, a transposed fc, a skipped hidden norm,
    context keys rotated at the wrong position;
  - draft block: the target's final norm used in place of the draft's, the head run over the
    wrong block rows, the embedding scale dropped.
"""
import math

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import synth
from tests.numpy_twin import Twin
from tests.util import rel_l1, zero_q4, zero_weights


def _q4_from_entries(n_out: int, n_in: int, entries):
    """Q4_1 image whose only nonzero weights are the given {(row, col): value}. Each value must be
    a small integer code times an fp16 scale: value = scale * code with code in 1..15 (min 0)."""
    nb = n_in // 32
    codes = np.zeros((n_out, n_in), dtype=np.int64)
    scale = np.zeros((n_out, nb))
    for (r, c), v in entries.items():
        code = 1
        for cand in range(15, 0, -1):   # the largest code whose scale is exact in fp16
            s = v / cand
            if float(np.float16(s)) == s:
                code = cand
                break
        s = v / code
        assert float(np.float16(s)) == s, "hand value not representable as fp16 scale x code"
        assert scale[r, c // 32] in (0.0, s), "one scale per block"
        scale[r, c // 32] = s
        codes[r, c] = code
    return synth.q4_1_from_parts(codes, scale, np.zeros((n_out, nb)))


def _bf16(v):
    return float(synth.bf16_to_f32(synth.bf16_bits(np.float64(v))))


def _f32(v):
    return float(np.float32(v))


def _bits(v):
    return synth.bf16_bits(np.asarray(v, dtype=np.float64))


# ------------------------------------------------------------------------------------------
# q/k path of a verify layer: per-head RMSNorm with the q and k gains, RoPE at the row position
# ------------------------------------------------------------------------------------------
def test_qk_path_closed_form():
    """One row at position p = 1 over one cached position. Hidden 256, 4 query heads and one KV head
    of 64 dims. x = 1 with a unit attention gain gives a = 1, so each projection row's output is its
    weight sum: q head 0 = c e0, k = d e0, v = g e1; query heads 1..3 are zero. The cached key at
    position 0 is b e32 (already rotated), its value e0. With RMSNorm gains gq (q) and gk (k) at
    dimension 0 and rotate-half RoPE (dimension 0 pairs with 32, angle p):
        qn = c gq / sqrt(c^2/64 + eps),  q' = (qn cos p) e0 + (qn sin p) e32
        kn = d gk / sqrt(d^2/64 + eps),  k' = (kn cos p) e0 + (kn sin p) e32   (appended at p)
        s0 = q' . (b e32) / 8,  s1 = q' . k' / 8,  w0 = 1 / (1 + exp(s1 - s0))
    Head 0 then outputs w0 e0 + (1 - w0) g e1; heads 1..3 see equal scores and output (e0 + g e1)/2.
    An identity o projection and a zero MLP put bf16(o) on top of x."""
    m = synth.tiny_model(max_ctx=8)
    w = zero_weights(m)
    L = w["layers"][0]
    H, hd = 256, 64
    c, d, g, b = 3.0, 2.0, 5.0, 4.0
    gq0, gk0 = 1.5, 0.75
    L["attn_norm"] = _bits(np.ones(H))
    qn_g = synth.bf16_to_f32(L["q_norm"]).astype(np.float64); qn_g[0] = gq0
    kn_g = synth.bf16_to_f32(L["k_norm"]).astype(np.float64); kn_g[0] = gk0
    L["q_norm"], L["k_norm"] = _bits(qn_g), _bits(kn_g)
    L["q"] = _q4_from_entries(H, H, {(0, 0): c})
    L["k"] = _q4_from_entries(hd, H, {(0, 0): d})
    L["v"] = _q4_from_entries(hd, H, {(1, 0): g})
    L["o"] = _q4_from_entries(H, H, {(i, i): 1.0 for i in range(H)})
    om = oracle.Model(m, w)
    kv = np.zeros((1, 2, hd), dtype=np.float32)
    kv[0, 0, 32] = b
    kv[0, 1, 0] = 1.0
    om.set_kv([kv], 1)
    p, eps = 1, m.rms_eps
    x = np.ones(H, dtype=np.float32)
    out = om.layer_forward(0, x, [p])[0].astype(np.float64)

    qn = c * gq0 / math.sqrt(c * c / hd + eps)
    kn = d * gk0 / math.sqrt(d * d / hd + eps)
    q0, q32 = _f32(qn * math.cos(p)), _f32(qn * math.sin(p))
    k0, k32 = _f32(kn * math.cos(p)), _f32(kn * math.sin(p))
    s0 = q32 * b / 8.0
    s1 = (q0 * k0 + q32 * k32) / 8.0
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    expect = np.ones(H)
    expect[0] = _f32(1.0 + _bf16(w0))
    expect[1] = _f32(1.0 + _bf16((1.0 - w0) * g))
    for h in range(1, 4):
        expect[h * hd] = 1.5
        expect[h * hd + 1] = _f32(1.0 + _bf16(g / 2.0))
    assert np.array_equal(out, expect), (out[:2], expect[:2])

    # the appended row at p: K normalised with the k gain and rotated at p, V as projected
    row = om.plane(0, 2)[1]
    kexp = np.zeros(hd); kexp[0], kexp[32] = k0, k32
    vexp = np.zeros(hd); vexp[1] = g
    assert np.array_equal(row[0].astype(np.float64), kexp)
    assert np.array_equal(row[1].astype(np.float64), vexp)


def test_qk_path_relative_position_of_two_new_rows():
    """Two rows at p = 4, 5 over four cached zero keys and values; both rows have x = 1, so
    q = e0, k = e0 and v = e2 before the norms. Row 1's score against row 0's appended key is
    q'(5) . k'(4) / 8 = qn kn cos(1) / 8 (dimension pair 0 turns by the position difference), and
    against its own key qn kn / 8; zero cached keys score 0. Row 1's head-0 output at dimension 2
    is the softmax weight on the two new keys (both values are e2)."""
    m = synth.tiny_model(max_ctx=8)
    w = zero_weights(m)
    L = w["layers"][0]
    H, hd = 256, 64
    L["attn_norm"] = _bits(np.ones(H))
    gq = synth.bf16_to_f32(L["q_norm"]).astype(np.float64)
    gk = synth.bf16_to_f32(L["k_norm"]).astype(np.float64)
    L["q"] = _q4_from_entries(H, H, {(0, 0): 1.0})
    L["k"] = _q4_from_entries(hd, H, {(0, 0): 1.0})
    L["v"] = _q4_from_entries(hd, H, {(2, 0): 1.0})
    L["o"] = _q4_from_entries(H, H, {(i, i): 1.0 for i in range(H)})
    om = oracle.Model(m, w)
    om.set_kv([np.zeros((4, 2, hd), dtype=np.float32)], 4)
    eps = m.rms_eps
    out = om.layer_forward(0, np.ones((2, H), dtype=np.float32), [4, 5]).astype(np.float64)
    qn = gq[0] / math.sqrt(1.0 / hd + eps)
    kn = gk[0] / math.sqrt(1.0 / hd + eps)
    def q_at(p):
        return _f32(qn * math.cos(p)), _f32(qn * math.sin(p))
    def k_at(p):
        return _f32(kn * math.cos(p)), _f32(kn * math.sin(p))
    qa, qb = q_at(5)
    ka, kb = k_at(4)
    kc, kd = k_at(5)
    s_prev = (qa * ka + qb * kb) / 8.0
    s_self = (qa * kc + qb * kd) / 8.0
    e = np.exp(np.array([0, 0, 0, 0, s_prev, s_self]) - max(0.0, s_prev, s_self))
    wts = e / e.sum()
    o2 = float(wts[4] + wts[5])            # both new values are e2
    assert out[1, 2] == _f32(1.0 + _bf16(o2))
    # row 0 at p = 4: its own key only among nonzero keys
    q4a, q4b = q_at(4)
    s_own = (q4a * ka + q4b * kb) / 8.0
    e0 = np.exp(np.array([0, 0, 0, 0, s_own]) - max(0.0, s_own))
    assert out[0, 2] == _f32(1.0 + _bf16(float(e0[4] / e0.sum())))
    # the closed form really depends on the position difference (cos 1 != 1)
    assert abs(s_prev - qn * kn * math.cos(1.0) / 8.0) < 1e-5 * abs(s_prev)


# ------------------------------------------------------------------------------------------
# draft: fc over the concatenated taps, hidden norm, context K/V at their positions
# ------------------------------------------------------------------------------------------
def _draft_case():
    dm = synth.tiny_draft_model(max_ctx=16, n_layers=1, n_taps=3, window=0)
    dw = synth.make_weights(dm)
    L = dw["layers"][0]
    for key, (n_out, n_in) in synth.layer_matrix_shapes(dm, 0).items():
        L[key] = zero_q4(n_out, n_in)
    return dm, dw


def test_draft_fc_append_closed_form():
    """fc has two nonzero entries, 1 at (row 7, tap 0 element 20) and 1 at (row 9, tap 2 element 20),
    so fc . concat(taps_j) = a_j e7 + b_j e9 with a_j = taps_j[0][20], b_j = taps_j[2][20]. The hidden
    norm (gains h7, h9) gives c = bf16(a h7 / r) e7 + bf16(b h9 / r) e9 with r = sqrt((a^2 + b^2)/256
    + eps). The layer's K projection picks c[7] into dimension 0 and V picks c[9] into dimension 2,
    so the context row at position j holds K = rope((c7 gk / sqrt(c7^2/64 + eps)) e0, j), V = c9 e2.
    Swapping the taps swaps a and b; a transposed fc or a skipped norm changes c7 and c9."""
    dm, dw = _draft_case()
    H, T, hd = 256, 3, 64
    fc = np.zeros((H, T * H)); fc[7, 0 * H + 20] = 1.0; fc[9, 2 * H + 20] = 1.0
    dw["fc"] = _bits(fc)
    gh = synth.bf16_to_f32(dw["hidden_norm"]).astype(np.float64); gh[7] = 1.25; gh[9] = 0.75
    dw["hidden_norm"] = _bits(gh)
    L = dw["layers"][0]
    L["k"] = _q4_from_entries(hd, H, {(0, 7): 1.0})
    L["v"] = _q4_from_entries(hd, H, {(2, 9): 1.0})
    gk0 = float(synth.bf16_to_f32(L["k_norm"])[0])
    taps = synth.bf16_normal(0, "pin.fc.taps", (2, T, H))
    ab = [(0.5, 2.0), (-1.0, 0.25)]
    for j in range(2):
        taps[j, 0, 20] = synth.bf16_bits(np.float64(ab[j][0]))
        taps[j, 2, 20] = synth.bf16_bits(np.float64(ab[j][1]))
    D = oracle.Model(dm, dw)
    D.draft_append(taps)
    plane = D.plane(0, 2).astype(np.float64)
    eps = dm.rms_eps
    for j in range(2):
        a, b = ab[j]
        r = math.sqrt((a * a + b * b) / H + eps)
        c7, c9 = _bf16(a * 1.25 / r), _bf16(b * 0.75 / r)
        kn = c7 * gk0 / math.sqrt(c7 * c7 / hd + eps)
        kexp = np.zeros(hd); kexp[0], kexp[32] = _f32(kn * math.cos(j)), _f32(kn * math.sin(j))
        vexp = np.zeros(hd); vexp[2] = c9
        assert np.array_equal(plane[j, 0], kexp), (j, plane[j, 0, [0, 32]], kexp[[0, 32]])
        assert np.array_equal(plane[j, 1], vexp), (j, plane[j, 1, 2], c9)


def test_draft_block_head_rows_closed_form():
    """All draft matrices zero: the layers add nothing, so block row i keeps x_i = fp32(E[tok_i] s)
    (tok_0 the last token, the others the mask). Rows 1..B-1 then give
    logits = E . bf16(rms(E[mask] s) g_final_draft): the draft's own final norm, the target's head.
    With s = 0.001 the mean square of x is near eps, so the scale shows through the norm."""
    tm = synth.tiny_model(max_ctx=32)
    tw = synth.make_weights(tm)
    dm, dw = _draft_case()
    dw["final_norm"] = synth.bf16_uniform(0, "pin.draft.final_norm", (dm.hidden,), 0.5, 1.5)
    for key in ("q", "k", "v", "o", "gate", "up", "down"):
        n_out, n_in = synth.layer_matrix_shapes(dm, 0)[key]
        dw["layers"][0][key] = zero_q4(n_out, n_in)
    T = oracle.Model(tm, tw)
    D = oracle.Model(dm, dw)
    D.draft_append(synth.bf16_normal(0, "pin.block.taps", (3, 3, dm.hidden)))
    s, last, mask, B = 0.001, 17, tm.vocab - 1, 6
    props, lg = D.draft_block(T, B, last, s, mask, with_logits=True)
    E = synth.bf16_to_f32(tw["embed"]).astype(np.float64)
    x = np.float32(E[mask] * s).astype(np.float64)
    a = synth.bf16_to_f32(synth.bf16_bits(x / np.sqrt(np.mean(x * x) + dm.rms_eps)
                                          * synth.bf16_to_f32(dw["final_norm"]).astype(np.float64))).astype(np.float64)
    expect = np.float32(E @ a).astype(np.float64)
    assert lg.shape == (B - 1, tm.vocab)
    for i in range(B - 1):
        np.testing.assert_allclose(lg[i].astype(np.float64), expect, rtol=2e-7, atol=1e-6)
        assert props[i] == int(np.argmax(expect))
    # the last token's row (block row 0) is not one of the head rows
    xl = np.float32(E[last] * s).astype(np.float64)
    al = synth.bf16_to_f32(synth.bf16_bits(xl / np.sqrt(np.mean(xl * xl) + dm.rms_eps)
                                           * synth.bf16_to_f32(dw["final_norm"]).astype(np.float64))).astype(np.float64)
    assert rel_l1(lg[0], E @ al) > 0.1


# ------------------------------------------------------------------------------------------
# two independent references agree (C oracle vs numpy twin)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("which", ["config1", "two_width"])
def test_numpy_twin_agrees_with_oracle(which):
    """The 1-layer decoder (hidden 256, FFN 512, 4 query / 1 KV heads of 64, vocab 1024, 64 cached
    positions, k = 8, seed 0), and the 6-layer two-width miniature with sliding, full and KV-shared
    layers: the numpy twin and the C oracle agree to 1e-12 rel-L1 on every row's logits, and on the
    appended K/V rows."""
    if which == "config1":
        m, P, k = synth.tiny_model(), 64, 8
    else:
        m, P, k = synth.tiny_two_width_model(), 21, 8
    w = synth.make_weights(m, 0)
    kv = synth.make_kv(m, P, 0)
    toks = synth.tokens(0, "twin.tokens", k, m.vocab)
    om = oracle.Model(m, w)
    om.set_kv(kv, P)
    ref = om.verify_batch(toks).astype(np.float64)
    tw = Twin(m, w)
    tw.set_kv(kv, P)
    got = tw.verify_batch(toks)
    err = rel_l1(got, ref)
    assert err <= 1e-12, err
    for l in range(m.n_layers):
        if m.own(l):
            diff = np.abs(om.plane(l, P + k).astype(np.float64) - tw.planes[l][:P + k])
            assert diff.max() <= 1e-12 * max(1.0, np.abs(tw.planes[l][:P + k]).max())


@pytest.mark.parametrize("window", [0, 4])
def test_numpy_twin_agrees_with_oracle_on_the_draft(window):
    """The tiny draft (2 layers, hidden 256, 3 taps) over 10 context rows appended in two calls,
    then a block of 8 (embedding scale 0.5, mask V-1): the numpy twin and the C oracle agree to
    1e-12 rel-L1 on the block logits and on the context planes; window 4 leaves 6 rows outside."""
    from tests.numpy_twin import DraftTwin
    tm = synth.tiny_model(max_ctx=64)
    tw = synth.make_weights(tm)
    dm = synth.tiny_draft_model(max_ctx=64, window=window)
    dw = synth.make_weights(dm)
    taps = synth.bf16_normal(0, "twin.draft.taps", (10, len(dm.tap_layers), dm.hidden))
    T = oracle.Model(tm, tw)
    D = oracle.Model(dm, dw)
    D.draft_append(taps[:3]); D.draft_append(taps[3:])
    _, ref = D.draft_block(T, 8, 3, 0.5, tm.vocab - 1, with_logits=True)
    twin = DraftTwin(dm, dw)
    twin.append(taps[:3]); twin.append(taps[3:])
    got = twin.block(tw["embed"], 8, 3, 0.5, tm.vocab - 1)
    assert rel_l1(got, ref) <= 1e-12
    for l in range(dm.n_layers):
        assert np.abs(D.plane(l, 10).astype(np.float64) - twin.planes[l][:10]).max() <= 1e-12


# ------------------------------------------------------------------------------------------
# per-layer embeddings (PLE): per-row inputs by token id, gate and projection, layer scalar
# ------------------------------------------------------------------------------------------
def _ple_model(n_layers=2, taps=(0, 1)):
    import dataclasses
    m = dataclasses.replace(synth.tiny_model(max_ctx=16, n_layers=n_layers), ple_dim=128, name="tinyple",
                            tap_layers=taps)
    return m


def test_ple_tail_closed_form():
    """Two layers, every attention and MLP matrix zero, so each layer's residual input passes
    unchanged to its PLE tail. Layer 0's PLE matrices are zero too: x1 = fp32(x0 s0). Layer 1's
    gate has one entry (row 5, column 7) = 2 and its projection one entry (row 9, column 5) = 3:
    u5 = 2 bf16(x1[7]), h5 = bf16(silu(u5) p), p = the per-layer input of the row's token for
    layer 1 at element 5, and x2 = fp32(fp32(x1 + 3 h5 e9) s1). The taps after layers 0 and 1 are
    bf16(x1) and bf16(x2); two rows with different tokens."""
    m = _ple_model()
    w = zero_weights(m)
    H, D = 256, 128
    w["ple_table"] = synth.bf16_normal(0, "pin.ple.table", (m.vocab, m.n_layers * D))
    for l in range(2):
        w["layers"][l]["layer_scalar"] = _bits([1.25 if l == 0 else 0.75])
        w["layers"][l]["ple_gate"] = zero_q4(D, H)
        w["layers"][l]["ple_proj"] = zero_q4(H, D)
    w["layers"][1]["ple_gate"] = _q4_from_entries(D, H, {(5, 7): 2.0})
    w["layers"][1]["ple_proj"] = _q4_from_entries(H, D, {(9, 5): 3.0})
    om = oracle.Model(m, w)
    om.set_kv([np.zeros((0, 2, 64), dtype=np.float32)] * 2, 0)
    toks = np.array([11, 500], dtype=np.int32)
    _, taps = om.verify_batch(toks, with_taps=True)
    E = synth.bf16_to_f32(w["embed"]).astype(np.float64)
    P = synth.bf16_to_f32(w["ple_table"]).astype(np.float64)
    for r, t in enumerate(toks):
        x1 = np.float32(E[t] * 1.25).astype(np.float64)
        u5 = _f32(2.0 * _bf16(x1[7]))
        h5 = _bf16(u5 / (1.0 + math.exp(-u5)) * P[t, 1 * D + 5])
        x2 = x1.copy()
        x2[9] = _f32(x1[9] + _f32(3.0 * h5))
        x2 = np.float32(x2 * 0.75).astype(np.float64)
        assert np.array_equal(synth.bf16_to_f32(taps[r, 0]).astype(np.float64), synth.bf16_to_f32(synth.bf16_bits(x1)))
        assert np.array_equal(synth.bf16_to_f32(taps[r, 1]).astype(np.float64), synth.bf16_to_f32(synth.bf16_bits(x2)))
    assert h5 != 0.0


def test_ple_batched_equals_sequential_and_injected_rows_refused():
    """With PLE the k batched rows still equal k sequential steps bit for bit; a verify of injected
    rows, and a single layer fed injected rows, are refused (the per-layer inputs need token ids)."""
    import dataclasses
    m = dataclasses.replace(synth.tiny_two_width_model(), ple_dim=128, name="tiny2wple")
    w = synth.make_weights(m, 0)
    kv = synth.make_kv(m, 10, 0)
    toks = synth.tokens(0, "pin.ple.seq", 5, m.vocab)
    A = oracle.Model(m, w); A.set_kv(kv, 10)
    B = oracle.Model(m, w); B.set_kv(kv, 10)
    la = A.verify_batch(toks)
    lb = np.stack([B.step(int(t)) for t in toks])
    assert np.array_equal(la, lb)
    with pytest.raises(RuntimeError):
        A.verify_embedded(np.zeros((2, m.hidden), dtype=np.float32))
    with pytest.raises(RuntimeError):
        A.layer_forward(0, np.zeros((2, m.hidden), dtype=np.float32), [15, 16])


def test_numpy_twin_agrees_with_oracle_with_ple():
    """The two-width miniature with per-layer embeddings (width 128): numpy twin and C oracle agree
    to 1e-12 on the logits."""
    import dataclasses
    m = dataclasses.replace(synth.tiny_two_width_model(), ple_dim=128, name="tiny2wple")
    w = synth.make_weights(m, 0)
    kv = synth.make_kv(m, 21, 0)
    toks = synth.tokens(0, "twin.ple.tokens", 8, m.vocab)
    om = oracle.Model(m, w); om.set_kv(kv, 21)
    tw = Twin(m, w); tw.set_kv(kv, 21)
    assert rel_l1(tw.verify_batch(toks), om.verify_batch(toks)) <= 1e-12


# ------------------------------------------------------------------------------------------
# ring planes: sliding planes of window + 16 position slots behave as the linear planes
# ------------------------------------------------------------------------------------------
def test_ring_planes_equal_linear_planes_over_a_state_sequence():
    """The two-width miniature (sliding window 16 -> ring of 32 slots; full and shared layers
    unchanged), once with linear planes and once with rings: through set_kv of 45 positions, verifies
    of 8, 5, 16 and 4 rows with commits of 3, 5, 0 and 4 rows, an extend_context of 7 rows, a
    snapshot and a restore, every verify's logits are bit-identical, the held positions agree, ring
    planes count the last min(held, window) positions at their width (engine PR #2303 "What changes"
    item 1: the count is per layer; older slots may carry rows a commit cut back), and the rows a
    ring holds equal the linear plane's rows."""
    import dataclasses
    base = synth.tiny_two_width_model()
    ring = dataclasses.replace(base, kv_ring=1)
    w = synth.make_weights(base, 0)
    kv = synth.make_kv(base, 45, 0)
    kv_new = synth.make_kv(base, 7, 1)
    L = oracle.Model(base, w); L.set_kv(kv, 45)
    R = oracle.Model(ring, w); R.set_kv(kv, 45)
    caps = [R.capacity(l) if base.own(l) else 0 for l in range(base.n_layers)]
    assert caps == [32 if (base.own(l) and base.layers[l].attn == synth.ATTN_SLIDING) else
                    (base.max_ctx if base.own(l) else 0) for l in range(base.n_layers)]

    keep = [base.layers[l].window if caps[l] == 32 else base.max_ctx for l in range(base.n_layers)]

    def counts(held):
        return [min(held, keep[l]) * 2 * base.kv_width(l) if base.own(l) else 0 for l in range(base.n_layers)]

    def step(k, n, tag):
        toks = synth.tokens(0, f"pin.ring.{tag}", k, base.vocab)
        assert np.array_equal(L.verify_batch(toks), R.verify_batch(toks)), tag
        assert L.commit_verify_rows(n) == 0 and R.commit_verify_rows(n) == 0
        assert L.held() == R.held()
        assert list(R.plane_floats()) == counts(R.held())
        for l in range(base.n_layers):
            if base.own(l):
                h = R.held()
                lo = max(0, h - keep[l])
                assert np.array_equal(R.plane(l, h)[lo:], L.plane(l, h)[lo:]), (tag, l)

    step(8, 3, "a")
    step(5, 5, "b")
    assert L.extend_context(kv_new, 7) == 0 and R.extend_context(kv_new, 7) == 0
    snap_l, snap_r = L.snapshot(), R.snapshot()
    assert snap_r.floats() == counts(R.held())
    step(16, 0, "c")
    assert L.restore(snap_l) == 0 and R.restore(snap_r) == 0
    step(4, 4, "d")
    assert L.held() == 45 + 3 + 5 + 7 + 4
    # a ring snapshot does not restore into a linear model (different plane capacities)
    assert L.restore(snap_r) != 0

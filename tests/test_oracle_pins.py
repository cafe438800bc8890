"""Pins of the CPU oracle against what the pages and the mathematics fix (closed forms, hand cases,
invariants, brute force on tiny inputs). No GPU; no HIP library."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import synth
from tests.util import golden, int_q4, no_weights, np_dequant, rel_l1, zero_q4, zero_weights


# ------------------------------------------------------------------------------------------
# Q4_1 dequant
# ------------------------------------------------------------------------------------------
def _block(scale_bits: int, min_bits: int, codes):
    """One canonical block from raw fp16 bits and 32 codes."""
    b = np.zeros(20, dtype=np.uint8)
    b[0], b[1] = scale_bits & 255, scale_bits >> 8
    b[2], b[3] = min_bits & 255, min_bits >> 8
    for j in range(16):
        b[4 + j] = (codes[j] & 15) | ((codes[j + 16] & 15) << 4)
    return b.reshape(1, 1, 20)


def test_dequant_hand_block():
    # scale 0x3800 = 0.5, min 0xBC00 = -1.0; codes 0..15 then 15..0
    codes = list(range(16)) + list(range(15, -1, -1))
    w = oracle.q4_1_dequant(_block(0x3800, 0xBC00, codes), 1, 32)[0]
    expect = [0.5 * c - 1.0 for c in codes]
    assert w.tolist() == expect


def test_dequant_nibble_order():
    # byte j holds code j in the low nibble and code j+16 in the high nibble
    img = np.zeros((1, 1, 20), dtype=np.uint8)
    img[0, 0, 0:2] = [0x00, 0x3C]      # scale 1.0
    img[0, 0, 4] = 0x21                # code 0 = 1, code 16 = 2
    img[0, 0, 19] = 0xF7               # code 15 = 7, code 31 = 15
    w = oracle.q4_1_dequant(img, 1, 32)[0]
    assert w[0] == 1 and w[16] == 2 and w[15] == 7 and w[31] == 15
    assert np.count_nonzero(w) == 4


def test_dequant_fp16_edges():
    # subnormal scale 2^-24 with code 15; largest finite min; negative zero scale
    w = oracle.q4_1_dequant(_block(0x0001, 0x0000, [15] * 32), 1, 32)[0]
    assert np.all(w == np.float32(15 * 2.0 ** -24))
    w = oracle.q4_1_dequant(_block(0x0000, 0x7BFF, [9] * 32), 1, 32)[0]
    assert np.all(w == 65504.0)
    w = oracle.q4_1_dequant(_block(0x8000, 0xFBFF, [3] * 32), 1, 32)[0]
    assert np.all(w == -65504.0)


def test_dequant_exact_at_config_ranges():
    """Every fp16 scale and min is a multiple of 2^-24 and |w| < 0.5 at these ranges, so
    scale*code+min is exact in fp32: the fp32 weight equals the exact rational value."""
    img = synth.q4_1_image(0, "pin.exact", 64, 512)
    w = oracle.q4_1_dequant(img, 64, 512).astype(np.float64)
    exact = np_dequant(img)      # float64 arithmetic on exact fp16 values is exact here
    assert np.array_equal(w, exact)
    assert np.max(np.abs(exact)) < 0.5


def test_bits_per_weight():
    g = golden("q4_1_bits_per_weight")
    img = synth.q4_1_image(0, "pin.size", 16, 256)
    assert img.nbytes * 8 / (16 * 256) == g["bits"]
    assert g["block_bytes"] * 8 / g["block"] == g["bits"]


def test_draft_geometry_matches_card():
    g = golden("draft_geometry")
    m = synth.draft_model()
    assert (m.n_layers, m.hidden, m.n_q_heads) == (g["layers"], g["hidden"], g["q_heads"])
    L = m.layers[0]
    assert (L.n_kv_heads, L.head_dim, L.ffn) == (g["kv_heads"], g["head_dim"], g["ffn"])
    q4 = sum(n_out * n_in for l in range(m.n_layers) for (n_out, n_in) in synth.layer_matrix_shapes(m, l).values())
    fc = m.hidden * g["n_taps"] * m.hidden
    assert q4 == 327_680_000
    assert round((q4 + fc) / 1e9, 2) == g["params_billions_rounded"]
    nbytes = q4 * 5 / 8 + fc * 2
    assert round(nbytes / 1e9, 2) == g["gbytes_rounded"]
    assert synth.q4_1_bytes(m) == q4 * 5 // 8


def test_target_geometry():
    m = synth.target_model()
    g = golden("two_widths")
    s = golden("shared_planes")
    assert m.n_layers == s["n_layers"]
    for l in range(m.n_layers):
        w = 2 * m.kv_width(m.layers[l].kv_owner if m.layers[l].kv_owner >= 0 else l)
        assert w == (g["full_floats_per_pos"] if l % 6 == 5 else g["sliding_floats_per_pos"])
        assert (m.layers[l].kv_owner >= 0) == (s["first_shared"] <= l <= s["last_shared"])
    assert {m.layers[l].kv_owner for l in range(24, 42)} == {22, 23}
    assert m.tap_layers == tuple(golden("taps")["layers"])
    assert abs(synth.q4_1_bytes(m) / 1e9 - 3.247) < 0.001


# ------------------------------------------------------------------------------------------
# GEMMs
# ------------------------------------------------------------------------------------------
def test_q4_1_matmul_all_codes_zero_is_min_times_block_sum():
    n_out, n_in = 24, 128
    rng = np.random.default_rng(1)
    mins = rng.uniform(-0.15, 0, size=(n_out, n_in // 32))
    img = synth.q4_1_from_parts(np.zeros((n_out, n_in)), rng.uniform(0.002, 0.02, (n_out, n_in // 32)), mins)
    x = synth.bf16_bits(rng.standard_normal((3, n_in)))
    xf = synth.bf16_to_f32(x).astype(np.float64)
    mins16 = mins.astype(np.float16).astype(np.float64)
    bsum = xf.reshape(3, n_in // 32, 32).sum(axis=2)          # [3, nb]
    expect = bsum @ mins16.T
    got = oracle.q4_1_matmul(img, n_out, n_in, x)
    np.testing.assert_allclose(got, expect, rtol=1e-6, atol=1e-6)


def test_q4_1_matmul_off_diagonal_entry():
    """One entry W[5][40] = 0.25 * 3: y[:, 5] = 0.75 x[:, 40] and nothing else. A transposed
    application would move it (and here would not even fit the shape)."""
    W = np.zeros((32, 64), dtype=np.int64)
    W[5, 40] = 3
    img = int_q4(W, scale=0.25)
    x = synth.bf16_bits(np.random.default_rng(2).standard_normal((2, 64)))
    y = oracle.q4_1_matmul(img, 32, 64, x)
    xf = synth.bf16_to_f32(x)
    assert np.all(y[:, 5] == np.float32(0.75) * xf[:, 40])
    y[:, 5] = 0
    assert not y.any()


def test_q4_1_matmul_brute_force():
    img = synth.q4_1_image(0, "pin.bf", 48, 96)
    x = synth.bf16_bits(np.random.default_rng(3).standard_normal((3, 96)))
    expect = synth.bf16_to_f32(x).astype(np.float64) @ np_dequant(img).T
    got = oracle.q4_1_matmul(img, 48, 96, x)
    np.testing.assert_allclose(got, expect, rtol=1e-6, atol=1e-7)


def test_q4_1_matmul_rows_are_independent():
    img = synth.q4_1_image(0, "pin.rows", 40, 128)
    x = synth.bf16_bits(np.random.default_rng(4).standard_normal((4, 128)))
    y = oracle.q4_1_matmul(img, 40, 128, x)
    for r in range(4):
        assert np.array_equal(y[r], oracle.q4_1_matmul(img, 40, 128, x[r:r + 1])[0])


def test_bf16_matmul_brute_force():
    W = synth.bf16_normal(0, "pin.bfw", (33, 64))
    x = synth.bf16_bits(np.random.default_rng(5).standard_normal((2, 64)))
    expect = synth.bf16_to_f32(x).astype(np.float64) @ synth.bf16_to_f32(W).astype(np.float64).T
    np.testing.assert_allclose(oracle.bf16_matmul(W, x), expect, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------------------------------
# RMSNorm / RoPE
# ------------------------------------------------------------------------------------------
def test_rmsnorm_constant_vector():
    n = 256
    g = synth.bf16_uniform(0, "pin.g", (n,), 0.5, 1.5)
    out = oracle.rmsnorm_bf16(np.full(n, -2.0, dtype=np.float32), g, eps=1e-6)
    expect = synth.bf16_bits(-2.0 / math.sqrt(4.0 + 1e-6) * synth.bf16_to_f32(g).astype(np.float64))
    assert np.array_equal(out, expect)


def test_rmsnorm_unit_gain_unit_rms():
    # x with mean square exactly 1 (entries +-1) and gain 1: output = x (eps negligible at bf16)
    x = np.where(np.arange(64) % 3 == 0, 1.0, -1.0).astype(np.float32)
    g = synth.bf16_bits(np.ones(64))
    out = synth.bf16_to_f32(oracle.rmsnorm_bf16(x, g, eps=0.0))
    assert np.array_equal(out, x)


def test_rope_identity_at_zero():
    v = np.random.default_rng(6).standard_normal(64).astype(np.float32)
    assert np.array_equal(oracle.rope(v, 0), v)


def test_rope_pairing_hand_case():
    """hd = 4, base 1e6, p = 1: pair (0, 2) turns by 1 rad, pair (1, 3) by 1e6^(-1/2) = 1e-3 rad
    (rotate-half pairing, not interleaved)."""
    v = np.array([1.0, 0.0, 0.0, 0.0], dtype=np.float32)
    out = oracle.rope(v, 1)
    np.testing.assert_allclose(out, [math.cos(1.0), 0.0, math.sin(1.0), 0.0], atol=1e-7)
    v = np.array([0.0, 1.0, 0.0, 0.0], dtype=np.float32)
    out = oracle.rope(v, 1)
    np.testing.assert_allclose(out, [0.0, math.cos(1e-3), 0.0, math.sin(1e-3)], atol=1e-7)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(7)
    q = rng.standard_normal(64).astype(np.float32)
    k = rng.standard_normal(64).astype(np.float32)
    for p in (1, 17, 1000):
        r = oracle.rope(q, p).astype(np.float64)
        pairs0 = q[:32].astype(np.float64) ** 2 + q[32:].astype(np.float64) ** 2
        np.testing.assert_allclose(r[:32] ** 2 + r[32:] ** 2, pairs0, rtol=1e-5)
    d1 = float(np.dot(oracle.rope(q, 10).astype(np.float64), oracle.rope(k, 7).astype(np.float64)))
    d2 = float(np.dot(oracle.rope(q, 503).astype(np.float64), oracle.rope(k, 500).astype(np.float64)))
    assert abs(d1 - d2) < 1e-4


# ------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------
def _planes(m, positions, seed=0):
    return synth.make_kv(m, positions, seed)


def test_attention_single_key_returns_value():
    m = synth.tiny_model()
    om = oracle.Model(m, zero_weights(m))
    kv = _planes(m, 1)
    om.set_kv(kv, 1)
    q = np.random.default_rng(8).standard_normal(256).astype(np.float32)
    out = om.attend(0, q, 0)
    for h in range(4):
        assert np.array_equal(out[h * 64:(h + 1) * 64], kv[0][0, 1, :].astype(np.float64))


def test_attention_equal_scores_is_mean_of_values():
    m = synth.tiny_model()
    om = oracle.Model(m, zero_weights(m))
    kv = _planes(m, 5)
    kv[0][:, 0, :] = kv[0][0, 0, :]          # identical keys
    om.set_kv(kv, 5)
    q = np.random.default_rng(9).standard_normal(256).astype(np.float32)
    out = om.attend(0, q, 4)
    np.testing.assert_allclose(out[:64], kv[0][:, 1, :].astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_two_keys_closed_form():
    m = synth.tiny_model()
    om = oracle.Model(m, zero_weights(m))
    kv = [np.zeros((2, 2, 64), dtype=np.float32)]
    kv[0][0, 0, 0] = 4.0                     # key 0 = 4 e0, key 1 = 0
    kv[0][0, 1, 1] = 1.0                     # value 0 = e1
    kv[0][1, 1, 2] = 1.0                     # value 1 = e2
    om.set_kv(kv, 2)
    q = np.zeros(256, dtype=np.float32)
    q[0] = 2.0                               # score0 = 8 / sqrt(64) = 1, score1 = 0
    out = om.attend(0, q, 1)
    w0 = math.exp(1.0) / (math.exp(1.0) + 1.0)
    np.testing.assert_allclose(out[:3], [0.0, w0, 1.0 - w0], rtol=1e-14)


def test_attention_window_edge_and_gqa_and_shared_owner():
    m = synth.tiny_two_width_model()
    om = oracle.Model(m, zero_weights(m))
    kv = _planes(m, 21)
    om.set_kv(kv, 21)
    q = np.random.default_rng(10).standard_normal(256).astype(np.float32)
    base = om.attend(0, q, 20)                 # sliding, window 16: keys 5..20
    kv[0][4] += 100.0                          # older than the window
    om.set_kv(kv, 21)
    assert np.array_equal(om.attend(0, q, 20), base)
    kv[0][5, 1] += 1.0                         # oldest visible key's value
    om.set_kv(kv, 21)
    assert not np.array_equal(om.attend(0, q, 20), base)
    # full layer 2 (2 KV heads, query heads 0,1 -> head 0; 2,3 -> head 1), single visible key
    out = om.attend(2, q, 0)
    for h in range(4):
        g = h // 2
        assert np.array_equal(out[h * 64:(h + 1) * 64], kv[2][0, 1, g * 64:(g + 1) * 64].astype(np.float64))
    # shared layers read the owner's plane: 4 -> 3 (sliding), 5 -> 2 (full)
    assert np.array_equal(om.attend(4, q, 20), om.attend(3, q, 20))
    assert np.array_equal(om.attend(5, q, 20), om.attend(2, q, 20))


# ------------------------------------------------------------------------------------------
# a layer with hand weights (off-diagonal v and down entries catch transposed projections)
# ------------------------------------------------------------------------------------------
def _hand_layer_model():
    m = synth.tiny_model(max_ctx=8)
    w = zero_weights(m)
    return m, w


def test_layer_hand_case_value_projection():
    m, w = _hand_layer_model()
    Wv = np.zeros((64, 256), dtype=np.int64)
    Wv[3, 10] = 2                              # v[3] = 2 a[10]
    w["layers"][0]["v"] = int_q4(Wv)
    w["layers"][0]["o"] = int_q4(np.eye(256, dtype=np.int64))
    om = oracle.Model(m, w)
    om.set_kv(_planes(m, 0), 0)
    x = synth.bf16_to_f32(synth.bf16_normal(0, "pin.x", (256,)))
    out = om.layer_forward(0, x, [0])[0]
    a = synth.bf16_to_f32(oracle.rmsnorm_bf16(x, w["layers"][0]["attn_norm"]))
    o = synth.bf16_to_f32(synth.bf16_bits(np.float64(2.0) * np.float64(a[10])))
    expect = x.copy()
    for h in range(4):                         # one KV head serves all 4 query heads; one key (itself)
        expect[h * 64 + 3] = np.float32(np.float64(x[h * 64 + 3]) + np.float64(o))
    assert np.array_equal(out, expect)


def test_layer_hand_case_down_projection():
    m, w = _hand_layer_model()
    Wg = np.zeros((512, 256), dtype=np.int64); Wg[5, 9] = 1
    Wu = np.zeros((512, 256), dtype=np.int64); Wu[5, 9] = 2
    Wd = np.zeros((256, 512), dtype=np.int64); Wd[12, 5] = 3
    w["layers"][0].update(gate=int_q4(Wg), up=int_q4(Wu), down=int_q4(Wd))
    om = oracle.Model(m, w)
    om.set_kv(_planes(m, 0), 0)
    x = synth.bf16_to_f32(synth.bf16_normal(0, "pin.x2", (256,)))
    out = om.layer_forward(0, x, [0])[0]
    b = float(synth.bf16_to_f32(oracle.rmsnorm_bf16(x, w["layers"][0]["mlp_norm"]))[9])
    mm = float(synth.bf16_to_f32(synth.bf16_bits(b / (1.0 + math.exp(-b)) * (2.0 * b))))
    expect = x.copy()
    expect[12] = np.float32(float(x[12]) + 3.0 * mm)
    assert np.array_equal(out, expect)


def test_embed_and_head_closed_form():
    m = synth.tiny_model()
    w = zero_weights(m)
    om = oracle.Model(m, w)
    om.set_kv(_planes(m, 4), 4)
    t = 77
    lg = om.step(t)
    x = synth.bf16_to_f32(w["embed"][t])
    a = synth.bf16_to_f32(oracle.rmsnorm_bf16(x, w["final_norm"])).astype(np.float64)
    expect = synth.bf16_to_f32(w["embed"]).astype(np.float64) @ a
    np.testing.assert_allclose(lg, expect, rtol=1e-6, atol=1e-5)


# ------------------------------------------------------------------------------------------
# batched == sequential; commit / rollback; snapshot / restore; per-layer widths
# ------------------------------------------------------------------------------------------
def _two_width(seed=0, positions=5):
    m = synth.tiny_two_width_model()
    w = synth.make_weights(m, seed)
    kv = synth.make_kv(m, positions, seed)
    return m, w, kv


def test_batched_rows_bit_identical_to_sequential_steps():
    m, w, kv = _two_width()
    toks = synth.tokens(0, "pin.toks", 4, m.vocab)
    A = oracle.Model(m, w); A.set_kv(kv, 5)
    B = oracle.Model(m, w); B.set_kv(kv, 5)
    lgA, tapsA = A.verify_batch(toks, with_taps=True)
    for i, t in enumerate(toks):
        lg, taps = B.step(int(t), with_taps=True)
        assert np.array_equal(lg, lgA[i])
        assert np.array_equal(taps, tapsA[i])
    assert A.held() == B.held() == 9
    for l in range(m.n_layers):
        if m.own(l):
            assert np.array_equal(A.plane(l, 9), B.plane(l, 9))


def test_commit_worked_case_and_next_step():
    g = golden("commit_worked_case")
    m, w, kv = _two_width(positions=g["prefix"])
    toks = synth.tokens(0, "pin.commit", g["k"], m.vocab)
    A = oracle.Model(m, w); A.set_kv(kv, g["prefix"])
    A.verify_batch(toks)
    assert A.commit_verify_rows(g["commit"]) == 0
    assert A.held() == g["held_after"]
    floats = A.plane_floats()
    for l in range(m.n_layers):
        expect = g["held_after"] * 2 * m.kv_width(l) if m.own(l) else 0
        assert floats[l] == expect
    # the next step equals a forward that only ever saw the accepted rows
    nxt = 5
    lgA = A.step(nxt)
    B = oracle.Model(m, w); B.set_kv(kv, g["prefix"])
    for t in toks[: g["commit"]]:
        B.step(int(t))
    assert np.array_equal(B.step(nxt), lgA)


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4])
def test_commit_every_n(n):
    m, w, kv = _two_width(positions=6)
    toks = synth.tokens(0, "pin.commit_n", 4, m.vocab)
    A = oracle.Model(m, w); A.set_kv(kv, 6)
    A.verify_batch(toks)
    assert A.commit_verify_rows(n) == 0
    assert A.held() == 6 + n
    lgA = A.verify_batch(toks[::-1].copy())
    B = oracle.Model(m, w); B.set_kv(kv, 6)
    for t in toks[:n]:
        B.step(int(t))
    assert np.array_equal(B.verify_batch(toks[::-1].copy()), lgA)


def test_commit_refusals():
    m, w, kv = _two_width()
    A = oracle.Model(m, w); A.set_kv(kv, 5)
    assert A.commit_verify_rows(0) == 2          # nothing pending
    A.verify_batch(np.array([1, 2, 3], dtype=np.int32))
    assert A.commit_verify_rows(4) == 2          # n > k
    assert A.held() == 8                         # unchanged by the refusal
    assert A.commit_verify_rows(3) == 0
    assert A.commit_verify_rows(1) == 2          # already committed


def test_extend_context_per_layer_widths():
    """extend_context appends each own plane's rows at its own width ([PR2303] "What changes" item 1:
    the count is per layer): extending 5 cached positions by 3 gives the planes, the counts and the
    next step of a model that cached all 8 from the start; shared planes stay empty."""
    m, w, kv8 = _two_width(positions=8)
    assert len({m.kv_width(l) for l in range(m.n_layers) if m.own(l)}) == 2   # two geometries
    A = oracle.Model(m, w); A.set_kv(kv8, 5)
    new = [None if kv is None else kv[5:8] for kv in kv8]
    assert A.extend_context(new, 3) == 0
    assert A.held() == 8
    assert list(A.plane_floats()) == [8 * 2 * m.kv_width(l) if m.own(l) else 0 for l in range(m.n_layers)]
    B = oracle.Model(m, w); B.set_kv(kv8, 8)
    for l in range(m.n_layers):
        if m.own(l):
            assert np.array_equal(A.plane(l, 8), B.plane(l, 8)), f"plane {l}"
    assert np.array_equal(A.step(11), B.step(11))


def test_extend_context_refusals_leave_state():
    m, w, kv8 = _two_width(positions=8)
    A = oracle.Model(m, w); A.set_kv(kv8, 5)
    new = [None if kv is None else kv[5:8] for kv in kv8]
    A.verify_batch(np.array([1, 2], dtype=np.int32))
    before = [A.plane(l, 8) for l in range(m.n_layers) if m.own(l)]
    assert A.extend_context(new, 3) == 2                 # a verify is pending
    assert A.held() == 7
    assert all(np.array_equal(b, A.plane(l, 8)) for b, l in zip(before, [l for l in range(m.n_layers) if m.own(l)]))
    assert A.commit_verify_rows(0) == 0
    big = [None if kv is None else np.zeros((m.max_ctx, 2, kv.shape[2]), np.float32) for kv in kv8]
    assert A.extend_context(big, m.max_ctx - 4) == 3     # past max_ctx
    assert A.held() == 5
    assert A.extend_context(new, 0) == 0 and A.held() == 5


def test_snapshot_restore_per_layer_widths():
    m, w, kv = _two_width(positions=6)
    A = oracle.Model(m, w); A.set_kv(kv, 6)
    snap = A.snapshot()
    assert snap.floats() == [6 * 2 * m.kv_width(l) if m.own(l) else 0 for l in range(m.n_layers)]
    A.verify_batch(np.array([4, 5, 6], dtype=np.int32))
    A.commit_verify_rows(3)
    assert A.restore(snap) == 0
    assert A.held() == 6
    lgA = A.step(9)
    B = oracle.Model(m, w); B.set_kv(kv, 6)
    assert np.array_equal(B.step(9), lgA)
    # a restore into a model with other widths is refused
    m2 = synth.tiny_model(max_ctx=m.max_ctx)
    C = oracle.Model(m2, synth.make_weights(m2))
    assert C.restore(snap) == 1


def test_cut_arithmetic_and_per_list_shorter_than_planes():
    g = golden("cut_arithmetic")
    assert oracle.cut_floats([g["width"]], 0, g["positions"]) == g["floats"]
    per = [256, 512, 128]
    for plane in range(5):
        assert oracle.cut_floats(per, plane, 7) == 7 * 2 * per[min(plane, 2)]


def test_old_single_width_cut_is_wrong_on_two_widths():
    """Negative control: the previous rule counted every layer at NKV*HD of the sliding geometry.
    On the target layout it reads twice the positions from a full plane and a cut keeps half."""
    m = synth.target_model(max_ctx=256, vocab=64)
    om = oracle.Model(m, no_weights(m))
    P = 100
    om.set_kv(synth.make_kv(m, P), P)
    floats = om.plane_floats()
    base = m.kv_width(0)                         # the single width of the old rule (256)
    full_own = [l for l in range(24) if l % 6 == 5]
    for l in full_own:
        assert floats[l] // (2 * base) == 2 * P                     # old count: twice the positions
        assert (P * 2 * base) * 2 == floats[l]                      # old cut: half the plane
        assert floats[l] // (2 * m.kv_width(l)) == P                # per-layer width: right
    # mutant: a single-width list gives wrong cuts exactly on the full planes and right ones elsewhere
    mutant = [base] * m.n_layers
    real = om.kv_widths()
    wrong = [l for l in range(24) if oracle.cut_floats(mutant, l, P) != oracle.cut_floats(real, l, P)]
    assert wrong == full_own
    assert all(floats[l] == 0 for l in range(24, 42))


# ------------------------------------------------------------------------------------------
# accept
# ------------------------------------------------------------------------------------------
def test_accept_constructed_mismatch_positions():
    rng = np.random.default_rng(11)
    k, V = 8, 300
    lg = rng.standard_normal((k, V)).astype(np.float32)
    y = lg.argmax(axis=1)
    for j in range(k):
        toks = np.zeros(k, dtype=np.int32)
        toks[0] = 5
        toks[1:j + 1] = y[:j]
        if j + 1 < k:
            toks[j + 1] = (y[j] + 1) % V
            toks[j + 2:] = y[j + 1:k - 1]        # later drafts agree but come after a miss
        a, out = oracle.accept_greedy(lg, toks)
        assert a == j
        assert out.tolist() == y[: j + 1].tolist()


def test_argmax_ties_and_nan():
    v = np.zeros(10, dtype=np.float32)
    v[7] = v[3] = 2.0
    assert oracle.argmax(v) == 3
    v[0] = np.nan
    assert oracle.argmax(v) == 3
    assert oracle.argmax(np.full(4, np.nan, dtype=np.float32)) == 0


def test_acceptance_accounting():
    g = golden("acceptance_accounting")
    assert round(g["accepted"] / g["passes"], 2) == g["accepted_per_pass"]
    assert round((g["accepted"] + g["passes"]) / g["passes"], 2) == g["tokens_per_pass"]


def test_speculative_output_equals_plain_greedy():
    m, w, kv = _two_width(positions=4)
    plain = oracle.Model(m, w); plain.set_kv(kv, 4)
    t = 11
    greedy = []
    for _ in range(14):
        t = oracle.argmax(plain.step(t))
        greedy.append(t)
    spec = oracle.Model(m, w); spec.set_kv(kv, 4)
    rng = np.random.default_rng(12)
    out, t = [], 11
    while len(out) < 14:
        # a draft that is partly right: the true continuation with random corruptions
        i = len(out)
        truth = greedy[i:i + 3] + [0] * 3
        d = [tok if rng.random() < 0.6 else int(rng.integers(m.vocab)) for tok in truth[:3]]
        lg = spec.verify_batch(np.array([t] + d, dtype=np.int32))
        a, emitted = oracle.accept_greedy(lg, np.array([t] + d, dtype=np.int32))
        spec.commit_verify_rows(a + 1)
        out += emitted.tolist()
        t = int(emitted[-1])
    assert out[:14] == greedy


# ------------------------------------------------------------------------------------------
# draft block forward: invariants (closed forms and the numpy twin in test_oracle_pins_paths.py)
# ------------------------------------------------------------------------------------------
def _draft_pair(window=0, n_ctx=10):
    tm = synth.tiny_model(max_ctx=64)
    tw = synth.make_weights(tm)
    dm = synth.tiny_draft_model(max_ctx=64, window=window)
    dw = synth.make_weights(dm)
    taps = synth.bf16_normal(0, "pin.taps", (n_ctx, len(dm.tap_layers), dm.hidden))
    T = oracle.Model(tm, tw)
    D = oracle.Model(dm, dw)
    return tm, dm, T, D, dw, taps


def test_draft_context_append_is_incremental():
    tm, dm, T, D, dw, taps = _draft_pair()
    D.draft_append(taps)
    p1, l1 = D.draft_block(T, 8, 3, 1.0, tm.vocab - 1, with_logits=True)
    D2 = oracle.Model(dm, dw)
    for i in range(taps.shape[0]):
        D2.draft_append(taps[i:i + 1])
    p2, l2 = D2.draft_block(T, 8, 3, 1.0, tm.vocab - 1, with_logits=True)
    assert np.array_equal(l1, l2) and np.array_equal(p1, p2)
    assert np.array_equal(p1, l1.argmax(axis=1))


def test_draft_window_covers_context_is_irrelevant_and_old_rows_ignored():
    tm, dm, T, D, dw, taps = _draft_pair(window=0)
    D.draft_append(taps)
    _, l_all = D.draft_block(T, 8, 3, 1.0, tm.vocab - 1, with_logits=True)
    dmw = synth.tiny_draft_model(max_ctx=64, window=10)
    Dw = oracle.Model(dmw, dw)
    Dw.draft_append(taps)
    _, l_w = Dw.draft_block(T, 8, 3, 1.0, tm.vocab - 1, with_logits=True)
    assert np.array_equal(l_all, l_w)
    # window 4 over 10 context rows: rows 0..5 are outside and must not matter
    dm4 = synth.tiny_draft_model(max_ctx=64, window=4)
    D4 = oracle.Model(dm4, dw); D4.draft_append(taps)
    _, l4 = D4.draft_block(T, 8, 3, 1.0, tm.vocab - 1, with_logits=True)
    taps2 = taps.copy()
    taps2[:6] = synth.bf16_normal(1, "pin.taps.other", taps2[:6].shape)
    D4b = oracle.Model(dm4, dw); D4b.draft_append(taps2)
    _, l4b = D4b.draft_block(T, 8, 3, 1.0, tm.vocab - 1, with_logits=True)
    assert np.array_equal(l4, l4b)
    assert not np.array_equal(l4, l_all)


def test_draft_block_rows_see_each_other():
    """No causal mask inside the draft block: row 1 changes when later rows are added."""
    tm, dm, T, D, dw, taps = _draft_pair()
    D.draft_append(taps)
    _, l8 = D.draft_block(T, 8, 3, 1.0, tm.vocab - 1, with_logits=True)
    _, l4 = D.draft_block(T, 4, 3, 1.0, tm.vocab - 1, with_logits=True)
    assert not np.array_equal(l8[0], l4[0])
    assert rel_l1(l8[0], l4[0]) < 1.0


def test_rmsnorm_eps_matters_for_small_inputs():
    # mean square 1e-6 and eps 1e-6: scale 1/sqrt(2e-6) (without eps it would be 1/sqrt(1e-6))
    x = np.full(32, 1e-3, dtype=np.float32)
    g = synth.bf16_bits(np.ones(32))
    out = synth.bf16_to_f32(oracle.rmsnorm_bf16(x, g, eps=1e-6))
    ms = float(np.mean(x.astype(np.float64) ** 2))
    assert np.all(out == synth.bf16_to_f32(synth.bf16_bits(np.float64(x[0]) / math.sqrt(ms + 1e-6))))
    assert abs(float(out[0]) - 0.7071) < 0.003


def test_attention_ignores_positions_after_the_row():
    """Causal: a row at position p reads keys j <= p only, whatever the plane holds beyond p."""
    m = synth.tiny_model()
    om = oracle.Model(m, zero_weights(m))
    kv = _planes(m, 21)
    om.set_kv(kv, 21)
    q = np.random.default_rng(13).standard_normal(256).astype(np.float32)
    base = om.attend(0, q, 10)
    kv[0][11:] += 50.0
    om.set_kv(kv, 21)
    assert np.array_equal(om.attend(0, q, 10), base)
    kv[0][10, 1] += 1.0
    om.set_kv(kv, 21)
    assert not np.array_equal(om.attend(0, q, 10), base)


def test_embedded_entries_equal_token_entries():
    """The injected-row hooks are the token paths with the embedding rows given explicitly."""
    m, w, kv = _two_width(positions=5)
    toks = synth.tokens(0, "pin.embedded", 4, m.vocab)
    A = oracle.Model(m, w); A.set_kv(kv, 5)
    B = oracle.Model(m, w); B.set_kv(kv, 5)
    la, ta = A.verify_batch(toks, with_taps=True)
    lb, tb = B.verify_embedded(synth.bf16_to_f32(w["embed"][toks]), with_taps=True)
    assert np.array_equal(la, lb) and np.array_equal(ta, tb) and B.held() == 9
    tm, dm, T, D, dw, taps = _draft_pair()
    D.draft_append(taps)
    p1, l1 = D.draft_block(T, 8, 3, 0.5, tm.vocab - 1, with_logits=True)
    x0 = synth.bf16_to_f32(T._keep[2]["embed"][[3] + [tm.vocab - 1] * 7]) * np.float32(0.5)
    p2, l2 = oracle.draft_block_embedded(D, T, x0)
    assert np.array_equal(l1, l2) and np.array_equal(p1, p2)


# ------------------------------------------------------------------------------------------
# Sampled verify: Philox4x32-10 uniforms, Gumbel-max draws, the sampled accept
# ------------------------------------------------------------------------------------------
def test_philox_known_answers():
    """The generator against the published known-answer vectors of Philox4x32-10."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["counter"]]
        key = [int(x, 16) for x in v["key"]]
        out = oracle.philox4x32_10(ctr, key)
        assert ["%08x" % x for x in out] == v["out"]


@pytest.mark.parametrize("temperature", [0.7, 2.0])
def test_sampled_draws_follow_softmax_of_logits_over_temperature(temperature):
    """60000 draws of one row (row index i of the counter = draw i): the counts against
    softmax(z / T) by a chi-square test at df = 5 (the 1e-6 quantile is 35.9). A sign error in the
    Gumbel noise, a missing temperature or a biased uniform fails it."""
    z = np.array([0.5, -1.0, 2.0, 0.0, 1.5, -0.3], dtype=np.float32)
    n = 60000
    y = oracle.sample_rows(np.repeat(z[None, :], n, axis=0), temperature, 12345, 7)
    cnt = np.bincount(y, minlength=6)
    p = np.exp(z.astype(np.float64) / temperature)
    p /= p.sum()
    chi2 = float(((cnt - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 35.9, (cnt, n * p)
    # the other temperature's distribution is rejected (the test has power)
    q = np.exp(z.astype(np.float64) / (temperature * 3.0))
    q /= q.sum()
    assert float(((cnt - n * q) ** 2 / (n * q)).sum()) > 200.0


def test_sampled_draws_depend_on_seed_offset_and_row_only():
    z = synth.f32_normal(0, "pins.sample.z", (3, 1000)).astype(np.float32)
    a = oracle.sample_rows(z, 1.0, 1, 2)
    assert np.array_equal(a, oracle.sample_rows(z, 1.0, 1, 2))           # deterministic
    same = oracle.sample_rows(np.repeat(z[1:2], 64, 0), 1.0, 1, 2)
    assert len(set(same.tolist())) > 1                                     # each row draws anew
    assert not np.array_equal(oracle.sample_rows(np.repeat(z[:1], 64, 0), 1.0, 1, 2),
                              oracle.sample_rows(np.repeat(z[:1], 64, 0), 1.0, 1, 3))   # offset matters
    assert not np.array_equal(oracle.sample_rows(np.repeat(z[:1], 64, 0), 1.0, 1, 2),
                              oracle.sample_rows(np.repeat(z[:1], 64, 0), 1.0, 2, 2))   # seed matters


def test_sampled_scores_closed_form():
    """One score written out from the definition: word j % 4 of the Philox block at counter
    (j / 4, row, offset), u = (x >> 9 + 1/2) / 2^23, score = z / T - log(-log u), in fp32."""
    z = np.linspace(-3, 3, 11).astype(np.float32)
    T, seed, offset, row = 0.8, 0x1234567890ABCDEF, 0x0000000100000002, 3
    sc = oracle.sample_scores(z, T, seed, offset, row)
    for j in range(11):
        x = oracle.philox4x32_10([j // 4, row, offset & 0xFFFFFFFF, offset >> 32], [seed & 0xFFFFFFFF, seed >> 32])[j % 4]
        u = ((int(x) >> 9) + 0.5) / 2.0 ** 23
        expect = float(z[j]) / T - math.log(-math.log(u))
        assert abs(float(sc[j]) - expect) < 1e-5 * max(1.0, abs(expect))


def test_gumbel_noise_is_finite_at_the_extreme_words():
    """Every generator word gives a finite noise: u stays inside (0, 1) after the fp32 conversion
    (the largest word must not round to u = 1, where -log(-log u) is infinite and that entry would
    win every draw), and the noise grows with the word."""
    words = [0, 1, 511, 512, 2 ** 31, 0xFFFFFDFF, 0xFFFFFE00, 0xFFFFFFFE, 0xFFFFFFFF]
    g = [oracle.gumbel_of_word(x) for x in words]
    assert all(math.isfinite(v) for v in g), g
    assert g == sorted(g)
    assert g[-1] < 17.0 and g[0] > -3.0                  # u in [2^-24, 1 - 2^-24]
    for x in (0, 0xFFFFFFFF):
        u = ((x >> 9) + 0.5) / 2.0 ** 23
        assert abs(oracle.gumbel_of_word(x) + math.log(-math.log(u))) < 1e-5 * 17


def test_sampled_small_temperature_is_greedy():
    """T -> 0: the Gumbel noise (|g| < 18 for u in (2^-25, 1 - 2^-25)) is negligible next to
    (z_max - z_second) / T, so the draw is the argmax."""
    z = synth.f32_normal(0, "pins.sample.greedy", (8, 2000)).astype(np.float32)
    top2 = np.sort(z, axis=1)[:, -2:]
    assert np.all(top2[:, 1] - top2[:, 0] > 1e-4)
    y = oracle.sample_rows(z, 1e-6, 99, 0)
    assert np.array_equal(y, np.argmax(z, axis=1))


def test_sampled_accept_with_concentrated_rows():
    """Rows whose mass sits on one token (z = 60 there, 0 elsewhere, T = 1: every other token has
    probability below e^-50) accept exactly like the greedy accept; the accept stops at the first
    row whose draw differs from the next draft, and that draw is emitted."""
    k, V = 6, 50
    lg = np.zeros((k, V), dtype=np.float32)
    target = [3, 7, 11, 13, 17, 19]
    for i, t in enumerate(target):
        lg[i, t] = 60.0
    for mism in range(k):
        toks = np.array([1] + target[:5], dtype=np.int32)
        if mism < k - 1:
            toks[mism + 1] = 0
        a, em, draws = oracle.accept_sampled(lg, toks, 1.0, 5, 9)
        assert draws.tolist() == target
        ga, gem = oracle.accept_greedy(lg, toks)
        assert (a, em.tolist()) == (ga, gem.tolist())
        assert a == min(mism, k - 1)
        assert em.tolist() == target[:a] + [target[a]]


# ------------------------------------------------------------------------------------------
# bf16 K/V planes (memory variant)
# ------------------------------------------------------------------------------------------
def _bf16_model(m):
    import dataclasses
    return dataclasses.replace(m, kv_bf16=1)


def test_bf16_planes_round_to_nearest_even_on_store():
    """Cached rows are stored rounded to bf16 (RNE from fp32): 1 + 2^-10 -> 1; the tie 1 + 2^-8
    -> 1 (even); the tie 1 + 3 2^-8 -> 1 + 2^-6 (even); -2.75 stays (exact)."""
    m = _bf16_model(synth.tiny_model(max_ctx=8))
    o = oracle.Model(m, zero_weights(m))
    kv = np.zeros((2, 2, m.kv_width(0)), dtype=np.float32)
    vals = [1 + 2 ** -10, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.75]
    kv[0, 0, :4] = vals
    o.set_kv([kv], 2)
    got = o.plane(0, 2)[0, 0, :4].tolist()
    assert got == [1.0, 1.0, 1 + 2 ** -6, -2.75]


def test_bf16_planes_single_key_returns_rounded_value():
    """One visible key: attention returns its value row as stored, i.e. bf16(v)."""
    m = _bf16_model(synth.tiny_model(max_ctx=8))
    om = oracle.Model(m, zero_weights(m))
    kv = np.zeros((1, 2, m.kv_width(0)), dtype=np.float32)
    kv[0, 1, :] = 1 + 2 ** -10                                # V row
    om.set_kv([kv], 1)
    out = om.attend(0, np.ones(256, dtype=np.float32), 0)
    assert np.all(out == 1.0)


def test_bf16_planes_appended_rows_are_the_fp32_rows_rounded():
    """A verify on bf16 planes stores each new K/V value as bf16 of the value the fp32 planes
    store (same weights, same rows); the cached rows stay bf16 of their input."""
    m32 = synth.tiny_two_width_model(max_ctx=64)
    m16 = _bf16_model(m32)
    w = synth.make_weights(m32)
    kv = synth.make_kv(m32, 10)
    toks = synth.tokens(0, "pins.bf16kv", 5, m32.vocab)
    a, b = oracle.Model(m32, w), oracle.Model(m16, w)
    a.set_kv(kv, 10)
    b.set_kv(kv, 10)
    a.verify_batch(toks)
    b.verify_batch(toks)
    r16 = lambda x: synth.bf16_to_f32(synth.bf16_bits(x.astype(np.float64)))
    for l in range(m32.n_layers):
        if not m32.own(l):
            continue
        pa, pb = a.plane(l, 15), b.plane(l, 15)
        assert np.array_equal(pb[:10], r16(pa[:10]))
        # layer 0's new rows see identical inputs on both models; later layers' inputs differ
        if l == 0:
            assert np.array_equal(pb[10:], r16(pa[10:]))
        assert np.array_equal(pb, r16(pb))


def test_snapshot_refused_while_a_verify_is_pending():
    """A snapshot is of committed state: between a verify and its commit it is refused and nothing
    changes, so the commit that follows still cuts the verify's rows (3 held + 4 verified,
    commit 2 -> 5 held, engine PR #2303 "Proof")."""
    m, w, kv = _two_width(positions=3)
    A = oracle.Model(m, w)
    A.set_kv(kv, 3)
    A.verify_batch(synth.tokens(0, "pin.snap.pending", 4, m.vocab))
    with pytest.raises(RuntimeError):
        A.snapshot()
    assert A.held() == 7
    assert A.commit_verify_rows(2) == 0 and A.held() == 5
    snap = A.snapshot()
    assert snap.floats() == [5 * 2 * m.kv_width(l) if m.own(l) else 0 for l in range(m.n_layers)]

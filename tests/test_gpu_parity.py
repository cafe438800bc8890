"""GPU parity of the HIP path against the CPU oracle, through the C ABI (small and ragged shapes).

Bars: dequantised weights, KV position counts, accepted lengths and emitted tokens bit-exact;
logits rel-L1 <= 2e-3 per row (sum|g - o| / sum|o|); GEMM outputs and K/V planes to fp32
accumulation-order tolerance."""
import dataclasses

import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.util import golden, noise_floor, rel_l1

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-3          # rel-L1 per row, bf16 inputs with fp32 accumulation
GEMM_TOL = 2e-5           # rel-L1 per row of a single GEMM (fp32 vs fp64 accumulation order)


def stack_tol(run_oracle, arrays):
    """Three times the oracle's own spread under fp32-level perturbation of its inputs, never below
    2e-3 (the bar of the tiny multi-layer stacks, see stack_bar). run_oracle(arrays) -> logits."""
    return max(LOGIT_TOL, 3.0 * noise_floor(run_oracle, arrays))


# Models whose logits take the fixed 2e-3 bar: the single-layer decoder of config 1 (and any
# single-layer model), the target-shaped stack of configs 3 and 4, and the full-size draft.
FIXED_BAR_MODELS = ("target", "draft")


def logits_bar(err, m, run_oracle, arrays, label=""):
    """The logits bar of one comparison, printed with the error.

    Fixed 2e-3 (rel-L1 per row) for config 1, the target-shaped stack and the full-size draft.
    Documented exception, the tiny multi-layer stacks (the 6-layer two-width miniature, the
    3-layer ragged model, the 2-layer tiny draft): there a single bf16 rounding flip of an attention
    output or SwiGLU product between two correct fp32 summation orders moves a row by about 1e-3
    with these weight distributions, and flips add up over the layers; their bar is
    max(2e-3, 3 x the oracle's own spread under a 1e-5 relative input perturbation), and the spread
    is printed with every comparison."""
    if m.n_layers == 1 or m.name in FIXED_BAR_MODELS:
        print(f"[bar] {m.name} {label}: logits rel-L1 {err:.2e}, fixed bar {LOGIT_TOL:.1e}")
        return LOGIT_TOL
    tol = stack_tol(run_oracle, arrays)
    print(f"[bar] {m.name} {label}: logits rel-L1 {err:.2e}, stack bar {tol:.2e}")
    return tol


def embed_rows(w, toks):
    return synth.bf16_to_f32(w["embed"][np.asarray(toks)]).astype(np.float32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    bvf.lib()
    yield
    torch.cuda.synchronize()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ragged_model(max_ctx=96):
    """Shapes that leave ragged tiles and splits: hidden 384 (3 superblocks), FFN 640 (5)."""
    layers = (synth.Layer(synth.ATTN_SLIDING, 1, 64, 12, 640, -1), synth.Layer(synth.ATTN_FULL, 2, 64, 0, 384, -1),
              synth.Layer(synth.ATTN_SLIDING, 1, 64, 12, 640, 0))
    return synth.Model("ragged", 3, 384, 4, 528, max_ctx, layers, tap_layers=(0, 2))


def build_pair(m, P, seed=0):
    w = synth.make_weights(m, seed)
    kv = synth.make_kv(m, P, seed)
    g = bvf.Model(m)
    g.load_weights(w)
    g.set_context(kv, P)
    o = oracle.Model(m, w)
    o.set_kv(kv, P)
    return g, o, w, kv


# ------------------------------------------------------------------------------------------
# kernels
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("mk", [synth.tiny_two_width_model, ragged_model])
def test_dequant_bit_exact(mk):
    m = mk()
    g, o, w, kv = build_pair(m, 4)
    for l in range(m.n_layers):
        for key, (n_out, n_in) in synth.layer_matrix_shapes(m, l).items():
            out = torch.empty((n_out, n_in), dtype=torch.float32, device="cuda")
            g.q4_1_dequant(l, bvf.MATRIX_IDS[key], out)
            ref = oracle.q4_1_dequant(w["layers"][l][key], n_out, n_in)
            assert np.array_equal(host(out), ref), f"layer {l} {key}"


@pytest.mark.parametrize("rows", [1, 3, 8, 16, 17, 32, 45, 64])
@pytest.mark.parametrize("mk", [synth.tiny_two_width_model, ragged_model])
def test_q4_1_gemm_parity(mk, rows):
    m = mk()
    g, o, w, kv = build_pair(m, 4)
    for l in range(m.n_layers):
        for key, (n_out, n_in) in synth.layer_matrix_shapes(m, l).items():
            x = synth.bf16_normal(rows, f"gemm.x.{l}.{key}", (rows, n_in))
            y = torch.empty((rows, n_out), dtype=torch.float32, device="cuda")
            g.q4_1_gemm(l, bvf.MATRIX_IDS[key], dev(x), rows, y)
            ref = oracle.q4_1_matmul(w["layers"][l][key], n_out, n_in, x)
            assert rel_l1(host(y), ref) < GEMM_TOL, f"layer {l} {key} rows {rows}"


def test_q4_1_gemm_hand_off_diagonal():
    """One nonzero weight at (n=5, k=40) of the tiny model's down projection input side."""
    m = synth.tiny_model()
    w = synth.make_weights(m)
    W = np.zeros((256, 512), dtype=np.int64)
    W[5, 40] = 3
    nb = 512 // 32
    w["layers"][0]["down"] = synth.q4_1_from_parts(W, np.full((256, nb), 0.25), np.zeros((256, nb)))
    g = bvf.Model(m)
    g.load_weights(w)
    x = synth.bf16_normal(0, "hand.x", (2, 512))
    y = torch.empty((2, 256), dtype=torch.float32, device="cuda")
    g.q4_1_gemm(0, bvf.DOWN, dev(x), 2, y)
    y = host(y)
    xf = synth.bf16_to_f32(x)
    assert np.all(y[:, 5] == np.float32(0.75) * xf[:, 40])
    y[:, 5] = 0
    assert not y.any()


# ------------------------------------------------------------------------------------------
# the verify pass
# ------------------------------------------------------------------------------------------
def run_verify(g, m, toks, with_taps=True):
    k = len(toks)
    lg = torch.empty((k, m.vocab), dtype=torch.float32, device="cuda")
    taps = torch.empty((k, len(m.tap_layers), m.hidden), dtype=torch.int16, device="cuda") if with_taps else None
    g.verify_batch(dev(toks), lg, taps)
    return host(lg), (host(taps).view(np.uint16) if with_taps else None)


def compare_taps(got, ref, tol):
    a = synth.bf16_to_f32(got).astype(np.float64)
    b = synth.bf16_to_f32(ref).astype(np.float64)
    err = rel_l1(a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1]))
    print(f"taps rel-L1 {err:.2e}")
    assert err < tol


@pytest.mark.parametrize("mk, P, k", [(synth.tiny_model, 64, 8), (synth.tiny_two_width_model, 40, 8),
                                      (synth.tiny_two_width_model, 0, 5), (ragged_model, 30, 16),
                                      (ragged_model, 7, 1)])
def test_verify_parity(mk, P, k):
    m = mk()
    g, o, w, kv = build_pair(m, P)
    toks = synth.tokens(0, f"verify.{m.name}", k, m.vocab)
    lg, taps = run_verify(g, m, toks)
    rlg, rtaps = o.verify_batch(toks, with_taps=True)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], P)
        return x.verify_embedded(arrs[0])

    err = rel_l1(lg, rlg)
    tol = logits_bar(err, m, run_oracle, [embed_rows(w, toks)] + kv, f"verify P={P} k={k}")
    assert err < tol
    if m.tap_layers:
        compare_taps(taps, rtaps, tol)
    assert g.positions_held() == o.held() == P + k
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    assert np.array_equal(g.kv_widths(), o.kv_widths())
    # greedy tokens agree wherever the top-2 margin is clear
    for i in range(k):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert lg[i].argmax() == rlg[i].argmax()


def test_verify_parity_config1_logits_tight():
    """Config 1 (tiny Qwen3-style decoder, 64 cached positions, k = 8, seed 0): the rows agree to
    fp32 accumulation order (far inside the 2e-3 bar)."""
    m = synth.tiny_model()
    g, o, w, kv = build_pair(m, 64)
    toks = synth.tokens(0, "config1.tokens", 8, m.vocab)
    lg, _ = run_verify(g, m, toks, with_taps=False)
    rlg = o.verify_batch(toks)
    err = rel_l1(lg, rlg)
    print(f"config 1 logits rel-L1 {err:.2e}")
    assert err < LOGIT_TOL


@pytest.mark.parametrize("mk, P, k", [(synth.tiny_two_width_model, 40, 8), (ragged_model, 30, 16),
                                      (synth.tiny_two_width_model, 3, 1)])
def test_layer_by_layer_parity(mk, P, k):
    """Teacher-forced: every layer gets the same input rows on both sides, so no error carries
    from layer to layer. The layer's contribution (x_out - x_in) must agree per row, within the
    2e-3 bar or three times the oracle's own spread under fp32-level input perturbation: a single
    bf16 rounding flip of the attention output or the SwiGLU product already moves a row's
    contribution by 1e-3 .. 2e-3 with these weight distributions."""
    m = mk()
    g, o, w, kv = build_pair(m, P)
    pos = np.arange(P, P + k)
    for l in range(m.n_layers):
        x = (synth.f32_normal(l, f"layer.x.{m.name}", (k, m.hidden)) * 3.0).astype(np.float32)
        xg = dev(x)
        g.layer_forward(l, xg, k)
        xo = o.layer_forward(l, x, pos)
        got = host(xg).astype(np.float64) - x
        ref = xo.astype(np.float64) - x
        err = rel_l1(got, ref)

        def run_oracle(arrs, l=l):
            xx = oracle.Model(m, w)
            xx.set_kv(arrs[1:], P)
            return xx.layer_forward(l, arrs[0], pos).astype(np.float64) - x

        tol = max(LOGIT_TOL, 3.0 * noise_floor(run_oracle, [x] + list(kv)))
        print(f"layer {l}: contribution rel-L1 {err:.2e} (bar {tol:.2e})")
        assert err < tol, f"layer {l}"


# ------------------------------------------------------------------------------------------
# accept
# ------------------------------------------------------------------------------------------
def accept_gpu(g, lg_dev, toks):
    out = torch.zeros(len(toks), dtype=torch.int32, device="cuda")
    na = torch.zeros(1, dtype=torch.int32, device="cuda")
    g.accept_greedy(lg_dev, dev(toks), out, na)
    a = int(host(na)[0])
    return a, host(out)[: a + 1]


def test_accept_constructed_mismatch_positions():
    m = synth.tiny_model()
    g = bvf.Model(m)
    g.load_weights(synth.make_weights(m))
    rng = np.random.default_rng(5)
    k, V = 8, m.vocab
    lg = rng.standard_normal((k, V)).astype(np.float32)
    y = lg.argmax(axis=1)
    for j in range(k):
        toks = np.zeros(k, dtype=np.int32)
        toks[0] = 3
        toks[1:j + 1] = y[:j]
        if j + 1 < k:
            toks[j + 1] = (y[j] + 1) % V
            toks[j + 2:] = y[j + 1:k - 1]
        a, out = accept_gpu(g, dev(lg), toks)
        ra, rout = oracle.accept_greedy(lg, toks)
        assert a == ra == j
        assert out.tolist() == rout.tolist()


def test_accept_ties_and_nan():
    m = synth.tiny_model()
    g = bvf.Model(m)
    g.load_weights(synth.make_weights(m))
    lg = np.zeros((2, m.vocab), dtype=np.float32)
    lg[0, 700] = lg[0, 300] = 5.0            # tie: the lower id wins
    lg[0, 0] = np.nan                        # NaN never wins
    lg[1, :] = np.nan                        # all NaN: id 0
    toks = np.array([1, 300], dtype=np.int32)
    a, out = accept_gpu(g, dev(lg), toks)
    assert (a, out.tolist()) == (1, [300, 0])
    assert oracle.accept_greedy(lg, toks)[0] == 1


def test_accept_after_verify_and_steering():
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, 20)
    toks = synth.tokens(0, "steer.toks", 8, m.vocab)
    lg = torch.empty((8, m.vocab), dtype=torch.float32, device="cuda")
    g.verify_batch(dev(toks), lg, None)
    # steer: rows 0..2 get a bonus on the next draft, row 3 a penalty on its draft
    a_target = 3
    tok = np.array([toks[i + 1] for i in range(7)] + [0], dtype=np.int32)
    add = np.array([1e4] * a_target + [-1e4] + [0.0] * 4, dtype=np.float32)
    g.steer_logits(lg, dev(tok), dev(add))
    a, out = accept_gpu(g, lg, toks)
    ref = o.verify_batch(toks)
    for i in range(8):
        ref[i, tok[i]] += add[i]
    ra, rout = oracle.accept_greedy(ref, toks)
    assert a == ra == a_target
    assert out[:a].tolist() == toks[1:a + 1].tolist()
    assert out.tolist() == rout.tolist()


# ------------------------------------------------------------------------------------------
# commit / rollback / snapshot (per-layer widths, shared planes)
# ------------------------------------------------------------------------------------------
def test_commit_worked_case_and_next_step():
    gc = golden("commit_worked_case")
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, gc["prefix"])
    toks = synth.tokens(0, "commit.toks", gc["k"], m.vocab)
    run_verify(g, m, toks, with_taps=False)
    g.commit_verify_rows(gc["commit"])
    assert g.positions_held() == gc["held_after"]
    floats = g.plane_floats()
    for l in range(m.n_layers):
        assert floats[l] == (gc["held_after"] * 2 * m.kv_width(l) if m.own(l) else 0)
    # the next pass equals a forward that only ever saw the accepted rows
    nxt = synth.tokens(1, "commit.next", 3, m.vocab)
    lg, _ = run_verify(g, m, nxt, with_taps=False)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], gc["prefix"])
        for t in toks[: gc["commit"]]:
            x.step(int(t))
        return x.verify_embedded(arrs[0])

    arrs = [embed_rows(w, nxt)] + kv
    err = rel_l1(lg, run_oracle(arrs))
    assert err < logits_bar(err, m, run_oracle, arrs, "commit worked case, next pass")


@pytest.mark.parametrize("n", range(0, 9))
def test_commit_every_n(n):
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, 24)
    toks = synth.tokens(0, "commit_n.toks", 8, m.vocab)
    run_verify(g, m, toks, with_taps=False)
    g.commit_verify_rows(n)
    assert g.positions_held() == 24 + n
    nxt = synth.tokens(2, "commit_n.next", 4, m.vocab)
    lg, _ = run_verify(g, m, nxt, with_taps=False)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], 24)
        for t in toks[:n]:
            x.step(int(t))
        return x.verify_embedded(arrs[0])

    arrs = [embed_rows(w, nxt)] + kv
    err = rel_l1(lg, run_oracle(arrs))
    assert err < logits_bar(err, m, run_oracle, arrs, f"commit({n}), next pass")


def test_commit_refusals_leave_state_unchanged():
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, 10)
    with pytest.raises(bvf.BvfError) as e:
        g.commit_verify_rows(0)
    assert e.value.status == bvf.BVF_E_STATE
    run_verify(g, m, np.array([1, 2, 3], dtype=np.int32), with_taps=False)
    with pytest.raises(bvf.BvfError) as e:
        g.commit_verify_rows(4)
    assert e.value.status == bvf.BVF_E_STATE
    assert g.positions_held() == 13
    g.commit_verify_rows(3)
    with pytest.raises(bvf.BvfError):
        g.commit_verify_rows(1)
    with pytest.raises(bvf.BvfError) as e:
        run_verify(g, m, np.zeros(17, dtype=np.int32), with_taps=False)
    assert e.value.status == bvf.BVF_E_INVALID
    assert g.positions_held() == 13


def test_capacity_refusal():
    m = synth.tiny_model(max_ctx=70)
    g, o, w, kv = build_pair(m, 64)
    with pytest.raises(bvf.BvfError) as e:
        run_verify(g, m, np.zeros(8, dtype=np.int32), with_taps=False)
    assert e.value.status == bvf.BVF_E_CAPACITY
    assert g.positions_held() == 64


def test_snapshot_restore_per_layer_widths():
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, 18)
    snap = g.snapshot_take()
    assert snap.floats().tolist() == [18 * 2 * m.kv_width(l) if m.own(l) else 0 for l in range(m.n_layers)]
    run_verify(g, m, synth.tokens(0, "snap.a", 6, m.vocab), with_taps=False)
    g.commit_verify_rows(6)
    g.restore(snap)
    assert g.positions_held() == 18
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    toks = synth.tokens(0, "snap.b", 5, m.vocab)
    lg, _ = run_verify(g, m, toks, with_taps=False)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], 18)
        return x.verify_embedded(arrs[0])

    arrs = [embed_rows(w, toks)] + kv
    err = rel_l1(lg, run_oracle(arrs))
    assert err < logits_bar(err, m, run_oracle, arrs, "after snapshot restore")
    # a snapshot of another geometry is refused
    m2 = synth.tiny_model(max_ctx=m.max_ctx)
    g2 = bvf.Model(m2)
    with pytest.raises(bvf.BvfError) as e:
        g2.restore(snap)
    assert e.value.status == bvf.BVF_E_INVALID


def test_snapshot_refused_while_a_verify_is_pending():
    """Both sides refuse a snapshot between a verify and its commit, with no state change; the
    commit that follows cuts the verify's rows on both (3 held + 4 verified, commit 2 -> 5)."""
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, 3)
    toks = synth.tokens(0, "snap.pending", 4, m.vocab)
    run_verify(g, m, toks, with_taps=False)
    o.verify_batch(toks)
    with pytest.raises(bvf.BvfError) as e:
        g.snapshot_take()
    assert e.value.status == bvf.BVF_E_STATE
    with pytest.raises(RuntimeError):
        o.snapshot()
    assert g.positions_held() == o.held() == 7
    g.commit_verify_rows(2)
    assert o.commit_verify_rows(2) == 0
    assert g.positions_held() == o.held() == 5
    assert np.array_equal(g.plane_floats(), o.plane_floats())
    assert np.array_equal(g.snapshot_take().floats(), o.snapshot().floats())


def test_shared_layers_read_owner_planes():
    """Perturbing an owner's cached plane changes the logits; shared planes stay empty."""
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, 12)
    toks = synth.tokens(0, "shared.toks", 4, m.vocab)
    lg0, _ = run_verify(g, m, toks, with_taps=False)
    assert all(g.plane_floats()[l] == 0 for l in range(m.n_layers) if not m.own(l))
    kv2 = [None if a is None else a.copy() for a in kv]
    kv2[3][:, 1] += 0.5                    # layer 3 owns layer 4's keys
    g2, o2, _, _ = build_pair(m, 12)
    g2.set_context(kv2, 12)
    o2.set_kv(kv2, 12)
    lg1, _ = run_verify(g2, m, toks, with_taps=False)

    def run_oracle(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs[1:], 12)
        return x.verify_embedded(arrs[0])

    arrs = [embed_rows(w, toks)] + kv2
    err = rel_l1(lg1, run_oracle(arrs))
    tol = logits_bar(err, m, run_oracle, arrs, "shared layers, perturbed owner plane")
    assert err < tol
    assert rel_l1(lg1, lg0) > 3 * tol


# ------------------------------------------------------------------------------------------
# DFlash draft block
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window, n_ctx, n_new, block", [(0, 12, 4, 8), (6, 20, 3, 8), (0, 0, 8, 8), (0, 9, 1, 4),
                                                     (0, 30, 0, 8), (0, 10, 4, 12), (0, 10, 0, 16), (5, 14, 7, 9)])
def test_draft_block_parity(window, n_ctx, n_new, block):
    """Context: n_ctx rows of cached draft K/V (set directly) plus n_new rows appended from taps;
    then the block [17, mask x (block - 1)] and the target head on rows 1.."""
    tm = synth.tiny_model(max_ctx=64)
    tw = synth.make_weights(tm)
    dm = synth.tiny_draft_model(max_ctx=64, window=window)
    dmg = dataclasses.replace(dm, vocab=tm.vocab)      # the draft's logits scratch takes the target's vocab
    dw = synth.make_weights(dm)
    kvd = synth.make_kv(dm, n_ctx)
    taps = synth.bf16_normal(0, "draft.taps", (n_new, len(dm.tap_layers), dm.hidden))
    T = bvf.Model(tm)
    T.load_weights(tw)
    D = bvf.Model(dmg)
    D.load_weights(dw)
    D.set_context(kvd, n_ctx)
    To = oracle.Model(tm, tw)
    props = torch.zeros(block - 1, dtype=torch.int32, device="cuda")
    lg = torch.empty((block - 1, tm.vocab), dtype=torch.float32, device="cuda")
    last = dev(np.array([17], dtype=np.int32))
    D.draft_block_forward(T, dev(taps) if n_new else None, n_new, last, block, 1.0, tm.vocab - 1, props, lg)
    assert D.positions_held() == n_ctx + n_new

    x0 = embed_rows(tw, [17] + [tm.vocab - 1] * (block - 1))

    def run_oracle(arrs):
        Do = oracle.Model(dm, dw)
        Do.set_kv(arrs[1:], n_ctx)
        if n_new:
            Do.draft_append(taps)
        return oracle.draft_block_embedded(Do, To, arrs[0])

    rp, rlg = run_oracle([x0] + kvd)
    glg = host(lg)
    err = rel_l1(glg, rlg)
    tol = logits_bar(err, dm, lambda a: run_oracle(a)[1], [x0] + kvd, f"draft block w={window} ctx={n_ctx} new={n_new} B={block}")
    assert err < tol
    gp = host(props)
    for i in range(block - 1):
        top2 = np.sort(rlg[i])[-2:]
        if top2[1] - top2[0] > 0.02 * np.sqrt(np.mean(rlg[i].astype(np.float64) ** 2)):
            assert gp[i] == rp[i]


def test_draft_append_only_then_block():
    """block = 0 appends context rows only; a later block sees them like rows appended with a block."""
    tm = synth.tiny_model(max_ctx=64)
    tw = synth.make_weights(tm)
    dm = synth.tiny_draft_model(max_ctx=64)
    dmg = dataclasses.replace(dm, vocab=tm.vocab)
    dw = synth.make_weights(dm)
    taps = synth.bf16_normal(1, "draft.taps2", (20, len(dm.tap_layers), dm.hidden))
    T = bvf.Model(tm)
    T.load_weights(tw)
    D = bvf.Model(dmg)
    D.load_weights(dw)
    D.set_positions(0)
    D.draft_block_forward(T, dev(taps[:16]), 16, None, 0, 1.0, 0, None, None)
    assert D.positions_held() == 16
    props = torch.zeros(7, dtype=torch.int32, device="cuda")
    lg = torch.empty((7, tm.vocab), dtype=torch.float32, device="cuda")
    D.draft_block_forward(T, dev(taps[16:]), 4, dev(np.array([5], dtype=np.int32)), 8, 1.0, tm.vocab - 1, props, lg)
    To = oracle.Model(tm, tw)

    def run_oracle(arrs):
        Do = oracle.Model(dm, dw)
        Do.draft_append(taps)
        return oracle.draft_block_embedded(Do, To, arrs[0])[1]

    arrs = [embed_rows(tw, [5] + [tm.vocab - 1] * 7)]
    err = rel_l1(host(lg), run_oracle(arrs))
    assert err < logits_bar(err, dm, run_oracle, arrs, "draft append-only then block")


def test_draft_graph_replay_matches_direct_launches():
    """The draft block replayed from graphs (one capture per context-row count, the positions read
    from device memory) gives bit-identical proposals, logits and appended K/V rows to a twin with
    direct launches, over rounds of 1..8 new context rows with eager work between the replays."""
    tm = synth.tiny_model(max_ctx=160)
    tw = synth.make_weights(tm)
    dm = synth.tiny_draft_model(max_ctx=160, window=32)
    dmg = dataclasses.replace(dm, vocab=tm.vocab)
    dw = synth.make_weights(dm)
    kvd = synth.make_kv(dm, 24)
    T = bvf.Model(tm)
    T.load_weights(tw)
    Ds = []
    for graph in (False, True):
        D = bvf.Model(dmg)
        D.load_weights(dw)
        D.set_context(kvd, 24)
        D.set_graph_mode(graph)
        Ds.append(D)
    B = 8
    taps = dev(synth.bf16_normal(3, "draft.graph.taps", (B, len(dm.tap_layers), dm.hidden)))
    last = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = [(torch.zeros(B - 1, dtype=torch.int32, device="cuda"), torch.empty((B - 1, tm.vocab), dtype=torch.float32, device="cuda"))
           for _ in Ds]
    n_news = [1, 4, 8, 4, 2, 1, 7, 4, 3, 8, 5, 6, 1]
    x = dev(synth.bf16_normal(0, "draft.graph.x", (8, tm.hidden)))
    y = torch.empty((8, 256), dtype=torch.float32, device="cuda")
    for r, n_new in enumerate(n_news):
        last.fill_(5 + 3 * r)
        taps.copy_(dev(synth.bf16_normal(10 + r, "draft.graph.taps", (B, len(dm.tap_layers), dm.hidden))))
        for D, (props, lg) in zip(Ds, out):
            lg.fill_(float("nan"))
            D.draft_block_forward(T, taps[:n_new], n_new, last, B, 1.0, tm.vocab - 1, props, lg)
            T.q4_1_gemm(0, bvf.Q, x, 8, y)      # eager work between replays
        assert np.array_equal(host(out[0][1]), host(out[1][1])), f"round {r} (n_new {n_new}) logits"
        assert np.array_equal(host(out[0][0]), host(out[1][0])), f"round {r} proposals"
    held = Ds[0].positions_held()
    assert held == Ds[1].positions_held() == 24 + sum(n_news)
    for l in range(dm.n_layers):
        assert np.array_equal(Ds[0].get_kv(l, held), Ds[1].get_kv(l, held)), f"layer {l} plane"
    print(f"[draft graph] {len(n_news)} rounds, captures {Ds[1].graph_captures()}", flush=True)
    assert Ds[0].graph_captures() == 0 and Ds[1].graph_captures() == len(set(n_news))


# ------------------------------------------------------------------------------------------
# graph replay
# ------------------------------------------------------------------------------------------
def test_graph_replay_matches_direct_launches():
    """The captured pass replays bit-identically to direct launches, over several replays with
    other device work in between, and at other positions held."""
    m = synth.tiny_two_width_model()
    g, o, w, kv = build_pair(m, 20)
    toks = dev(synth.tokens(0, "graph.toks", 8, m.vocab))
    ref = torch.empty((8, m.vocab), dtype=torch.float32, device="cuda")
    g.verify_batch(toks, ref, None)
    g.commit_verify_rows(0)
    ref = host(ref)
    g.set_graph_mode(True)
    lg = torch.empty((8, m.vocab), dtype=torch.float32, device="cuda")
    x = dev(synth.bf16_normal(0, "graph.x", (8, m.hidden)))
    y = torch.empty((8, 2 * m.layers[0].n_kv_heads * 64 + 256), dtype=torch.float32, device="cuda")
    for rep in range(4):
        lg.fill_(float("nan"))
        g.verify_batch(toks, lg, None)
        g.commit_verify_rows(0)
        assert np.array_equal(host(lg), ref), f"replay {rep}"
        g.q4_1_gemm(0, bvf.Q, x, 8, y[:, :256])      # eager work between replays
        torch.cuda.synchronize()
    assert g.graph_captures() == 1
    # new positions (same 256-position span): the capture is replayed and still matches direct launches
    g.verify_batch(toks, lg, None)
    g.commit_verify_rows(3)
    g.verify_batch(toks, lg, None)
    got = host(lg)
    g.commit_verify_rows(0)
    assert g.graph_captures() == 1
    g.set_graph_mode(False)
    g.verify_batch(toks, lg, None)
    assert np.array_equal(host(lg), got)


def test_graph_serves_a_position_span_across_rounds():
    """A loop-shaped sequence on the two-width miniature (max_ctx 600): verifies of 8 rows with
    commits of 1..8 rows from 200 cached positions past 256 and 512. The graph model (positions read
    from device memory at replay) and a direct-launch twin give bit-identical logits and taps at every
    round, the graph is captured once per 256-position span (3 captures), the planes agree, and the
    last round's logits agree with the oracle replaying the same sequence."""
    m = synth.tiny_two_width_model(max_ctx=600)
    P = 200
    gd, o, w, kv = build_pair(m, P)
    gg = bvf.Model(m)
    gg.load_weights(w)
    gg.set_context(kv, P)
    gg.set_graph_mode(True)
    T = len(m.tap_layers)
    buf = lambda: (torch.empty((8, m.vocab), dtype=torch.float32, device="cuda"),
                   torch.empty((8, T, m.hidden), dtype=torch.int16, device="cuda"))
    (lgd, tpd), (lgg, tpg) = buf(), buf()
    toks = torch.empty(8, dtype=torch.int32, device="cuda")
    commits = [int(c) for c in synth.accept_lengths(0, 200, max_a=7) + 1]
    seq = []
    r = 0
    while gd.positions_held() + 8 <= 530:
        t = synth.tokens(r, "graph.span", 8, m.vocab)
        toks.copy_(torch.from_numpy(t))
        gd.verify_batch(toks, lgd, tpd)
        gg.verify_batch(toks, lgg, tpg)
        a, b = host(lgd), host(lgg)
        assert np.array_equal(a, b), f"round {r} at {gd.positions_held() - 8}"
        assert np.array_equal(host(tpd), host(tpg)), f"round {r} taps"
        n = commits[r]
        gd.commit_verify_rows(n)
        gg.commit_verify_rows(n)
        seq.append((t, n))
        r += 1
    held = gg.positions_held()
    print(f"[graph span] {r} rounds, positions {P} -> {held}, captures {gg.graph_captures()}", flush=True)
    assert held > 512 and gg.graph_captures() == 3
    assert np.array_equal(gg.plane_floats(), gd.plane_floats())
    for l in range(m.n_layers):
        if m.own(l):
            assert np.array_equal(gg.get_kv(l, held), gd.get_kv(l, held)), f"layer {l} plane"

    def run(arrs):
        x = oracle.Model(m, w)
        x.set_kv(arrs, P)
        for t, n in seq[:-1]:
            x.verify_batch(t)
            assert x.commit_verify_rows(n) == 0
        return x.verify_batch(seq[-1][0])

    err = rel_l1(b, run(kv))
    assert err < logits_bar(err, m, run, kv, f"graph replays over {r} rounds, last at {held - seq[-1][1]}")

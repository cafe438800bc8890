"""The sampled accept (temperature > 0) on the GPU against the oracle: every row's Gumbel-max draw
over Philox4x32-10 uniforms at the full 262144-entry vocabulary and at vocabularies with a ragged last span,
the accept decision on constructed drafts, the distribution of the draws, the refusals.

A draw is an argmax decided in fp32 on both sides; the two logf implementations may differ by an
ulp, so a row is compared exactly where its top-2 score margin is clear (more than a few ulps),
and elsewhere the GPU's draw must be one of the near-top entries."""
import numpy as np
import pytest

import oracle
from block_verify_forward_amd import bvf, synth
from tests.test_gpu_parity import dev, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def sampled_gpu(g, lg, toks, T, seed, offset):
    k = len(toks)
    out = torch.zeros(k, dtype=torch.int32, device="cuda")
    na = torch.zeros(1, dtype=torch.int32, device="cuda")
    draws = torch.full((k,), -1, dtype=torch.int32, device="cuda")
    g.accept_sampled(dev(lg), dev(np.asarray(toks, dtype=np.int32)), out, na, T, seed, offset, draws)
    a = int(host(na)[0])
    return a, host(out)[: a + 1], host(draws)


def check_draws(lg, T, seed, offset, gd):
    """Returns how many rows were compared exactly."""
    rd = oracle.sample_rows(lg, T, seed, offset)
    compared = 0
    for i in range(lg.shape[0]):
        sc = oracle.sample_scores(lg[i], T, seed, offset, i)
        top = np.sort(sc)[-2:]
        bar = 4e-6 * max(1.0, abs(float(top[1])))
        if top[1] - top[0] > bar:
            assert gd[i] == rd[i], f"row {i}"
            compared += 1
        else:
            assert sc[gd[i]] >= top[1] - bar, f"row {i}: not a near-top entry"
    return compared


@pytest.fixture(scope="module")
def full_vocab():
    return bvf.Model(synth.tiny_model(vocab=262144))


@pytest.mark.parametrize("T,seed,offset", [(1.0, 0, 0), (0.6, 12345, 7), (1.7, 2 ** 40 + 3, 2 ** 33 + 5)])
def test_sampled_draws_full_vocab(full_vocab, T, seed, offset):
    k, V = 8, 262144
    lg = (synth.f32_normal(0, f"sampled.full.{seed}", (k, V)) * 2.0).astype(np.float32)
    _, _, gd = sampled_gpu(full_vocab, lg, np.zeros(k, dtype=np.int32), T, seed, offset)
    assert check_draws(lg, T, seed, offset, gd) >= k - 1


@pytest.mark.parametrize("V", [16, 1008, 4112, 8208])
def test_sampled_draws_ragged_vocab(V):
    """Vocabularies (multiples of 16, as a model's vocabulary is) that leave a ragged last 4096-entry
    span, and a single 16-entry span; k = 16 rows."""
    g = bvf.Model(synth.tiny_model(vocab=V))
    k = 16
    lg = synth.f32_normal(0, f"sampled.ragged.{V}", (k, V)).astype(np.float32)
    _, _, gd = sampled_gpu(g, lg, np.zeros(k, dtype=np.int32), 0.9, 77, 11)
    assert check_draws(lg, 0.9, 77, 11, gd) >= k - 2


def test_sampled_accept_constructed_mismatch_positions(full_vocab):
    """Drafts equal to the oracle's draws up to position j, then different: the accepted length is j
    and the emitted tokens are the drafts plus row j's draw."""
    k, V = 8, 262144
    T, seed, offset = 0.8, 4242, 99
    lg = synth.f32_normal(0, "sampled.accept", (k, V)).astype(np.float32)
    y = oracle.sample_rows(lg, T, seed, offset)
    _, _, gd = sampled_gpu(full_vocab, lg, np.zeros(k, dtype=np.int32), T, seed, offset)
    assert check_draws(lg, T, seed, offset, gd) == k, "the rows of this case have clear margins"
    for j in range(k):
        toks = np.zeros(k, dtype=np.int32)
        toks[0] = 5
        toks[1:j + 1] = y[:j]
        if j + 1 < k:
            toks[j + 1] = (y[j] + 1) % V
            toks[j + 2:] = y[j + 1:k - 1]
        a, out, _ = sampled_gpu(full_vocab, lg, toks, T, seed, offset)
        ra, rout, _ = oracle.accept_sampled(lg, toks, T, seed, offset)
        assert a == ra == j
        assert out.tolist() == rout.tolist()


def test_sampled_draws_follow_softmax():
    """16 rows of the same 16 logits, 400 offsets: 6400 draws against softmax(z / T) by chi-square
    (df = 15; the 1e-6 quantile is 56.5), and the test's power: a wrong temperature is rejected."""
    g = bvf.Model(synth.tiny_model(vocab=16))
    z = np.linspace(-1.5, 2.2, 16).astype(np.float32)[np.argsort(np.arange(16) * 7 % 16)]
    T = 1.3
    lg = np.repeat(z[None, :], 16, axis=0)
    counts = np.zeros(16)
    for off in range(400):
        _, _, gd = sampled_gpu(g, lg, np.zeros(16, dtype=np.int32), T, 2024, off)
        counts += np.bincount(gd, minlength=16)

    def chi2(temp):
        p = np.exp(z.astype(np.float64) / temp)
        p /= p.sum()
        e = counts.sum() * p
        return float(((counts - e) ** 2 / e).sum())

    assert chi2(T) < 56.5, counts
    assert chi2(3 * T) > 150.0


def test_sampled_refusals():
    g = bvf.Model(synth.tiny_model())
    lg = np.zeros((2, 1024), dtype=np.float32)
    for T in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(Exception):
            sampled_gpu(g, lg, np.zeros(2, dtype=np.int32), T, 1, 1)


def test_sampled_dominant_token_always_drawn(full_vocab):
    """A token 5000 above every other (T = 1) is drawn in every row and at every counter offset:
    the noise is bounded (|g| < 17), so no other entry can win. 16 rows x 64 offsets x 262144
    entries; a mapping of the generator word that let u reach 1 (infinite noise) would fail here
    about 16 times."""
    k, V = 16, 262144
    lg = synth.f32_normal(0, "sampled.dominant", (k, V)).astype(np.float32)
    hot = (np.arange(k) * 9973 + 17) % V
    lg[np.arange(k), hot] += 5000.0
    for off in range(64):
        _, _, gd = sampled_gpu(full_vocab, lg, np.zeros(k, dtype=np.int32), 1.0, 99, off)
        assert np.array_equal(gd, hot), f"offset {off}"

"""Helpers shared by the tests: hand-built Q4_1 matrices, independent numpy decodes, tiny models."""
from __future__ import annotations

import json
import os

import numpy as np

from block_verify_forward_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        return json.load(f)[name]


def zero_q4(n_out: int, n_in: int) -> np.ndarray:
    """A Q4_1 image whose every weight is exactly 0 (scale 0, min 0)."""
    nb = n_in // 32
    return synth.q4_1_from_parts(np.zeros((n_out, n_in)), np.zeros((n_out, nb)), np.zeros((n_out, nb)))


def int_q4(w_int: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Q4_1 image of a matrix of small non-negative integers (codes, scale `scale`, min 0)."""
    w_int = np.asarray(w_int)
    n_out, n_in = w_int.shape
    nb = n_in // 32
    return synth.q4_1_from_parts(w_int, np.full((n_out, nb), scale), np.zeros((n_out, nb)))


def np_dequant(img: np.ndarray) -> np.ndarray:
    """Independent decode with numpy's own fp16 conversion: float64 [n_out, n_in]."""
    n_out, nb, _ = img.shape
    s = img[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    m = img[:, :, 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    lo = (img[:, :, 4:] & 15).astype(np.float64)
    hi = (img[:, :, 4:] >> 4).astype(np.float64)
    codes = np.concatenate([lo, hi], axis=2)          # [n_out, nb, 32]
    return (codes * s[..., None] + m[..., None]).reshape(n_out, nb * 32)


def f32_bits_of_bf16(b: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(b).astype(np.float64)


def zero_weights(m: synth.Model, seed: int = 0) -> dict:
    """Weights of model m with every Q4_1 matrix exactly zero; norms and embedding drawn as usual."""
    w = {"layers": []}
    for l in range(m.n_layers):
        d = {key: zero_q4(n_out, n_in) for key, (n_out, n_in) in synth.layer_matrix_shapes(m, l).items()}
        hd = m.layers[l].head_dim
        d["attn_norm"] = synth.bf16_uniform(seed, f"{m.name}.L{l}.attn_norm", (m.hidden,), 0.5, 1.5)
        d["mlp_norm"] = synth.bf16_uniform(seed, f"{m.name}.L{l}.mlp_norm", (m.hidden,), 0.5, 1.5)
        d["q_norm"] = synth.bf16_uniform(seed, f"{m.name}.L{l}.q_norm", (hd,), 0.5, 1.5)
        d["k_norm"] = synth.bf16_uniform(seed, f"{m.name}.L{l}.k_norm", (hd,), 0.5, 1.5)
        w["layers"].append(d)
    if m.vocab > 0:
        w["embed"] = synth.bf16_normal(seed, f"{m.name}.embed", (m.vocab, m.hidden))
    w["final_norm"] = synth.bf16_uniform(seed, f"{m.name}.final_norm", (m.hidden,), 0.5, 1.5)
    return w


def no_weights(m: synth.Model) -> dict:
    """An empty weight set: enough for the state bookkeeping (widths, cuts), never for a forward."""
    return {"layers": [{} for _ in range(m.n_layers)]}


def rel_l1(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of sum|g - o| / sum|o|."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.asarray(ref).shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    num = np.abs(got - ref).sum(axis=1)
    den = np.abs(ref).sum(axis=1)
    return float(np.max(num / np.maximum(den, 1e-300)))


def perturbed(kv_list, eps: float, seed: int):
    """Cached K/V with a relative perturbation of size eps (float64 draw, rounded back to fp32)."""
    rng = np.random.default_rng(seed)
    return [None if x is None else (x.astype(np.float64) * (1.0 + eps * rng.standard_normal(x.shape))).astype(np.float32)
            for x in kv_list]


def noise_floor(run, arrays, eps: float = 1e-5, seeds=(1, 2, 3)) -> float:
    """How far the oracle's own logits move when its fp32 inputs (entry rows, cached K/V) carry a
    relative perturbation of eps: every bf16 rounding point in the stack can then flip by one step,
    as it can between any two fp32 implementations that sum in different orders.
    run(arrays) -> logits. Returns the largest rel-L1 over the seeds."""
    base = run(arrays)
    return max(rel_l1(run(perturbed(arrays, eps, s)), base) for s in seeds)

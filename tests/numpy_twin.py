"""A second, independent CPU reference of the verify forward, in numpy float64 (test infrastructure).

It shares nothing with the C oracle except the precision contract both follow: every operation in
double precision, rounded to the storage precision where a value is stored (residual stream, GEMM
outputs, K/V planes and logits fp32; GEMM inputs bf16, round to nearest even). It is written from
the same definitions:
  - Q4_1 weights, w = scale * code + min per 32-weight block ("FastFlowLM build:
    Nemotron-3.5-Bolt-E4B-DFlash-NPU2", table row "Weights"), decoded with numpy's own fp16 cast;
  - a Qwen3-style decoder layer (the card's "Draft" row): RMSNorm with a multiplicative gain,
    q|k|v projections, per-head RMSNorm on q and k, rotate-half RoPE, GQA attention over the own
    plane (or the owner's plane on a KV-shared layer, engine PR #2303 "What changes"), the o
    projection and a SwiGLU MLP, each added to the residual;
  - the head tied to the embedding table (the card's "Draft" row).
The verify runs its k rows layer by layer with a causal mask inside the block (engine PR #2303,
"Proof": batched rows equal sequential steps). Matrix products use numpy's float64 matmul, so the
summation order differs from the C oracle's; the two agree to about 1e-15 relative.
"""
from __future__ import annotations

import numpy as np

from block_verify_forward_amd import synth


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    return synth.bf16_to_f32(synth.bf16_bits(np.asarray(x, dtype=np.float64))).astype(np.float64)


def bf16_values(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def q4_1_weights(img: np.ndarray) -> np.ndarray:
    """[n_out][n_in] float64 weights of a canonical Q4_1 image [n_out][n_in/32][20]."""
    n_out, nb, _ = img.shape
    scale = img[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    mins = img[:, :, 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    code_bytes = img[:, :, 4:].astype(np.int64)
    codes = np.concatenate([code_bytes & 15, code_bytes >> 4], axis=2)   # element j < 16 low nibble
    return f32(codes * scale[..., None] + mins[..., None]).reshape(n_out, nb * 32)


def rmsnorm(x: np.ndarray, gain_bits: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g along the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * bf16_values(gain_bits)


def rope(v: np.ndarray, p: int, base: float) -> np.ndarray:
    """Rotate-half RoPE of one head vector at position p: pairs (i, i + hd/2), angle p base^(-2i/hd)."""
    hd = v.shape[-1]
    h = hd // 2
    ang = p * base ** (-2.0 * np.arange(h) / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., :h], v[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


class Twin:
    """Model state of the twin: float64 copies of the planes (holding fp32 values)."""

    def __init__(self, m: synth.Model, weights: dict):
        assert not getattr(m, "kv_bf16", 0) and m.block_causal == 1
        self.m = m
        self.w = weights
        self.W = []
        for l in range(m.n_layers):
            d = weights["layers"][l]
            self.W.append({key: q4_1_weights(d[key]) for key in ("q", "k", "v", "o", "gate", "up", "down", "ple_gate",
                                                                  "ple_proj") if key in d})
        self.E = bf16_values(weights["embed"])
        self.planes = [None] * m.n_layers
        self.held = 0

    def set_kv(self, kv_list, positions: int):
        for l in range(self.m.n_layers):
            if self.m.own(l):
                pl = np.zeros((self.m.max_ctx, 2, self.m.kv_width(l)))
                pl[:positions] = np.asarray(kv_list[l][:positions], dtype=np.float64)
                self.planes[l] = pl
        self.held = positions

    def _layer(self, l: int, x: np.ndarray, pos) -> np.ndarray:
        m, L, d, W = self.m, self.m.layers[l], self.w["layers"][l], self.W[l]
        hd, Hq, nkv = L.head_dim, m.n_q_heads, L.n_kv_heads
        group = Hq // nkv
        own = L.kv_owner < 0
        plane = self.planes[l if own else L.kv_owner]
        a = bf16(rmsnorm(x, d["attn_norm"], m.rms_eps))
        q = f32(a @ W["q"].T).reshape(len(pos), Hq, hd)
        if own:
            kx = f32(a @ W["k"].T).reshape(len(pos), nkv, hd)
            vx = f32(a @ W["v"].T).reshape(len(pos), nkv, hd)
        o = np.zeros((len(pos), Hq, hd))
        for r, p in enumerate(pos):
            qr = q[r]
            if m.qk_norm:
                qr = rmsnorm(qr, d["q_norm"], m.rms_eps)
            qr = f32(np.stack([rope(qr[h], p, m.rope_base) for h in range(Hq)]))
            if own:
                kr = kx[r]
                if m.qk_norm:
                    kr = rmsnorm(kr, d["k_norm"], m.rms_eps)
                kr = f32(np.stack([rope(kr[g], p, m.rope_base) for g in range(nkv)]))
                plane[p, 0] = kr.reshape(-1)
                plane[p, 1] = vx[r].reshape(-1)
            lo = max(0, p - L.window + 1) if (L.attn == synth.ATTN_SLIDING and L.window > 0) else 0
            K = plane[lo:p + 1, 0].reshape(-1, nkv, hd)
            V = plane[lo:p + 1, 1].reshape(-1, nkv, hd)
            for h in range(Hq):
                g = h // group
                s = K[:, g, :] @ qr[h] / np.sqrt(hd)
                e = np.exp(s - s.max())
                o[r, h] = (e / e.sum()) @ V[:, g, :]
        o = bf16(o.reshape(len(pos), Hq * hd))
        x = f32(x + f32(o @ W["o"].T))
        b = bf16(rmsnorm(x, d["mlp_norm"], m.rms_eps))
        gg = f32(b @ W["gate"].T)
        uu = f32(b @ W["up"].T)
        mm = bf16(gg / (1.0 + np.exp(-gg)) * uu)
        x = f32(x + f32(mm @ W["down"].T))
        if getattr(m, "ple_dim", 0):
            # per-layer embeddings: the gate reads bf16 of the layer's output, the row's per-layer
            # input (layer l of its token's table row) multiplies silu of it, the projection adds
            # to the residual stream, and the layer scalar scales the result
            D = m.ple_dim
            u = f32(bf16(x) @ W["ple_gate"].T)
            p = bf16_values(self.w["ple_table"][self.tokens])[:, l * D:(l + 1) * D]
            h = bf16(u / (1.0 + np.exp(-u)) * p)
            s = float(bf16_values(d["layer_scalar"])[0])
            x = f32(f32(x + f32(h @ W["ple_proj"].T)) * s)
        return x

    def verify_batch(self, tokens):
        """Logits [k][V] (fp32 values as float64) of a verify of the tokens at the held positions;
        the k rows stay appended."""
        tokens = np.asarray(tokens)
        self.tokens = tokens
        pos = [self.held + r for r in range(len(tokens))]
        x = self.E[tokens].copy()
        for l in range(self.m.n_layers):
            x = self._layer(l, x, pos)
        a = bf16(rmsnorm(x, self.w["final_norm"], self.m.rms_eps))
        self.held += len(tokens)
        return f32(a @ self.E.T)


class DraftTwin:
    """The DFlash draft ("FastFlowLM build: Nemotron-3.5-Bolt-E4B-DFlash-NPU2", rows "Draft" and
    "Taps", "How it is used"): context rows are the fc fusion of the tapped target rows, normalised
    with the hidden norm, and enter every draft layer as keys/values at their positions; the block
    [token, mask, ...] (embedding rows times the embedding scale) runs through the layers with no
    causal mask inside the block and sees the context rows inside the window; rows 1..B-1 go
    through the draft's final norm and the target's tied head."""

    def __init__(self, m: synth.Model, weights: dict):
        assert not getattr(m, "kv_bf16", 0) and m.block_causal == 0
        self.m = m
        self.w = weights
        self.W = [{key: q4_1_weights(weights["layers"][l][key]) for key in ("q", "k", "v", "o", "gate", "up", "down")}
                  for l in range(m.n_layers)]
        self.fc = bf16_values(weights["fc"])
        self.planes = [np.zeros((m.max_ctx, 2, m.kv_width(l))) for l in range(m.n_layers)]
        self.held = 0

    def _kv(self, l: int, a: np.ndarray, pos):
        L, d, W = self.m.layers[l], self.w["layers"][l], self.W[l]
        hd, nkv = L.head_dim, L.n_kv_heads
        kx = f32(a @ W["k"].T).reshape(len(pos), nkv, hd)
        vx = f32(a @ W["v"].T).reshape(len(pos), nkv, hd)
        ks = []
        for r, p in enumerate(pos):
            kr = kx[r]
            if self.m.qk_norm:
                kr = rmsnorm(kr, d["k_norm"], self.m.rms_eps)
            ks.append(f32(np.stack([rope(kr[g], p, self.m.rope_base) for g in range(nkv)])))
        return np.stack(ks), vx

    def append(self, taps: np.ndarray):
        """taps [n][T][H] bf16 bits of the new context positions held .. held + n - 1."""
        n = taps.shape[0]
        f = f32(bf16_values(taps).reshape(n, -1) @ self.fc.T)
        c = bf16(rmsnorm(f, self.w["hidden_norm"], self.m.rms_eps))
        pos = [self.held + r for r in range(n)]
        for l in range(self.m.n_layers):
            k, v = self._kv(l, c, pos)
            self.planes[l][self.held:self.held + n, 0] = k.reshape(n, -1)
            self.planes[l][self.held:self.held + n, 1] = v.reshape(n, -1)
        self.held += n

    def block(self, E_bits: np.ndarray, B: int, last_token: int, scale: float, mask_token: int):
        """Logits [B-1][V] of the block at positions held .. held + B - 1 (the block is not kept)."""
        m = self.m
        E = bf16_values(E_bits)
        s = self.held
        lo = max(0, s - m.draft_window) if m.draft_window > 0 else 0
        x = f32(E[[last_token] + [mask_token] * (B - 1)] * scale)
        pos = [s + r for r in range(B)]
        for l in range(m.n_layers):
            L, d, W = m.layers[l], self.w["layers"][l], self.W[l]
            hd, Hq, nkv = L.head_dim, m.n_q_heads, L.n_kv_heads
            group = Hq // nkv
            a = bf16(rmsnorm(x, d["attn_norm"], m.rms_eps))
            q = f32(a @ W["q"].T).reshape(B, Hq, hd)
            kb, vb = self._kv(l, a, pos)
            K = np.concatenate([self.planes[l][lo:s, 0].reshape(-1, nkv, hd), kb])
            V = np.concatenate([self.planes[l][lo:s, 1].reshape(-1, nkv, hd), vb])
            o = np.zeros((B, Hq, hd))
            for r, p in enumerate(pos):
                qr = q[r]
                if m.qk_norm:
                    qr = rmsnorm(qr, d["q_norm"], m.rms_eps)
                qr = f32(np.stack([rope(qr[h], p, m.rope_base) for h in range(Hq)]))
                for h in range(Hq):
                    g = h // group
                    sc = K[:, g, :] @ qr[h] / np.sqrt(hd)
                    e = np.exp(sc - sc.max())
                    o[r, h] = (e / e.sum()) @ V[:, g, :]
            o = bf16(o.reshape(B, Hq * hd))
            x = f32(x + f32(o @ W["o"].T))
            b = bf16(rmsnorm(x, d["mlp_norm"], m.rms_eps))
            gg = f32(b @ W["gate"].T)
            uu = f32(b @ W["up"].T)
            x = f32(x + f32(bf16(gg / (1.0 + np.exp(-gg)) * uu) @ W["down"].T))
        a = bf16(rmsnorm(x[1:], self.w["final_norm"], m.rms_eps))
        return f32(a @ E.T)

"""Seeded synthetic inputs: model geometries, Q4_1 weight images, bf16 tensors, cached KV planes, tokens.

This module only *draws* inputs. It holds none of the method's arithmetic, imports nothing from the
HIP binding or from the oracle, and is the one piece both sides share: the tests and the benchmark
draw a workload here and hand the same arrays to the CPU oracle and to the GPU library.

Conventions
-----------
* Every tensor has its own named sub-stream: ``numpy.random.SeedSequence(seed, spawn_key=(crc32(name),))``
  feeding PCG64, so adding or reordering tensors never changes another tensor's values.
* Every fp16 / bf16 value is the round-to-nearest-even of a float64 draw (bf16 rounded directly from
  float64, no intermediate float32 rounding).
* A Q4_1 weight image is the canonical host format the library loads: for each output row, n_in/32
  blocks of 20 bytes = {fp16 scale (little-endian), fp16 min, 16 code bytes}; code j < 16 sits in the
  low nibble of byte j and code j + 16 in the high nibble. Weight = scale * code + min. The model
  card ("Weights" row of the Nemotron-3.5-Bolt-E4B-DFlash-NPU2 page) gives Q4_1 as 32-weight blocks
  with a scale and a minimum, 5 bits per weight; the byte order inside a block is not given there and
  is this module's choice (the common Q4_1 convention).
* Distributions: codes uniform 0..15 (each code byte is a uniform byte = two uniform nibbles), scale
  U(0.002, 0.02), min U(-0.15, 0), activations/embeddings/taps bf16 N(0,1), norm gains bf16
  U(0.5, 1.5), fc weights bf16 N(0,1)/sqrt(fan_in), cached K/V fp32 N(0,1).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, List, Optional, Sequence

import numpy as np

Q4_1_BLOCK = 32          # weights per block
Q4_1_BLOCK_BYTES = 20    # 2 (fp16 scale) + 2 (fp16 min) + 16 (32 four-bit codes)

ATTN_SLIDING = 0
ATTN_FULL = 1


# --------------------------------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Layer:
    attn: int            # ATTN_SLIDING or ATTN_FULL
    n_kv_heads: int
    head_dim: int
    window: int          # visible keys on a sliding layer (0 = unlimited)
    ffn: int
    kv_owner: int        # -1 = the layer holds its own KV plane; else the layer whose plane it reads


@dataclasses.dataclass(frozen=True)
class Model:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    vocab: int
    max_ctx: int
    layers: tuple
    tap_layers: tuple = ()
    qk_norm: int = 1
    rope_base: float = 1.0e6
    rms_eps: float = 1.0e-6
    block_causal: int = 1     # 1: verify block (causal); 0: draft block (all block rows see each other)
    draft_window: int = 0     # draft only: context rows visible to the block (0 = all)
    kv_bf16: int = 0          # 1: K/V planes stored in bf16 (a memory variant; the default planes are fp32)
    ple_dim: int = 0          # per-layer embedding width (Gemma4-style PLE); 0 = none
    kv_ring: int = 0          # 1: sliding planes of a verify model are rings of window + 16 position slots

    def kv_width(self, l: int) -> int:
        L = self.layers[l]
        return L.n_kv_heads * L.head_dim

    def own(self, l: int) -> bool:
        return self.layers[l].kv_owner < 0


def tiny_model(max_ctx: int = 128, n_layers: int = 1, vocab: int = 1024) -> Model:
    """Tiny Qwen3-style decoder: hidden 256, FFN 512 (SwiGLU), 4 query / 1 KV heads of 64, vocab 1024."""
    layers = tuple(Layer(ATTN_FULL, 1, 64, 0, 512, -1) for _ in range(n_layers))
    return Model("tiny", n_layers, 256, 4, vocab, max_ctx, layers)


def tiny_two_width_model(max_ctx: int = 128, vocab: int = 1024) -> Model:
    """A 6-layer miniature of the target's layout: sliding layers (KV width 64, window 16) and a full
    layer at l % 3 == 2 (two KV heads, width 128); layers 4..5 share the last own layer of their type.
    Small enough for brute-force oracle checks of the per-layer widths and shared planes."""
    ls = []
    n = 6
    n_own = 4
    for l in range(n):
        full = (l % 3 == 2)
        owner = -1
        if l >= n_own:
            # last own layer of the same attention type
            owner = max(j for j in range(n_own) if (j % 3 == 2) == full)
        ls.append(Layer(ATTN_FULL if full else ATTN_SLIDING, 2 if full else 1, 64,
                        0 if full else 16, 512 if l >= n_own else 256, owner))
    return Model("tiny2w", n, 256, 4, vocab, max_ctx, tuple(ls), tap_layers=(1, 2, 4))


def target_model(max_ctx: int = 1024 + 64, n_layers: int = 42, vocab: int = 262144) -> Model:
    """Target-shaped stack: 42 layers, hidden 2560, 8 query heads of 256; sliding layers 1 KV head
    (KV row 2 x 256 floats/position), window 512; every 6th layer (l % 6 == 5) full with 2 KV heads
    (2 x 512); layers 24..41 KV-shared with the last own layer of their type; FFN 10240 on own layers,
    20480 on shared ones; taps after layers 5, 11, 17, 23, 35."""
    n_own = min(24, n_layers)
    ls = []
    for l in range(n_layers):
        full = (l % 6 == 5)
        owner = -1
        if l >= n_own:
            owner = max(j for j in range(n_own) if (j % 6 == 5) == full)
        ls.append(Layer(ATTN_FULL if full else ATTN_SLIDING, 2 if full else 1, 256,
                        0 if full else 512, 20480 if l >= n_own else 10240, owner))
    taps = tuple(t for t in (5, 11, 17, 23, 35) if t < n_layers)
    return Model("target", n_layers, 2560, 8, vocab, max_ctx, tuple(ls), tap_layers=taps)


def draft_model(max_ctx: int = 1024 + 64, n_layers: int = 5, n_taps: int = 5, window: int = 1024) -> Model:
    """DFlash draft: 5 Qwen3-style layers, hidden 2560, FFN 5120, 32 query / 8 KV heads of 128,
    attention window 1024, block of 8; its fc fuses n_taps tapped target rows."""
    layers = tuple(Layer(ATTN_SLIDING, 8, 128, window, 5120, -1) for _ in range(n_layers))
    return Model("draft", n_layers, 2560, 32, 0, max_ctx, layers, tap_layers=tuple(range(n_taps)),
                 block_causal=0, draft_window=window)


def tiny_draft_model(max_ctx: int = 128, n_layers: int = 2, n_taps: int = 3, window: int = 0) -> Model:
    layers = tuple(Layer(ATTN_SLIDING, 1, 64, window, 384, -1) for _ in range(n_layers))
    return Model("tinydraft", n_layers, 256, 4, 0, max_ctx, layers, tap_layers=tuple(range(n_taps)),
                 block_causal=0, draft_window=window)


# --------------------------------------------------------------------------------------------------
# rounding of draws
# --------------------------------------------------------------------------------------------------
def f16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 -> IEEE half bits, round to nearest even (numpy's cast rounds that way)."""
    return np.asarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits, round to nearest even directly from float64 (normal range):
    round the float64 significand to 8 bits (ties to even) on its bit pattern, then the value is
    exact in float32 and its top 16 bits are the bfloat16."""
    x0 = np.asarray(x64, dtype=np.float64)
    x = np.ascontiguousarray(x0.reshape(-1))
    u = x.view(np.uint64)
    r = (u + (np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1)))) & ~np.uint64((1 << 45) - 1)
    f = r.view(np.float64)
    f = np.where(np.abs(x) < 2.0 ** -126, 0.0, f)   # draws never land there; flush for safety
    return (f.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16).reshape(x0.shape)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------------------------------
def stream(seed: int, name: str) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(zlib.crc32(name.encode()),))
    return np.random.Generator(np.random.PCG64(ss))


def q4_1_image(seed: int, name: str, n_out: int, n_in: int,
               scale_lo: float = 0.002, scale_hi: float = 0.02,
               min_lo: float = -0.15, min_hi: float = 0.0) -> np.ndarray:
    """Canonical Q4_1 image, uint8 [n_out, n_in/32, 20]."""
    assert n_in % Q4_1_BLOCK == 0
    g = stream(seed, name)
    nb = n_out * (n_in // Q4_1_BLOCK)
    img = np.empty((nb, Q4_1_BLOCK_BYTES), dtype=np.uint8)
    img[:, 4:] = g.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    img[:, 0:2] = f16_bits(g.uniform(scale_lo, scale_hi, size=nb)).view(np.uint8).reshape(nb, 2)
    img[:, 2:4] = f16_bits(g.uniform(min_lo, min_hi, size=nb)).view(np.uint8).reshape(nb, 2)
    return img.reshape(n_out, n_in // Q4_1_BLOCK, Q4_1_BLOCK_BYTES)


def q4_1_from_parts(codes: np.ndarray, scale: np.ndarray, mins: np.ndarray) -> np.ndarray:
    """Pack explicit codes [n_out, n_in] (0..15) with fp16 scale/min [n_out, n_in/32] (given as float64
    values, rounded to fp16 here) into the canonical image. Used to build hand cases."""
    codes = np.asarray(codes, dtype=np.uint8)
    n_out, n_in = codes.shape
    nbk = n_in // Q4_1_BLOCK
    c = codes.reshape(n_out, nbk, 32)
    img = np.empty((n_out, nbk, Q4_1_BLOCK_BYTES), dtype=np.uint8)
    img[:, :, 4:] = (c[:, :, :16] & 15) | ((c[:, :, 16:] & 15) << 4)
    img[:, :, 0:2] = f16_bits(np.asarray(scale, dtype=np.float64)).view(np.uint8).reshape(n_out, nbk, 2)
    img[:, :, 2:4] = f16_bits(np.asarray(mins, dtype=np.float64)).view(np.uint8).reshape(n_out, nbk, 2)
    return img


_CHUNK = 1 << 24


def _chunked_bf16(draw, shape) -> np.ndarray:
    """bf16 bits of a long float64 draw, drawn and rounded in chunks (the generator's sequence does
    not depend on the chunking); keeps the float64 temporaries small."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, _CHUNK):
        out[i:i + _CHUNK] = bf16_bits(draw(min(_CHUNK, n - i)))
    return out.reshape(shape)


def bf16_normal(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    g = stream(seed, name)
    return _chunked_bf16(lambda n: g.standard_normal(size=n) * std, shape)


def bf16_uniform(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    g = stream(seed, name)
    return _chunked_bf16(lambda n: g.uniform(lo, hi, size=n), shape)


def f32_normal(seed: int, name: str, shape) -> np.ndarray:
    return stream(seed, name).standard_normal(size=shape).astype(np.float32)


def tokens(seed: int, name: str, k: int, vocab: int) -> np.ndarray:
    return stream(seed, name).integers(0, vocab, size=k, dtype=np.int64).astype(np.int32)


# --------------------------------------------------------------------------------------------------
# whole weight sets
# --------------------------------------------------------------------------------------------------
def layer_matrix_shapes(m: Model, l: int) -> Dict[str, tuple]:
    """(n_out, n_in) of each Q4_1 matrix of layer l. A KV-shared layer has no K/V projection."""
    L = m.layers[l]
    H, qd = m.hidden, m.n_q_heads * L.head_dim
    kvd = L.n_kv_heads * L.head_dim
    s = {"q": (qd, H)}
    if L.kv_owner < 0:
        s["k"] = (kvd, H)
        s["v"] = (kvd, H)
    s.update({"o": (H, qd), "gate": (L.ffn, H), "up": (L.ffn, H), "down": (H, L.ffn)})
    if getattr(m, "ple_dim", 0):
        s["ple_gate"] = (m.ple_dim, H)
        s["ple_proj"] = (H, m.ple_dim)
    return s


def make_weights(m: Model, seed: int = 0, with_head: bool = True, threads: int = 1) -> dict:
    """All weights of a target-style model (or the layer part of a draft). Keys:
    'layers': list of dicts {q,k,v,o,gate,up,down: Q4_1 images; attn_norm, mlp_norm, q_norm, k_norm:
    bf16}; 'embed': bf16 [V, H] (tied embedding table and output head); 'final_norm': bf16 [H].
    Every tensor has its own named stream, so drawing layers on several threads gives the same arrays."""
    def layer(l):
        d = {}
        for key, (n_out, n_in) in layer_matrix_shapes(m, l).items():
            if key.startswith("ple_"):
                # per-layer embedding gate and projection: a tenth of the layer matrices' scale and
                # minimum, so the tail's contribution stays a few percent of the residual stream
                # (with the layer matrices' ranges the unnormalised gate input grows x about 3x per
                # layer and the stream overflows fp32 within 42 layers)
                d[key] = q4_1_image(seed, f"{m.name}.L{l}.{key}", n_out, n_in, 0.0002, 0.002, -0.015, 0.0)
            else:
                d[key] = q4_1_image(seed, f"{m.name}.L{l}.{key}", n_out, n_in)
        hd = m.layers[l].head_dim
        d["attn_norm"] = bf16_uniform(seed, f"{m.name}.L{l}.attn_norm", (m.hidden,), 0.5, 1.5)
        d["mlp_norm"] = bf16_uniform(seed, f"{m.name}.L{l}.mlp_norm", (m.hidden,), 0.5, 1.5)
        d["q_norm"] = bf16_uniform(seed, f"{m.name}.L{l}.q_norm", (hd,), 0.5, 1.5)
        d["k_norm"] = bf16_uniform(seed, f"{m.name}.L{l}.k_norm", (hd,), 0.5, 1.5)
        if getattr(m, "ple_dim", 0):
            d["layer_scalar"] = bf16_uniform(seed, f"{m.name}.L{l}.layer_scalar", (1,), 0.5, 1.5)
        return d

    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            out = {"layers": list(ex.map(layer, range(m.n_layers)))}
    else:
        out = {"layers": [layer(l) for l in range(m.n_layers)]}
    if with_head and m.vocab > 0 and m.block_causal == 1:
        out["embed"] = embedding_table(seed, m, max(threads, 8))
    if getattr(m, "ple_dim", 0):
        out["ple_table"] = ple_table(seed, m, max(threads, 8))
    out["final_norm"] = bf16_uniform(seed, f"{m.name}.final_norm", (m.hidden,), 0.5, 1.5)
    if m.block_causal == 0:
        T = len(m.tap_layers)
        out["fc"] = bf16_normal(seed, f"{m.name}.fc", (m.hidden, T * m.hidden), std=1.0 / np.sqrt(T * m.hidden))
        out["hidden_norm"] = bf16_uniform(seed, f"{m.name}.hidden_norm", (m.hidden,), 0.5, 1.5)
    return out


EMBED_ROWS_PER_STREAM = 16384


def embedding_table(seed: int, m: Model, threads: int = 8) -> np.ndarray:
    """The tied bf16 embedding/head table [V, H], N(0,1): row block b (16384 rows) is drawn from the
    sub-stream '<model>.embed.<b>' so blocks can be drawn in parallel."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty((m.vocab, m.hidden), dtype=np.uint16)
    blocks = range(0, m.vocab, EMBED_ROWS_PER_STREAM)

    def one(r0):
        r1 = min(m.vocab, r0 + EMBED_ROWS_PER_STREAM)
        out[r0:r1] = bf16_normal(seed, f"{m.name}.embed.{r0 // EMBED_ROWS_PER_STREAM}", (r1 - r0, m.hidden))

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, blocks))
    return out


def ple_table(seed: int, m: Model, threads: int = 8) -> np.ndarray:
    """The per-layer input table [V, n_layers * ple_dim] bf16, N(0,1): row block b (16384 rows) is
    drawn from the sub-stream '<model>.ple.<b>'."""
    from concurrent.futures import ThreadPoolExecutor
    w = m.n_layers * m.ple_dim
    out = np.empty((m.vocab, w), dtype=np.uint16)

    def one(r0):
        r1 = min(m.vocab, r0 + EMBED_ROWS_PER_STREAM)
        out[r0:r1] = bf16_normal(seed, f"{m.name}.ple.{r0 // EMBED_ROWS_PER_STREAM}", (r1 - r0, w))

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(0, m.vocab, EMBED_ROWS_PER_STREAM)))
    return out


def make_kv(m: Model, positions: int, seed: int = 0, threads: int = 1) -> List[Optional[np.ndarray]]:
    """Cached K/V for every own plane: fp32 [positions, 2, w_l] N(0,1) (K read as already roped)."""
    def plane(l):
        if m.layers[l].kv_owner < 0:
            return f32_normal(seed, f"{m.name}.kv{l}", (positions, 2, m.kv_width(l)))
        return None

    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            return list(ex.map(plane, range(m.n_layers)))
    return [plane(l) for l in range(m.n_layers)]


def q4_1_bytes(m: Model) -> int:
    n = 0
    for l in range(m.n_layers):
        for (n_out, n_in) in layer_matrix_shapes(m, l).values():
            n += n_out * n_in // Q4_1_BLOCK * Q4_1_BLOCK_BYTES
    return n


def accept_lengths(seed: int, rounds: int, p: float = 0.8467, max_a: int = 7) -> np.ndarray:
    """Steering draws for the full-loop workload: a ~ truncated geometric over 0..max_a,
    P(a=j) = p^j (1-p) for j < max_a and P(max_a) = p^max_a (mean about 3.8 at p = 0.8467)."""
    g = stream(seed, "accept")
    u = g.uniform(size=rounds)
    probs = np.array([p ** j * (1 - p) for j in range(max_a)] + [p ** max_a])
    cdf = np.cumsum(probs)
    return np.minimum(np.searchsorted(cdf, u, side="right"), max_a).astype(np.int32)

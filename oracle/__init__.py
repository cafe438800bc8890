"""CPU oracle for the DFlash batched verify forward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this
package. The GPU library neither links nor calls it. ``oracle.c`` holds the arithmetic (plain C,
double precision, rounded to the storage precisions); this file is a ctypes wrapper around it plus
the build step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build() -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P, I, L64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_double
        sig = {
            "orc_q4_1_dequant": (None, [P, I, I, P]),
            "orc_q4_1_matmul": (None, [P, I, I, P, I, P]),
            "orc_bf16_matmul": (None, [P, I, I, P, I, P]),
            "orc_rmsnorm_bf16": (None, [P, P, I, D, P]),
            "orc_rope": (None, [P, I, L64, D, P]),
            "orc_model_new": (P, [I, I, I, I, L64, I, D, D, I, I, P, P, I]),
            "orc_model_free": (None, [P]),
            "orc_set_layer": (None, [P, I] + [P] * 11),
            "orc_set_ple": (None, [P, I, P]),
            "orc_set_layer_ple": (None, [P, I, P, P, P]),
            "orc_set_globals": (None, [P, P, P, P, P]),
            "orc_set_kv": (I, [P, I, P, L64]),
            "orc_set_kv_bf16": (None, [P, I]),
            "orc_set_kv_ring": (None, [P, I]),
            "orc_plane_capacity": (L64, [P, I]),
            "orc_set_held": (None, [P, L64]),
            "orc_positions_held": (L64, [P]),
            "orc_plane": (ctypes.POINTER(ctypes.c_float), [P, I]),
            "orc_kv_widths": (None, [P, P]),
            "orc_plane_floats": (None, [P, P]),
            "orc_cut_floats": (L64, [P, I, I, L64]),
            "orc_step": (I, [P, I, P, P]),
            "orc_verify_batch": (I, [P, P, I, P, P]),
            "orc_commit_verify_rows": (I, [P, I]),
            "orc_extend_context": (I, [P, P, L64]),
            "orc_argmax": (I, [P, I]),
            "orc_accept_greedy": (I, [P, I, I, P, P, P]),
            "orc_philox4x32_10": (None, [P, P, P]),
            "orc_gumbel_of_word": (ctypes.c_float, [ctypes.c_uint32]),
            "orc_sample_scores": (None, [P, I, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, I, P]),
            "orc_sample_rows": (None, [P, I, I, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, P]),
            "orc_accept_sampled": (I, [P, I, I, P, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, P, P, P]),
            "orc_snapshot_take": (P, [P]),
            "orc_snapshot_floats": (L64, [P, I]),
            "orc_snapshot_restore": (I, [P, P]),
            "orc_snapshot_free": (None, [P]),
            "orc_draft_append": (I, [P, P, I]),
            "orc_draft_block": (I, [P, P, I, I, D, I, P, P]),
            "orc_threads": (I, []),
            "orc_set_threads": (None, [I]),
            "orc_attend": (None, [P, I, P, L64, P]),
            "orc_layer_forward": (I, [P, I, I, P, P, P]),
            "orc_verify_embedded": (I, [P, P, I, P, P]),
            "orc_draft_block_embedded": (I, [P, P, I, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def threads() -> int:
    return int(lib().orc_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (results do not depend on it)."""
    lib().orc_set_threads(int(n))


# ---- kernels as functions -------------------------------------------------------------------
def q4_1_dequant(img: np.ndarray, n_out: int, n_in: int) -> np.ndarray:
    out = np.empty((n_out, n_in), dtype=np.float32)
    lib().orc_q4_1_dequant(_p(np.ascontiguousarray(img)), n_out, n_in, _p(out))
    return out


def q4_1_matmul(img: np.ndarray, n_out: int, n_in: int, x_bf16: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1, n_in)
    y = np.empty((x.shape[0], n_out), dtype=np.float32)
    lib().orc_q4_1_matmul(_p(np.ascontiguousarray(img)), n_out, n_in, _p(x), x.shape[0], _p(y))
    return y


def bf16_matmul(w_bf16: np.ndarray, x_bf16: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    n_out, n_in = w.shape
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1, n_in)
    y = np.empty((x.shape[0], n_out), dtype=np.float32)
    lib().orc_bf16_matmul(_p(w), n_out, n_in, _p(x), x.shape[0], _p(y))
    return y


def rmsnorm_bf16(x: np.ndarray, g_bf16: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape[0], dtype=np.uint16)
    lib().orc_rmsnorm_bf16(_p(x), _p(np.ascontiguousarray(g_bf16, dtype=np.uint16)), x.shape[0], eps, _p(out))
    return out


def rope(v: np.ndarray, p: int, base: float = 1e6) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty_like(v)
    lib().orc_rope(_p(v), v.shape[0], p, base, _p(out))
    return out


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return int(lib().orc_argmax(_p(v), v.shape[0]))


def accept_greedy(logits_all: np.ndarray, tokens: np.ndarray):
    """Returns (a, emitted tokens [a+1])."""
    lg = np.ascontiguousarray(logits_all, dtype=np.float32)
    k, V = lg.shape
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.zeros(k, dtype=np.int32)
    a = ctypes.c_int(0)
    lib().orc_accept_greedy(_p(lg), k, V, _p(t), _p(out), ctypes.byref(a))
    return a.value, out[: a.value + 1].copy()


def philox4x32_10(counter, key) -> np.ndarray:
    """One Philox4x32-10 block: 4 counter words, 2 key words -> 4 output words (uint32)."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def gumbel_of_word(x: int) -> float:
    """The Gumbel noise -log(-log u) of one 32-bit generator word (fp32)."""
    return float(lib().orc_gumbel_of_word(int(x) & 0xFFFFFFFF))


def sample_scores(z_row: np.ndarray, temperature: float, seed: int, offset: int, row: int) -> np.ndarray:
    """fp32 Gumbel-perturbed scores z / T + g of one row (the sampled verify's draw is their argmax)."""
    z = np.ascontiguousarray(z_row, dtype=np.float32)
    out = np.empty(z.size, dtype=np.float32)
    lib().orc_sample_scores(_p(z), z.size, float(temperature), int(seed), int(offset), int(row), _p(out))
    return out


def sample_rows(logits: np.ndarray, temperature: float, seed: int, offset: int) -> np.ndarray:
    """The draws y_i of every row of logits [k][V] (row i uses counter row i)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    k, V = lg.shape
    y = np.zeros(k, dtype=np.int32)
    lib().orc_sample_rows(_p(lg), k, V, float(temperature), int(seed), int(offset), _p(y))
    return y


def accept_sampled(logits_all: np.ndarray, tokens: np.ndarray, temperature: float, seed: int, offset: int):
    """Sampled longest-prefix accept: returns (a, emitted tokens [a+1], draws [k])."""
    lg = np.ascontiguousarray(logits_all, dtype=np.float32)
    k, V = lg.shape
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.zeros(k, dtype=np.int32)
    draws = np.zeros(k, dtype=np.int32)
    a = ctypes.c_int(0)
    lib().orc_accept_sampled(_p(lg), k, V, _p(t), float(temperature), int(seed), int(offset), _p(out),
                             ctypes.byref(a), _p(draws))
    return a.value, out[: a.value + 1].copy(), draws


def cut_floats(per, plane: int, positions: int) -> int:
    per = np.ascontiguousarray(per, dtype=np.int64)
    return int(lib().orc_cut_floats(_p(per), len(per), plane, positions))


# ---- model ----------------------------------------------------------------------------------
class Model:
    """Oracle model over caller-owned host arrays (kept alive here)."""

    def __init__(self, m, weights: dict):
        self.m = m
        fields = np.array([[L.attn, L.n_kv_heads, L.head_dim, L.window, L.ffn, L.kv_owner] for L in m.layers],
                          dtype=np.int32)
        taps = np.array(list(m.tap_layers) or [0], dtype=np.int32)
        self._keep = [fields, taps, weights]
        self.h = lib().orc_model_new(m.n_layers, m.hidden, m.n_q_heads, m.vocab, m.max_ctx, m.qk_norm,
                                     m.rope_base, m.rms_eps, m.block_causal, m.draft_window,
                                     _p(fields), _p(taps), len(m.tap_layers))
        if getattr(m, "kv_bf16", 0):
            lib().orc_set_kv_bf16(self.h, 1)
        if getattr(m, "kv_ring", 0):
            lib().orc_set_kv_ring(self.h, 1)
        for l, d in enumerate(weights["layers"]):
            g = lambda k: _p(d[k]) if k in d else None
            lib().orc_set_layer(self.h, l, g("q"), g("k"), g("v"), g("o"), g("gate"), g("up"), g("down"),
                                g("attn_norm"), g("mlp_norm"), g("q_norm"), g("k_norm"))
        lib().orc_set_globals(self.h, _p(weights.get("embed")), _p(weights.get("final_norm")),
                              _p(weights.get("fc")), _p(weights.get("hidden_norm")))
        if getattr(m, "ple_dim", 0):
            lib().orc_set_ple(self.h, m.ple_dim, _p(weights["ple_table"]))
            for l, d in enumerate(weights["layers"]):
                lib().orc_set_layer_ple(self.h, l, _p(d["ple_gate"]), _p(d["ple_proj"]), _p(d["layer_scalar"]))

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().orc_model_free(self.h)
                self.h = None
        except Exception:
            pass

    # state
    def set_kv(self, kv_list, positions: int):
        for l, kv in enumerate(kv_list):
            if kv is None:
                continue
            kv = np.ascontiguousarray(kv[:positions], dtype=np.float32)
            assert lib().orc_set_kv(self.h, l, _p(kv), positions) == 0
        lib().orc_set_held(self.h, positions)

    def extend_context(self, kv_new, n: int) -> int:
        """Append n positions of K/V rows to every own plane (kv_new[l]: [n][2][w_l] fp32 for an own
        layer, ignored for a shared one). Returns 0, or 2 (verify pending) / 3 (past max_ctx) with no
        state change."""
        parts = [np.ascontiguousarray(kv_new[l][:n], dtype=np.float32).ravel()
                 for l in range(self.m.n_layers) if self.m.layers[l].kv_owner < 0]
        flat = np.concatenate(parts) if parts else np.zeros(1, dtype=np.float32)
        return int(lib().orc_extend_context(self.h, _p(flat), n))

    def held(self) -> int:
        return int(lib().orc_positions_held(self.h))

    def kv_widths(self) -> np.ndarray:
        out = np.zeros(self.m.n_layers, dtype=np.int64)
        lib().orc_kv_widths(self.h, _p(out))
        return out

    def plane_floats(self) -> np.ndarray:
        out = np.zeros(self.m.n_layers, dtype=np.int64)
        lib().orc_plane_floats(self.h, _p(out))
        return out

    def capacity(self, l: int) -> int:
        """Positions the plane of layer l holds at most (ring planes: window + 16)."""
        return int(lib().orc_plane_capacity(self.h, l))

    def plane(self, l: int, positions: int) -> np.ndarray:
        """Rows of positions 0 .. positions - 1 of layer l's plane [positions][2][w]; on a ring plane
        the positions older than its capacity are no longer held and read as NaN."""
        w = self.m.kv_width(l)
        cap = self.capacity(l)
        ptr = lib().orc_plane(self.h, l)
        arr = np.ctypeslib.as_array(ptr, shape=(cap, 2, w))
        if cap >= self.m.max_ctx:
            return arr[:positions].copy()
        out = np.full((positions, 2, w), np.nan, dtype=np.float32)
        for p in range(max(0, positions - cap), positions):
            out[p] = arr[p % cap]
        return out

    # forward
    def step(self, token: int, with_taps: bool = False):
        lg = np.empty(self.m.vocab, dtype=np.float32)
        taps = np.empty((len(self.m.tap_layers), self.m.hidden), dtype=np.uint16) if with_taps else None
        rc = lib().orc_step(self.h, int(token), _p(lg), _p(taps))
        if rc:
            raise RuntimeError(f"oracle step: status {rc}")
        return (lg, taps) if with_taps else lg

    def verify_batch(self, tokens, with_taps: bool = False):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        k = t.shape[0]
        lg = np.empty((k, self.m.vocab), dtype=np.float32)
        taps = np.empty((k, len(self.m.tap_layers), self.m.hidden), dtype=np.uint16) if with_taps else None
        rc = lib().orc_verify_batch(self.h, _p(t), k, _p(lg), _p(taps))
        if rc:
            raise RuntimeError(f"oracle verify: status {rc}")
        return (lg, taps) if with_taps else lg

    def verify_embedded(self, x0: np.ndarray, with_taps: bool = False):
        """A verify whose rows enter as given fp32 residual rows x0 [k][H]."""
        x0 = np.ascontiguousarray(x0, dtype=np.float32).reshape(-1, self.m.hidden)
        k = x0.shape[0]
        lg = np.empty((k, self.m.vocab), dtype=np.float32)
        taps = np.empty((k, len(self.m.tap_layers), self.m.hidden), dtype=np.uint16) if with_taps else None
        rc = lib().orc_verify_embedded(self.h, _p(x0), k, _p(lg), _p(taps))
        if rc:
            raise RuntimeError(f"oracle verify: status {rc}" + (" (injected rows on a PLE model)" if rc == 4 else ""))
        return (lg, taps) if with_taps else lg

    def commit_verify_rows(self, n: int) -> int:
        return int(lib().orc_commit_verify_rows(self.h, n))

    def snapshot(self):
        """Snapshot of the committed state; refused (RuntimeError, no state change) while a verify
        is pending."""
        h = lib().orc_snapshot_take(self.h)
        if not h:
            raise RuntimeError("oracle snapshot: a verify is pending")
        return Snapshot(h, self.m.n_layers)

    def restore(self, snap) -> int:
        return int(lib().orc_snapshot_restore(self.h, snap.h))

    def attend(self, l: int, q: np.ndarray, p: int) -> np.ndarray:
        """Attention output of one row (before the bf16 rounding), q [Hq*hd] fp32."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        out = np.empty(q.shape[0], dtype=np.float64)
        lib().orc_attend(self.h, l, _p(q), p, _p(out))
        return out

    def layer_forward(self, l: int, x: np.ndarray, pos) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, self.m.hidden)
        pos = np.ascontiguousarray(pos, dtype=np.int64)
        out = np.empty_like(x)
        rc = lib().orc_layer_forward(self.h, l, x.shape[0], _p(x), _p(pos), _p(out))
        if rc:
            raise RuntimeError(f"oracle layer forward: status {rc}" + (" (injected rows on a PLE model)" if rc == 4 else ""))
        return out

    # draft
    def draft_append(self, taps: np.ndarray):
        t = np.ascontiguousarray(taps, dtype=np.uint16)
        rc = lib().orc_draft_append(self.h, _p(t), t.shape[0])
        if rc:
            raise RuntimeError(f"oracle draft append: status {rc}")

    def draft_block(self, target: "Model", block: int, last_token: int, embedding_scale: float,
                    mask_token: int, with_logits: bool = False):
        props = np.zeros(block - 1, dtype=np.int32)
        lg = np.empty((block - 1, target.m.vocab), dtype=np.float32) if with_logits else None
        rc = lib().orc_draft_block(self.h, target.h, block, int(last_token), float(embedding_scale),
                                   int(mask_token), _p(props), _p(lg))
        if rc:
            raise RuntimeError(f"oracle draft block: status {rc}")
        return (props, lg) if with_logits else props


def draft_block_embedded(draft: Model, target: Model, x0: np.ndarray):
    """The draft block from given fp32 block rows x0 [B][H]; returns (proposals, logits [B-1][V])."""
    x0 = np.ascontiguousarray(x0, dtype=np.float32).reshape(-1, draft.m.hidden)
    B = x0.shape[0]
    props = np.zeros(B - 1, dtype=np.int32)
    lg = np.empty((B - 1, target.m.vocab), dtype=np.float32)
    rc = lib().orc_draft_block_embedded(draft.h, target.h, B, _p(x0), _p(props), _p(lg))
    if rc:
        raise RuntimeError(f"oracle draft block: status {rc}")
    return props, lg


class Snapshot:
    def __init__(self, h, n_layers):
        self.h = h
        self.n_layers = n_layers

    def floats(self) -> List[int]:
        return [int(lib().orc_snapshot_floats(self.h, l)) for l in range(self.n_layers)]

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().orc_snapshot_free(self.h)
                self.h = None
        except Exception:
            pass

"""Thin Python binding of libbvf.so (include/bvf.h): argument marshalling only.

Every step of the verify path runs in the library's HIP kernels. PyTorch supplies device memory
(the model arena and the caller's input/output tensors) and the HIP stream; nothing here computes.
If the built library is missing the import fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbvf.so")

BVF_OK, BVF_E_INVALID, BVF_E_STATE, BVF_E_CAPACITY, BVF_E_DEVICE = range(5)
ATTN_SLIDING, ATTN_FULL = 0, 1
Q, K, V, O, GATE, UP, DOWN = range(7)
EMBED, FINAL_NORM, ATTN_NORM, MLP_NORM, Q_NORM, K_NORM, FC, HIDDEN_NORM = range(8)
PLE_GATE, PLE_PROJ = 7, 8
PLE_TABLE, LAYER_SCALAR = 8, 9
MATRIX_IDS = {"q": Q, "k": K, "v": V, "o": O, "gate": GATE, "up": UP, "down": DOWN, "ple_gate": PLE_GATE,
              "ple_proj": PLE_PROJ}


class BvfError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"bvf status {status}: {msg}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("attn", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("ffn", ctypes.c_int32), ("kv_owner", ctypes.c_int32)]


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
                ("block_causal", ctypes.c_int32), ("draft_window", ctypes.c_int32), ("n_taps", ctypes.c_int32),
                ("tap_layers", ctypes.POINTER(ctypes.c_int32)), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("layers", ctypes.POINTER(LayerDesc)), ("kv_bf16", ctypes.c_int32),
                ("ple_dim", ctypes.c_int32), ("kv_ring", ctypes.c_int32)]


# exported symbol -> (restype, argtypes); the list is the header's declarations
_P, _I32, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "bvf_last_error": (ctypes.c_char_p, []),
    "bvf_arena_bytes": (_SZ, [_P]),
    "bvf_create": (_I32, [_P, _P, _SZ, _P, ctypes.POINTER(_P)]),
    "bvf_destroy": (None, [_P]),
    "bvf_load_q4_1": (_I32, [_P, _I32, _I32, _P, _SZ, _I32, _I32]),
    "bvf_load_bf16": (_I32, [_P, _I32, _I32, _P, _SZ]),
    "bvf_set_kv": (_I32, [_P, _I32, _P, _I64]),
    "bvf_get_kv": (_I32, [_P, _I32, _P, _I64]),
    "bvf_set_positions": (_I32, [_P, _I64]),
    "bvf_extend_context": (_I32, [_P, _P, _I64]),
    "bvf_kv_widths": (_I32, [_P, _P, _I32]),
    "bvf_plane_floats": (_I32, [_P, _P, _I32]),
    "bvf_positions_held": (_I32, [_P, _P]),
    "bvf_verify_batch": (_I32, [_P, _P, _I32, _P, _P]),
    "bvf_set_graph_mode": (_I32, [_P, _I32]),
    "bvf_graph_captures": (_I32, [_P, _P]),
    "bvf_accept_greedy": (_I32, [_P, _P, _I32, _P, _P, _P]),
    "bvf_accept_greedy_static": (_I32, [_P, _I32, _I32, _P, _P, _P, _P]),
    "bvf_prefill": (_I32, [_P, _P, _I32, _P]),
    "bvf_accept_sampled": (_I32, [_P, _P, _I32, _P, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, _P, _P, _P]),
    "bvf_steer_logits": (_I32, [_P, _P, _I32, _P, _P]),
    "bvf_commit_verify_rows": (_I32, [_P, _I32]),
    "bvf_snapshot_take": (_I32, [_P, ctypes.POINTER(_P)]),
    "bvf_snapshot_update": (_I32, [_P, _P]),
    "bvf_restore": (_I32, [_P, _P]),
    "bvf_snapshot_floats": (_I32, [_P, _P, _I32]),
    "bvf_snapshot_free": (None, [_P]),
    "bvf_draft_block_forward": (_I32, [_P, _P, _P, _I32, _P, _I32, _F, _I32, _P, _P]),
    "bvf_q4_1_dequant": (_I32, [_P, _I32, _I32, _P]),
    "bvf_q4_1_gemm": (_I32, [_P, _I32, _I32, _P, _I32, _P]),
    "bvf_layer_forward": (_I32, [_P, _I32, _P, _I32]),
    "bvf_time_gemms": (_I32, [_P, _I32, _I32, _P, _P]),
    "bvf_pass_bytes": (_I32, [_P, _P, _P]),
    "bvf_cut_floats": (_I64, [_P, _I32, _I32, _I64]),
}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc for gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().bvf_last_error().decode()


def _check(status: int):
    if status != BVF_OK:
        raise BvfError(status, last_error())


def _ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    return t.data_ptr()


def _host(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def make_desc(m) -> tuple:
    """ctypes descriptor of a synth.Model (kept alive by the returned tuple)."""
    layers = (LayerDesc * m.n_layers)(*[LayerDesc(L.attn, L.n_kv_heads, L.head_dim, L.window, L.ffn, L.kv_owner)
                                        for L in m.layers])
    taps = (ctypes.c_int32 * max(1, len(m.tap_layers)))(*(list(m.tap_layers) or [0]))
    vocab = m.vocab
    d = ModelDesc(m.n_layers, m.hidden, m.n_q_heads, vocab, m.max_ctx, m.qk_norm, m.block_causal, m.draft_window,
                  len(m.tap_layers), ctypes.cast(taps, ctypes.POINTER(ctypes.c_int32)), m.rope_base, m.rms_eps,
                  ctypes.cast(layers, ctypes.POINTER(LayerDesc)), int(getattr(m, "kv_bf16", 0)),
                  int(getattr(m, "ple_dim", 0)), int(getattr(m, "kv_ring", 0)))
    return d, layers, taps


def arena_bytes(m) -> int:
    d, _l, _t = make_desc(m)
    n = lib().bvf_arena_bytes(ctypes.byref(d))
    if n == 0:
        raise BvfError(BVF_E_INVALID, last_error())
    return int(n)


def cut_floats(per: Sequence[int], plane: int, positions: int) -> int:
    a = np.ascontiguousarray(per, dtype=np.int64)
    return int(lib().bvf_cut_floats(_host(a), len(a), plane, positions))


def accept_greedy_static(d_logits_all, d_tokens, d_out_tokens, d_n_accepted, stream=None):
    """The greedy accept with no model and no allocation (bvf_accept_greedy_static): logits
    [k][vocab] fp32, tokens [k] int32, out tokens [k] int32, n_accepted [1] int32, all on the device;
    enqueued on stream (a torch stream; None: the current torch stream)."""
    import torch
    k, vocab = int(d_logits_all.shape[0]), int(d_logits_all.shape[1])
    st = stream if stream is not None else torch.cuda.current_stream()
    _check(lib().bvf_accept_greedy_static(_ptr(d_logits_all), k, vocab, _ptr(d_tokens), _ptr(d_out_tokens),
                                          _ptr(d_n_accepted), st.cuda_stream))


class Model:
    """A model in a device arena allocated by torch on the current CUDA (HIP) device."""

    def __init__(self, m, device="cuda", stream=None):
        import torch
        self.m = m
        self.torch = torch
        self._desc = make_desc(m)
        nbytes = lib().bvf_arena_bytes(ctypes.byref(self._desc[0]))
        if nbytes == 0:
            raise BvfError(BVF_E_INVALID, last_error())
        self.arena = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.arena.device)
        h = ctypes.c_void_p()
        _check(lib().bvf_create(ctypes.byref(self._desc[0]), self.arena.data_ptr(), int(nbytes),
                                ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h)))
        self.h = h

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().bvf_destroy(self.h)
                self.h = None
        except Exception:
            pass

    # ---- loading ----
    def load_q4_1(self, layer: int, matrix: int, img: np.ndarray):
        img = np.ascontiguousarray(img, dtype=np.uint8)
        n_out, nb = img.shape[0], img.shape[1]
        _check(lib().bvf_load_q4_1(self.h, layer, matrix, _host(img), img.nbytes, n_out, nb * 32))

    def load_bf16(self, tensor: int, layer: int, a: np.ndarray):
        a = np.ascontiguousarray(a, dtype=np.uint16)
        _check(lib().bvf_load_bf16(self.h, tensor, layer, _host(a), a.size))

    def load_weights(self, w: dict):
        for l, d in enumerate(w["layers"]):
            for key, mid in MATRIX_IDS.items():
                if key in d:
                    self.load_q4_1(l, mid, d[key])
            self.load_bf16(ATTN_NORM, l, d["attn_norm"])
            self.load_bf16(MLP_NORM, l, d["mlp_norm"])
            self.load_bf16(Q_NORM, l, d["q_norm"])
            self.load_bf16(K_NORM, l, d["k_norm"])
            if "layer_scalar" in d:
                self.load_bf16(LAYER_SCALAR, l, d["layer_scalar"])
        if "ple_table" in w:
            self.load_bf16(PLE_TABLE, 0, w["ple_table"])
        if "embed" in w:
            self.load_bf16(EMBED, 0, w["embed"])
        self.load_bf16(FINAL_NORM, 0, w["final_norm"])
        if "fc" in w:
            self.load_bf16(FC, 0, w["fc"])
            self.load_bf16(HIDDEN_NORM, 0, w["hidden_norm"])

    def set_kv(self, layer: int, kv: np.ndarray, positions: int):
        kv = np.ascontiguousarray(kv[:positions], dtype=np.float32)
        _check(lib().bvf_set_kv(self.h, layer, _host(kv), positions))

    def get_kv(self, layer: int, positions: int) -> np.ndarray:
        """The first `positions` rows of layer's own plane, [positions, 2, w] fp32."""
        out = np.empty((positions, 2, self.kv_widths()[layer]), dtype=np.float32)
        _check(lib().bvf_get_kv(self.h, layer, _host(out), positions))
        return out

    def set_positions(self, positions: int):
        _check(lib().bvf_set_positions(self.h, positions))

    def extend_context(self, kv_new, n: int):
        """Append n positions of K/V rows to every own plane (kv_new[l]: [n][2][w_l] fp32 for an own
        layer, ignored for a shared one); positions held += n."""
        parts = [np.ascontiguousarray(kv_new[l][:n], dtype=np.float32).ravel()
                 for l in range(self.m.n_layers) if self.m.layers[l].kv_owner < 0]
        flat = np.concatenate(parts) if parts else np.zeros(1, dtype=np.float32)
        _check(lib().bvf_extend_context(self.h, _host(flat), n))

    def set_context(self, kv_list, positions: int):
        """set_kv on every own plane, then set_positions."""
        for l, kv in enumerate(kv_list):
            if kv is not None:
                self.set_kv(l, kv, positions)
        self.set_positions(positions)

    # ---- bookkeeping ----
    def kv_widths(self) -> np.ndarray:
        out = np.zeros(self.m.n_layers, dtype=np.int64)
        _check(lib().bvf_kv_widths(self.h, _host(out), self.m.n_layers))
        return out

    def plane_floats(self) -> np.ndarray:
        out = np.zeros(self.m.n_layers, dtype=np.int64)
        _check(lib().bvf_plane_floats(self.h, _host(out), self.m.n_layers))
        return out

    def positions_held(self) -> int:
        out = np.zeros(1, dtype=np.int64)
        _check(lib().bvf_positions_held(self.h, _host(out)))
        return int(out[0])

    # ---- the path ----
    def verify_batch(self, d_tokens, d_logits_all, d_taps=None):
        _check(lib().bvf_verify_batch(self.h, _ptr(d_tokens), int(d_tokens.numel()), _ptr(d_logits_all), _ptr(d_taps)))

    def set_graph_mode(self, on: bool):
        _check(lib().bvf_set_graph_mode(self.h, 1 if on else 0))

    def graph_captures(self) -> int:
        out = np.zeros(1, dtype=np.int64)
        _check(lib().bvf_graph_captures(self.h, _host(out)))
        return int(out[0])

    def prefill(self, d_tokens, d_last_logits=None):
        _check(lib().bvf_prefill(self.h, _ptr(d_tokens), int(d_tokens.numel()),
                                 None if d_last_logits is None else _ptr(d_last_logits)))

    def accept_greedy(self, d_logits_all, d_tokens, d_out_tokens, d_n_accepted):
        _check(lib().bvf_accept_greedy(self.h, _ptr(d_logits_all), int(d_tokens.numel()), _ptr(d_tokens),
                                       _ptr(d_out_tokens), _ptr(d_n_accepted)))

    def accept_sampled(self, d_logits_all, d_tokens, d_out_tokens, d_n_accepted, temperature: float, seed: int,
                       offset: int, d_draws=None):
        _check(lib().bvf_accept_sampled(self.h, _ptr(d_logits_all), int(d_tokens.numel()), _ptr(d_tokens),
                                        float(temperature), int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1),
                                        _ptr(d_out_tokens), _ptr(d_n_accepted),
                                        None if d_draws is None else _ptr(d_draws)))

    def steer_logits(self, d_logits_all, d_tok, d_add):
        _check(lib().bvf_steer_logits(self.h, _ptr(d_logits_all), int(d_tok.numel()), _ptr(d_tok), _ptr(d_add)))

    def commit_verify_rows(self, n: int):
        _check(lib().bvf_commit_verify_rows(self.h, n))

    def snapshot_take(self) -> "Snapshot":
        h = ctypes.c_void_p()
        _check(lib().bvf_snapshot_take(self.h, ctypes.byref(h)))
        return Snapshot(h, self.m.n_layers)

    def snapshot_update(self, snap: "Snapshot"):
        _check(lib().bvf_snapshot_update(self.h, snap.h))

    def restore(self, snap: "Snapshot"):
        _check(lib().bvf_restore(self.h, snap.h))

    def draft_block_forward(self, target: "Model", d_new_taps, n_new: int, d_last_token, block: int,
                            embedding_scale: float, mask_token: int, d_proposals, d_logits=None):
        _check(lib().bvf_draft_block_forward(self.h, target.h, _ptr(d_new_taps), n_new, _ptr(d_last_token), block,
                                             float(embedding_scale), int(mask_token), _ptr(d_proposals),
                                             _ptr(d_logits)))

    # ---- kernel-level ----
    def q4_1_dequant(self, layer: int, matrix: int, d_w):
        _check(lib().bvf_q4_1_dequant(self.h, layer, matrix, _ptr(d_w)))

    def q4_1_gemm(self, layer: int, matrix: int, d_x, rows: int, d_y):
        _check(lib().bvf_q4_1_gemm(self.h, layer, matrix, _ptr(d_x), rows, _ptr(d_y)))

    def layer_forward(self, layer: int, d_x, rows: int):
        _check(lib().bvf_layer_forward(self.h, layer, _ptr(d_x), rows))

    def time_gemms(self, rows: int, iters: int):
        """(ms per launch [5], bytes per launch [5]) for q|k|v, o, gate|up, down, head."""
        ms = np.zeros(5, dtype=np.float32)
        by = np.zeros(5, dtype=np.int64)
        _check(lib().bvf_time_gemms(self.h, rows, iters, _host(ms), _host(by)))
        return ms, by

    def pass_bytes(self):
        q = np.zeros(1, dtype=np.int64)
        hb = np.zeros(1, dtype=np.int64)
        _check(lib().bvf_pass_bytes(self.h, _host(q), _host(hb)))
        return int(q[0]), int(hb[0])


class Snapshot:
    def __init__(self, h, n_layers: int):
        self.h = h
        self.n_layers = n_layers

    def floats(self) -> np.ndarray:
        out = np.zeros(self.n_layers, dtype=np.int64)
        _check(lib().bvf_snapshot_floats(self.h, _host(out), self.n_layers))
        return out

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().bvf_snapshot_free(self.h)
                self.h = None
        except Exception:
            pass

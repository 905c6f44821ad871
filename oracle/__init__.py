"""CPU oracle for the compressed-KV decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product library (``evicted_kv_cache_amd``)
never imports, links or calls it, and this package never imports the product.

Arithmetic lives in the plain C file ``kvq_oracle.c`` (fp32 exactly as the
specification fixes it for quantization, fp64 for attention and SnapKV
scores); ``cache.py`` holds the cache bookkeeping (slots, residual group,
eviction, SnapKV selection and gather) in numpy.  Every function is pinned by
``tests/test_oracle_pins.py``; see the module docstrings for the passages of
the source pages each one follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """Load (building if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.kvo_f32_to_f16.restype = ctypes.c_uint16
        L.kvo_f32_to_f16.argtypes = [ctypes.c_float]
        L.kvo_f16_to_f32.restype = ctypes.c_float
        L.kvo_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvo_f32_to_f16_n.argtypes = [P, i64, P]
        L.kvo_f16_to_f32_n.argtypes = [P, i64, P]
        L.kvo_quant_tok_affine.argtypes = [P, i64, i32, i32, i32, P, P]
        L.kvo_quant_channel_group.argtypes = [P, i32, i32, i32, P, P]
        L.kvo_quant_sym4.argtypes = [P, i64, i32, P, P, P]
        L.kvo_dequant.restype = f64
        L.kvo_dequant.argtypes = [P, i32, i32]
        L.kvo_decode_head.argtypes = [P, P, i32, P, f64, P]
        L.kvo_rope_rotate.argtypes = [P, i32, f64, i32]
        L.kvo_decode_head_rope.argtypes = [P, P, i32, P, f64, f64, i32, P]
        L.kvo_snapkv_scores.argtypes = [P, i32, i32, i32, P]
        L.kvo_snapkv_scores_rows.argtypes = [P, i32, P, i32, i32, P]
        L.kvo_maxpool1d.argtypes = [P, i32, i32, P]
        L.kvo_snapkv_select.restype = i32
        L.kvo_snapkv_select.argtypes = [P, i32, i32, i32, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().kvo_f32_to_f16_n(_p(x), x.size, _p(out))
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().kvo_f16_to_f32_n(_p(h), h.size, _p(out))
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def widen(x, dtype: str) -> np.ndarray:
    """Stored values (f32 / f16 / bf16 bits) to exact float32."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return f16_bits_to_f32(np.ascontiguousarray(x).view(np.uint16))
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# quantizers (fp32, bit-exact specification)
# ---------------------------------------------------------------------------

def quant_tok_affine(x: np.ndarray, G: int, bits: int):
    """Per-token groups of G channels.  x [..., D] fp32 -> (u [..., D], meta [..., D/G, 2])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    rows = x.size // D
    u = np.empty(x.shape, dtype=np.uint8)
    meta = np.empty(x.shape[:-1] + (D // G, 2), dtype=np.uint16)
    lib().kvo_quant_tok_affine(_p(x), rows, D, G, bits, _p(u), _p(meta))
    return u, meta


def quant_channel_group(x: np.ndarray, bits: int):
    """One closed group: x [Gt][D] fp32 -> (u [Gt][D], meta [D][2])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    Gt, D = x.shape
    u = np.empty((Gt, D), dtype=np.uint8)
    meta = np.empty((D, 2), dtype=np.uint16)
    lib().kvo_quant_channel_group(_p(x), Gt, D, bits, _p(u), _p(meta))
    return u, meta


def quant_sym4(x: np.ndarray, bias: np.ndarray | None):
    """x [..., D] fp32, bias [D] fp32 or None -> (u [..., D], scale [..., D/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    rows = x.size // D
    u = np.empty(x.shape, dtype=np.uint8)
    sc = np.empty(x.shape[:-1] + (D // 32,), dtype=np.uint16)
    bp = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        bp = _p(bias)
    lib().kvo_quant_sym4(_p(x), rows, D, bp, _p(u), _p(sc))
    return u, sc


# ---------------------------------------------------------------------------
# attention (fp64)
# ---------------------------------------------------------------------------

PLAIN, CHANNEL, TOK_AFFINE, SYM4 = 0, 1, 2, 3


class View(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("D", ctypes.c_int), ("G", ctypes.c_int),
                ("u", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("row", ctypes.c_void_p), ("plain", ctypes.c_void_p),
                ("n_coded", ctypes.c_int)]


def make_view(kind, D, G=0, u=None, meta=None, row=None, plain=None, n_coded=0):
    """Build a dequantization view; the returned tuple keeps the arrays alive."""
    keep = []

    def ptr(a, dt):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dt)
        keep.append(a)
        return _p(a).value

    v = View(kind, D, G, ptr(u, np.uint8), ptr(meta, np.uint16),
             ptr(row, np.int32), ptr(plain, np.float32), n_coded)
    return v, keep


def dequant(view, T: int, D: int) -> np.ndarray:
    """Dequantized [T][D] fp64 values of a view (for tests)."""
    v, _keep = view
    out = np.empty((T, D), dtype=np.float64)
    L = lib()
    for t in range(T):
        for d in range(D):
            out[t, d] = L.kvo_dequant(ctypes.byref(v), t, d)
    return out


def rope_rotate(x: np.ndarray, base: float, pos: int) -> np.ndarray:
    """x [D] rotated at position pos (half-split pairs), fp64."""
    x = np.array(x, dtype=np.float64)
    lib().kvo_rope_rotate(_p(x), x.shape[0], float(base), int(pos))
    return x


def decode_head_rope(kview, vview, T: int, q: np.ndarray, scale: float, base: float,
                     q_pos: int) -> np.ndarray:
    """fp64 attention output [D] with keys rotated at their slot index and the
    query at q_pos (q fp32 [D], stored before the rotation)."""
    kv, _k = kview
    vv, _v = vview
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.shape[-1], dtype=np.float64)
    lib().kvo_decode_head_rope(ctypes.byref(kv), ctypes.byref(vv), T, _p(q), float(scale), float(base),
                               int(q_pos), _p(out))
    return out


def decode_head(kview, vview, T: int, q: np.ndarray, scale: float) -> np.ndarray:
    """fp64 attention output [D] of one query (q fp32 [D])."""
    kv, _k = kview
    vv, _v = vview
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.shape[-1], dtype=np.float64)
    lib().kvo_decode_head(ctypes.byref(kv), ctypes.byref(vv), T, _p(q), float(scale), _p(out))
    return out


# ---------------------------------------------------------------------------
# SnapKV
# ---------------------------------------------------------------------------

def snapkv_scores(K: np.ndarray, w: int) -> np.ndarray:
    """fp64 scores [S] of one head; K [S][D] fp32."""
    K = np.ascontiguousarray(K, dtype=np.float32)
    S, D = K.shape
    out = np.empty(S, dtype=np.float64)
    lib().kvo_snapkv_scores(_p(K), S, D, w, _p(out))
    return out


def snapkv_scores_rows(Q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """fp64 scores [S] of one kv-head from observation rows Q [n][D] and K [S][D] (fp32)."""
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    S, D = K.shape
    out = np.empty(S, dtype=np.float64)
    lib().kvo_snapkv_scores_rows(_p(Q), Q.shape[0], _p(K), S, D, _p(out))
    return out


def maxpool1d(x: np.ndarray, kernel: int) -> np.ndarray:
    """Max over a centered window of odd width `kernel`, clipped at the ends (fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().kvo_maxpool1d(_p(x), x.shape[0], kernel, _p(out))
    return out


def snapkv_select(score: np.ndarray, n_sink: int, budget: int) -> np.ndarray:
    """Kept positions (ascending int32) from fp32 scores [S]."""
    score = np.ascontiguousarray(score, dtype=np.float32)
    S = score.shape[0]
    n = max(0, min(budget, S))
    kept = np.empty(max(n, 1), dtype=np.int32)
    k = lib().kvo_snapkv_select(_p(score), S, n_sink, budget, _p(kept))
    return kept[:k]

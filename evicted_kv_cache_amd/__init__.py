"""Python binding of libkvq (compressed-KV decode attention on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libkvq.so``.  PyTorch supplies device memory and the current HIP stream.
There is no CPU fallback: importing the binding without the built library
raises, and so does a call when no GPU is present.

The functions carry the C ABI names (see include/kvq.h):
``kvq_cache_sizes``, ``kvq_quantize_append``, ``kvq_decode_attention``,
``kvq_evict_streaming``, ``kvq_snapkv_select``, ``kvq_snapkv_select_ex``,
``kvq_snapkv_select_from_scores``, ``kvq_snapkv_pool_scores``,
``kvq_decode_workspace_bytes``, ``kvq_snapkv_workspace_bytes``,
``kvq_snapkv_workspace_bytes_ex``, ``kvq_quantize_append_at``,
``kvq_snapkv_chunk_workspace_bytes``, ``kvq_snapkv_prefill_chunk``,
``kvq_rope_table``, ``kvq_decode_attention_rope``, ``kvq_prefill_workspace_bytes``,
``kvq_prefill_attention``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

# ---- enums (mirror include/kvq.h) -------------------------------------------
KVQ_OK, KVQ_NOOP = 0, 1
KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_CAPACITY = -1, -2, -3
KVQ_ERR_ALIGNMENT, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP, KVQ_ERR_SCRATCH = -4, -5, -6, -7
KVQ_F32, KVQ_F16, KVQ_BF16 = 0, 1, 2
KVQ_PLAIN, KVQ_KIVI_CH, KVQ_TOK_AFFINE, KVQ_TOK_SYM4 = 0, 1, 2, 3
KVQ_CENTER_K, KVQ_TEST_CENTER_ANY, KVQ_POS_PER_HEAD = 0x1, 0x2, 0x4

KINDS = {"plain": KVQ_PLAIN, "kivi_ch": KVQ_KIVI_CH, "tok_affine": KVQ_TOK_AFFINE,
         "tok_sym4": KVQ_TOK_SYM4}
DTYPES = {"f32": KVQ_F32, "f16": KVQ_F16, "bf16": KVQ_BF16}

EXPORTS = ("kvq_cache_sizes", "kvq_cache_reset", "kvq_quantize_append",
           "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_evict_streaming",
           "kvq_snapkv_workspace_bytes", "kvq_snapkv_select",
           "kvq_snapkv_select_from_scores", "kvq_snapkv_workspace_bytes_ex",
           "kvq_snapkv_select_ex", "kvq_snapkv_pool_scores", "kvq_quantize_append_at",
           "kvq_snapkv_chunk_workspace_bytes", "kvq_snapkv_prefill_chunk", "kvq_rope_table",
           "kvq_decode_attention_rope", "kvq_prefill_workspace_bytes", "kvq_prefill_attention",
           "kvq_decode_attention_noalloc", "kvq_snapkv_set_wait_us", "kvq_status_string",
           "kvq_version")


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})" if what else status_string(status))


class c_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_kv_heads", "head_dim", "capacity", "k_kind", "k_bits", "k_group",
        "v_kind", "v_bits", "v_group", "in_dtype", "flags")]


class c_cache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_meta", ctypes.c_void_p),
                ("k_resid", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_meta", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("k_row", ctypes.c_void_p), ("k_bias", ctypes.c_void_p),
                ("n_stored", ctypes.c_int32), ("n_quant", ctypes.c_int32),
                ("next_pos", ctypes.c_int32), ("n_head", ctypes.c_int32)]


class c_snapkv_opts(ctypes.Structure):
    _fields_ = [("q_window", ctypes.c_void_p), ("n_q_heads", ctypes.c_int32),
                ("pool_kernel", ctypes.c_int32)]


class c_snapkv_state(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("capacity", ctypes.c_int32), ("n_kept", ctypes.c_int32), ("next_pos", ctypes.c_int32)]


class c_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "k_codes", "k_meta", "k_resid", "v_codes", "v_meta", "pos", "k_row")] + [
        ("k_table_rows", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libkvq (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libkvq.so not built at {LIB_PATH}; run "
                              "`python -m evicted_kv_cache_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        L.kvq_cache_sizes.argtypes = [P, P]
        L.kvq_cache_reset.argtypes = [P]
        L.kvq_quantize_append.argtypes = [P, P, P, P, i32, P]
        L.kvq_decode_workspace_bytes.restype = sz
        L.kvq_decode_workspace_bytes.argtypes = [P, i32]
        L.kvq_decode_attention.argtypes = [P, P, P, i32, i32, f32, P, P, sz, P]
        L.kvq_decode_attention_noalloc.argtypes = [P, P, P, i32, i32, f32, P, P]
        L.kvq_evict_streaming.argtypes = [P, P, P, i32, i32, P]
        L.kvq_snapkv_workspace_bytes.restype = sz
        L.kvq_snapkv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.kvq_snapkv_select.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P]
        L.kvq_snapkv_select_from_scores.argtypes = [P, i32, i32, i32, i32, i32, P, P]
        L.kvq_snapkv_workspace_bytes_ex.restype = sz
        L.kvq_snapkv_workspace_bytes_ex.argtypes = [P, i32, i32, i32, i32, i32]
        L.kvq_snapkv_select_ex.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P]
        L.kvq_snapkv_pool_scores.argtypes = [P, P, i32, i32, i32, i32, P]
        L.kvq_snapkv_set_wait_us.argtypes = [i32]
        L.kvq_snapkv_set_wait_us.restype = i32
        L.kvq_quantize_append_at.argtypes = [P, P, P, P, i32, i32, P, i32, i32, P]
        L.kvq_rope_table.argtypes = [P, i32, i32, f32, P]
        L.kvq_prefill_workspace_bytes.restype = sz
        L.kvq_prefill_workspace_bytes.argtypes = [P, i32, i32]
        L.kvq_prefill_attention.argtypes = [P, P, P, i32, i32, i32, f32, i32, P, P, sz, P]
        L.kvq_decode_attention_rope.argtypes = [P, P, P, i32, i32, f32, P, i32, i32, P, P, sz, P]
        L.kvq_snapkv_chunk_workspace_bytes.restype = sz
        L.kvq_snapkv_chunk_workspace_bytes.argtypes = [P, i32, i32, i32, i32, i32]
        L.kvq_snapkv_prefill_chunk.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, P, P, sz, P]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_status_string.argtypes = [ctypes.c_int]
        L.kvq_version.restype = i32
        for name in EXPORTS:
            getattr(L, name).restype = getattr(L, name).restype or ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(status).decode()


def _check(status: int, what: str, allow_noop: bool = False) -> int:
    if status == KVQ_OK or (allow_noop and status == KVQ_NOOP):
        return status
    raise KvqError(status, what)


# ---- layout / cache ---------------------------------------------------------

@dataclass(frozen=True)
class Layout:
    batch: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    k_kind: str = "tok_affine"
    k_bits: int = 4
    k_group: int = 64
    v_kind: str = "tok_affine"
    v_bits: int = 4
    v_group: int = 64
    in_dtype: str = "f16"
    flags: int = 0

    def c(self) -> c_layout:
        return c_layout(self.batch, self.n_kv_heads, self.head_dim, self.capacity,
                        KINDS[self.k_kind], self.k_bits, self.k_group, KINDS[self.v_kind],
                        self.v_bits, self.v_group, DTYPES[self.in_dtype], self.flags)


def kvq_cache_sizes(layout: Layout) -> c_sizes:
    out = c_sizes()
    cl = layout.c()
    _check(lib().kvq_cache_sizes(ctypes.byref(cl), ctypes.byref(out)), "kvq_cache_sizes")
    return out


def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Cache:
    """A cache's device buffers (torch tensors) plus the C struct with host counters."""

    def __init__(self, layout: Layout, device="cuda", k_bias=None):
        torch = _torch()
        self.layout = layout
        sz = kvq_cache_sizes(layout)
        self.sizes = sz

        def buf(n):
            # 16-byte aligned: torch's caching allocator returns 512-byte aligned blocks
            return torch.zeros(max(int(n), 16), dtype=torch.uint8, device=device) if n else None

        self.k_codes = buf(sz.k_codes)
        self.k_meta = buf(sz.k_meta)
        self.k_resid = buf(sz.k_resid)
        self.v_codes = buf(sz.v_codes)
        self.v_meta = buf(sz.v_meta)
        self.pos = buf(sz.pos)
        self.k_row = buf(sz.k_row)
        self.k_bias = None if k_bias is None else k_bias.to(device=device, dtype=torch.float32).contiguous()
        self.c = c_cache(_ptr(self.k_codes), _ptr(self.k_meta), _ptr(self.k_resid),
                         _ptr(self.v_codes), _ptr(self.v_meta), _ptr(self.pos),
                         _ptr(self.k_row), _ptr(self.k_bias), 0, 0, 0, 0)

    @property
    def n_stored(self) -> int:
        return self.c.n_stored

    @property
    def n_quant(self) -> int:
        return self.c.n_quant

    @property
    def next_pos(self) -> int:
        return self.c.next_pos


def kvq_cache_reset(cache: Cache) -> None:
    """Zero the cache's host counters (an empty cache; device buffers untouched)."""
    _check(lib().kvq_cache_reset(ctypes.byref(cache.c)), "kvq_cache_reset")


def kvq_quantize_append(layout: Layout, cache: Cache, k_new, v_new, stream=None) -> None:
    """k_new, v_new: [B][Hkv][n_new][D] contiguous device tensors of in_dtype."""
    assert k_new.is_contiguous() and v_new.is_contiguous()
    cl = layout.c()
    _check(lib().kvq_quantize_append(ctypes.byref(cl), ctypes.byref(cache.c), k_new.data_ptr(),
                                     v_new.data_ptr(), int(k_new.shape[2]), _stream(stream)),
           "kvq_quantize_append")


def kvq_quantize_append_at(layout: Layout, cache: Cache, k_new, v_new, positions, next_pos: int,
                           n_new: int | None = None, stream=None) -> None:
    """Append rows [0, n_new) of each slice of k_new, v_new [B][Hkv][rows][D]
    (contiguous; rows >= n_new) at the given positions ([B][Hkv][rows'] int32
    with KVQ_POS_PER_HEAD, else [n_new]); the cache's counter becomes next_pos."""
    assert k_new.is_contiguous() and v_new.is_contiguous() and positions.is_contiguous()
    n = int(k_new.shape[2]) if n_new is None else int(n_new)
    pos_rows = int(positions.shape[-1]) if positions.dim() == 3 else 0
    cl = layout.c()
    _check(lib().kvq_quantize_append_at(ctypes.byref(cl), ctypes.byref(cache.c), k_new.data_ptr(),
                                        v_new.data_ptr(), n, int(k_new.shape[2]), positions.data_ptr(),
                                        pos_rows, int(next_pos), _stream(stream)),
           "kvq_quantize_append_at")


def kvq_decode_workspace_bytes(layout: Layout, n_q_heads: int) -> int:
    cl = layout.c()
    return int(lib().kvq_decode_workspace_bytes(ctypes.byref(cl), n_q_heads))


def _qdtype(t) -> int:
    torch = _torch()
    return {torch.float32: KVQ_F32, torch.float16: KVQ_F16, torch.bfloat16: KVQ_BF16}[t.dtype]


def kvq_decode_attention(layout: Layout, cache: Cache, q, sm_scale: float = 0.0, out=None,
                         ws=None, stream=None):
    """q: [B][Hq][D] device tensor (f32/f16/bf16).  Returns out [B][Hq][D] fp32."""
    torch = _torch()
    assert q.is_contiguous()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    nbytes = kvq_decode_workspace_bytes(layout, Hq)
    if ws is None:
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    cl = layout.c()
    _check(lib().kvq_decode_attention(ctypes.byref(cl), ctypes.byref(cache.c), q.data_ptr(),
                                      _qdtype(q), Hq, float(sm_scale), out.data_ptr(),
                                      ws.data_ptr(), ws.numel() * ws.element_size(),
                                      _stream(stream)),
           "kvq_decode_attention")
    return out


def kvq_decode_attention_noalloc(layout: Layout, cache: Cache, q, sm_scale: float = 0.0, out=None,
                                 stream=None):
    """kvq_decode_attention without a workspace: the library's fixed per-GPU
    scratch holds the split partials.  q: [B][Hq][D]; returns out [B][Hq][D] fp32."""
    torch = _torch()
    assert q.is_contiguous()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    cl = layout.c()
    _check(lib().kvq_decode_attention_noalloc(ctypes.byref(cl), ctypes.byref(cache.c), q.data_ptr(),
                                              _qdtype(q), Hq, float(sm_scale), out.data_ptr(),
                                              _stream(stream)),
           "kvq_decode_attention_noalloc")
    return out


def kvq_prefill_workspace_bytes(layout: Layout, n_q_heads: int, n_q: int) -> int:
    cl = layout.c()
    return int(lib().kvq_prefill_workspace_bytes(ctypes.byref(cl), n_q_heads, n_q))


def kvq_prefill_attention(layout: Layout, cache: Cache, q, causal: bool = False, sm_scale: float = 0.0,
                          out=None, ws=None, stream=None):
    """q: [B][Hq][n_q][D] device tensor.  Returns out [B][Hq][n_q][D] fp32."""
    torch = _torch()
    assert q.is_contiguous() and q.dim() == 4
    B, Hq, n_q, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, n_q, D), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(kvq_prefill_workspace_bytes(layout, Hq, n_q), 16), dtype=torch.uint8,
                         device=q.device)
    cl = layout.c()
    _check(lib().kvq_prefill_attention(ctypes.byref(cl), ctypes.byref(cache.c), q.data_ptr(), _qdtype(q), Hq,
                                       n_q, float(sm_scale), int(bool(causal)), out.data_ptr(), ws.data_ptr(),
                                       ws.numel() * ws.element_size(), _stream(stream)),
           "kvq_prefill_attention")
    return out


def kvq_rope_table(n_pos: int, head_dim: int, base: float = 10000.0, device="cuda", stream=None):
    """(cos, sin) table [n_pos][head_dim/2][2] fp32 for RoPE on read."""
    torch = _torch()
    t = torch.empty((n_pos, head_dim // 2, 2), dtype=torch.float32, device=device)
    _check(lib().kvq_rope_table(t.data_ptr(), n_pos, head_dim, float(base), _stream(stream)), "kvq_rope_table")
    return t


def kvq_decode_attention_rope(layout: Layout, cache: Cache, q, rope_table, q_pos: int,
                              sm_scale: float = 0.0, out=None, ws=None, stream=None):
    """kvq_decode_attention with keys rotated at their slot index and the
    query (q [B][Hq][D], before the rotation) at q_pos."""
    torch = _torch()
    assert q.is_contiguous() and rope_table.is_contiguous() and rope_table.dtype == torch.float32
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(kvq_decode_workspace_bytes(layout, Hq), 16), dtype=torch.uint8, device=q.device)
    cl = layout.c()
    _check(lib().kvq_decode_attention_rope(ctypes.byref(cl), ctypes.byref(cache.c), q.data_ptr(), _qdtype(q),
                                           Hq, float(sm_scale), rope_table.data_ptr(), int(rope_table.shape[0]),
                                           int(q_pos), out.data_ptr(), ws.data_ptr(),
                                           ws.numel() * ws.element_size(), _stream(stream)),
           "kvq_decode_attention_rope")
    return out


def kvq_evict_streaming(layout: Layout, src: Cache, dst: Cache, sink: int, window: int,
                        stream=None) -> int:
    """Returns KVQ_OK (dst now holds the compacted cache) or KVQ_NOOP (src unchanged)."""
    cl = layout.c()
    return _check(lib().kvq_evict_streaming(ctypes.byref(cl), ctypes.byref(src.c),
                                            ctypes.byref(dst.c), sink, window, _stream(stream)),
                  "kvq_evict_streaming", allow_noop=True)


def kvq_snapkv_workspace_bytes(batch, n_kv_heads, seq_len, head_dim, obs_window) -> int:
    return int(lib().kvq_snapkv_workspace_bytes(batch, n_kv_heads, seq_len, head_dim, obs_window))


def kvq_snapkv_select(k, v, obs_window: int, n_sink: int, budget: int, scores=None,
                      kept=None, k_out=None, v_out=None, ws=None, stream=None):
    """k, v: [B][Hkv][S][D] fp16 device tensors.  Returns (scores, kept, k_out, v_out)."""
    torch = _torch()
    assert k.dtype == torch.float16 and v.dtype == torch.float16
    assert k.is_contiguous() and v.is_contiguous()
    B, H, S, D = k.shape
    n_keep = min(budget, S)
    dev = k.device
    if scores is None:
        scores = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    if kept is None:
        kept = torch.empty((B, H, n_keep), dtype=torch.int32, device=dev)
    if k_out is None:
        k_out = torch.empty((B, H, n_keep, D), dtype=torch.float16, device=dev)
    if v_out is None:
        v_out = torch.empty((B, H, n_keep, D), dtype=torch.float16, device=dev)
    if ws is None:
        ws = torch.empty(max(kvq_snapkv_workspace_bytes(B, H, S, D, obs_window), 16),
                         dtype=torch.uint8, device=dev)
    _check(lib().kvq_snapkv_select(k.data_ptr(), v.data_ptr(), B, H, S, D, obs_window, n_sink,
                                   budget, scores.data_ptr(), kept.data_ptr(), k_out.data_ptr(),
                                   v_out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)),
           "kvq_snapkv_select")
    return scores, kept, k_out, v_out


def _snap_opts(q_window, pool_kernel: int):
    torch = _torch()
    if q_window is None:
        return c_snapkv_opts(None, 0, pool_kernel)
    assert q_window.dtype == torch.float16 and q_window.is_contiguous() and q_window.dim() == 4
    return c_snapkv_opts(q_window.data_ptr(), q_window.shape[1], pool_kernel)


def kvq_snapkv_workspace_bytes_ex(batch, n_kv_heads, seq_len, head_dim, obs_window,
                                  q_window=None, pool_kernel: int = 1) -> int:
    o = _snap_opts(q_window, pool_kernel)
    return int(lib().kvq_snapkv_workspace_bytes_ex(ctypes.byref(o), batch, n_kv_heads, seq_len,
                                                   head_dim, obs_window))


def kvq_snapkv_select_ex(k, v, obs_window: int, n_sink: int, budget: int, q_window=None,
                         pool_kernel: int = 1, scores=None, kept=None, k_out=None, v_out=None,
                         ws=None, stream=None):
    """kvq_snapkv_select with query windows q_window [B][Hq][obs_window][D] fp16
    (None: the key proxy) and max-pool width pool_kernel (1: none).
    Returns (scores, kept, k_out, v_out); scores are the unpooled ones."""
    torch = _torch()
    assert k.dtype == torch.float16 and v.dtype == torch.float16
    assert k.is_contiguous() and v.is_contiguous()
    B, H, S, D = k.shape
    if q_window is not None:
        assert q_window.shape[0] == B and q_window.shape[2] == obs_window and q_window.shape[3] == D
    n_keep = min(budget, S)
    dev = k.device
    if scores is None:
        scores = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    if kept is None:
        kept = torch.empty((B, H, n_keep), dtype=torch.int32, device=dev)
    if k_out is None:
        k_out = torch.empty((B, H, n_keep, D), dtype=torch.float16, device=dev)
    if v_out is None:
        v_out = torch.empty((B, H, n_keep, D), dtype=torch.float16, device=dev)
    o = _snap_opts(q_window, pool_kernel)
    if ws is None:
        nb = lib().kvq_snapkv_workspace_bytes_ex(ctypes.byref(o), B, H, S, D, obs_window)
        ws = torch.empty(max(int(nb), 16), dtype=torch.uint8, device=dev)
    _check(lib().kvq_snapkv_select_ex(ctypes.byref(o), k.data_ptr(), v.data_ptr(), B, H, S, D,
                                      obs_window, n_sink, budget, scores.data_ptr(),
                                      kept.data_ptr(), k_out.data_ptr(), v_out.data_ptr(),
                                      ws.data_ptr(), ws.numel(), _stream(stream)),
           "kvq_snapkv_select_ex")
    return scores, kept, k_out, v_out


def kvq_snapkv_set_wait_us(microseconds: int) -> int:
    """Bound (us) on the one-read SnapKV scores' wait for the rest of a head;
    returns the previous bound."""
    return int(lib().kvq_snapkv_set_wait_us(int(microseconds)))


def kvq_snapkv_pool_scores(scores, pool_kernel: int, pooled=None, stream=None):
    """Max-pool smoothing of [B][Hkv][S] fp32 scores over odd width pool_kernel."""
    torch = _torch()
    assert scores.dtype == torch.float32 and scores.is_contiguous()
    B, H, S = scores.shape
    if pooled is None:
        pooled = torch.empty_like(scores)
    _check(lib().kvq_snapkv_pool_scores(scores.data_ptr(), pooled.data_ptr(), B, H, S, pool_kernel,
                                        _stream(stream)), "kvq_snapkv_pool_scores")
    return pooled


def kvq_snapkv_select_from_scores(scores, n_sink: int, budget: int, kept=None, stream=None):
    """scores: [B][Hkv][S] fp32 device tensor.  Returns kept [B][Hkv][min(budget,S)] int32."""
    torch = _torch()
    assert scores.dtype == torch.float32 and scores.is_contiguous()
    B, H, S = scores.shape
    if kept is None:
        kept = torch.empty((B, H, min(budget, S)), dtype=torch.int32, device=scores.device)
    _check(lib().kvq_snapkv_select_from_scores(scores.data_ptr(), B, H, S, n_sink, budget,
                                               kept.data_ptr(), _stream(stream)),
           "kvq_snapkv_select_from_scores")
    return kept


class SnapState:
    """Rows kept by chunked SnapKV prefill: device k, v [B][Hkv][capacity][D]
    fp16 and pos [B][Hkv][capacity] int32, plus the C struct's host counters."""

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, capacity: int, device="cuda"):
        torch = _torch()
        self.k = torch.zeros((batch, n_kv_heads, capacity, head_dim), dtype=torch.float16, device=device)
        self.v = torch.zeros_like(self.k)
        self.pos = torch.zeros((batch, n_kv_heads, capacity), dtype=torch.int32, device=device)
        self.c = c_snapkv_state(self.k.data_ptr(), self.v.data_ptr(), self.pos.data_ptr(), capacity, 0, 0)

    @property
    def n_kept(self) -> int:
        return self.c.n_kept

    @property
    def next_pos(self) -> int:
        return self.c.next_pos


def kvq_snapkv_chunk_workspace_bytes(batch, n_kv_heads, head_dim, capacity, obs_window,
                                     q_window=None, pool_kernel: int = 1) -> int:
    o = _snap_opts(q_window, pool_kernel)
    return int(lib().kvq_snapkv_chunk_workspace_bytes(ctypes.byref(o), batch, n_kv_heads, head_dim,
                                                      capacity, obs_window))


def kvq_snapkv_prefill_chunk(state_in: SnapState, state_out: SnapState, k_chunk, v_chunk,
                             obs_window: int, n_sink: int, budget: int, q_window=None,
                             pool_kernel: int = 1, scores=None, ws=None, stream=None):
    """One chunk of SnapKV prefill: k_chunk, v_chunk [B][Hkv][n][D] fp16 are
    appended to state_in's kept rows, the selection runs over all of them and
    the kept rows land in state_out.  Returns state_out."""
    torch = _torch()
    assert k_chunk.dtype == torch.float16 and k_chunk.is_contiguous() and v_chunk.is_contiguous()
    B, H, n, D = k_chunk.shape
    o = _snap_opts(q_window, pool_kernel)
    if ws is None:
        nb = lib().kvq_snapkv_chunk_workspace_bytes(ctypes.byref(o), B, H, D, state_in.c.capacity, obs_window)
        ws = torch.empty(max(int(nb), 16), dtype=torch.uint8, device=k_chunk.device)
    _check(lib().kvq_snapkv_prefill_chunk(ctypes.byref(o), ctypes.byref(state_in.c), ctypes.byref(state_out.c),
                                          k_chunk.data_ptr(), v_chunk.data_ptr(), n, B, H, D, obs_window,
                                          n_sink, budget, _ptr(scores), ws.data_ptr(), ws.numel(),
                                          _stream(stream)),
           "kvq_snapkv_prefill_chunk")
    return state_out

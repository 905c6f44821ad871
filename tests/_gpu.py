"""Plumbing shared by the GPU parity tests: moving seeded inputs to the GPU,
building matching product and oracle caches, and unpacking the product's
packed buffers into the oracle's canonical (one code per byte) arrays.
Nothing here computes any part of the method.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import evicted_kv_cache_amd as K
from oracle.cache import Layout as OLayout
from oracle.cache import OracleCache

DEV = "cuda"
NP_OF = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
TORCH_OF = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def say(*a):
    """Name the case before GPU work (flushes, so a dying box still shows it)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(x)
    return t.to(DEV)


def layouts(**kw):
    """(product Layout, oracle Layout) with the same fields."""
    flags = kw.pop("flags", 0)
    ol = OLayout(pos_per_head=bool(flags & K.KVQ_POS_PER_HEAD), **kw)
    pl = K.Layout(flags=flags, **kw)
    return pl, ol


def _sel(buf: torch.Tensor, B, H, row_bytes, bh):
    """Bytes of buffer [B][H][rows][row_bytes]; optionally only slice (b, h), as [1][1][...]."""
    t = buf.view(B, H, -1, row_bytes)
    if bh is not None:
        b, h = bh
        t = t[b:b + 1, h:h + 1]
    return t.cpu().numpy()


def unpack_codes(buf: torch.Tensor, B, H, cap, D, bits, bh=None) -> np.ndarray:
    raw = _sel(buf, B, H, D * bits // 8, bh)
    if bh is not None:
        B = H = 1
    if bits == 8:
        return raw.copy()
    out = np.empty((B, H, cap, D), dtype=np.uint8)
    if bits == 2:
        for r in range(4):
            out[..., r::4] = (raw >> (2 * r)) & 0x3
        return out
    out[..., 0::2] = raw & 0xF
    out[..., 1::2] = raw >> 4
    return out


def u16(buf: torch.Tensor, shape) -> np.ndarray:
    return buf.cpu().numpy().view(np.uint16).reshape(shape)


def i32(buf: torch.Tensor, n) -> np.ndarray:
    return buf.cpu().numpy().view(np.int32)[:n]


def gpu_state(c: K.Cache, bh=None):
    """Canonical numpy view of a product cache, trimmed to the stored slots
    (optionally only slice bh = (b, h), shaped [1][1][...])."""
    L = c.layout
    B, H, D, C = L.batch, L.n_kv_heads, L.head_dim, L.capacity
    n, nq = c.n_stored, c.n_quant
    es = {"f32": 4, "f16": 2, "bf16": 2}[L.in_dtype]
    npdt = NP_OF[L.in_dtype]
    if L.flags & K.KVQ_POS_PER_HEAD:
        st = {"pos": _sel(c.pos, B, H, C * 4, bh).view(np.int32).reshape(
            B if bh is None else 1, H if bh is None else 1, C)[:, :, :n]}
    else:
        st = {"pos": i32(c.pos, n)}
    if L.k_kind == "plain":
        st["k_plain"] = _sel(c.k_codes, B, H, D * es, bh).view(npdt)[:, :, :n]
    else:
        st["k_u"] = unpack_codes(c.k_codes, B, H, C, D, L.k_bits, bh)[:, :, :nq]
    if L.k_kind == "tok_affine":
        st["k_meta"] = _sel(c.k_meta, B, H, D // L.k_group * 4, bh).view(np.uint16)[:, :, :n].reshape(
            -1 if bh is None else 1, *((H,) if bh is None else (1,)), n, D // L.k_group, 2)
    elif L.k_kind == "tok_sym4":
        st["k_meta"] = _sel(c.k_meta, B, H, D // 32 * 2, bh).view(np.uint16)[:, :, :n]
    elif L.k_kind == "kivi_ch":
        rows = c.sizes.k_table_rows
        st["k_row"] = i32(c.k_row, nq)
        live = int(st["k_row"].max()) + 1 if nq else 0
        st["k_table"] = _sel(c.k_meta, B, H, D * 4, bh).view(np.uint16)[:, :, :live].reshape(
            -1 if bh is None else 1, *((H,) if bh is None else (1,)), live, D, 2)
        st["k_resid"] = _sel(c.k_resid, B, H, D * es, bh).view(npdt)[:, :, :n - nq]
    if L.v_kind == "plain":
        st["v_plain"] = _sel(c.v_codes, B, H, D * es, bh).view(npdt)[:, :, :n]
    else:
        st["v_u"] = unpack_codes(c.v_codes, B, H, C, D, L.v_bits, bh)[:, :, :n]
        st["v_meta"] = _sel(c.v_meta, B, H, D // L.v_group * 4, bh).view(np.uint16)[:, :, :n].reshape(
            -1 if bh is None else 1, *((H,) if bh is None else (1,)), n, D // L.v_group, 2)
    return st


def oracle_state(o: OracleCache):
    L = o.L
    n, nq = o.n_stored, o.n_quant
    st = {"pos": o.pos[..., :n]}
    if L.k_kind == "plain":
        st["k_plain"] = o.k_plain[:, :, :n]
    else:
        st["k_u"] = o.k_u[:, :, :nq]
    if L.k_kind in ("tok_affine", "tok_sym4"):
        st["k_meta"] = o.k_meta[:, :, :n]
    elif L.k_kind == "kivi_ch":
        st["k_row"] = o.k_row[:nq]
        live = int(st["k_row"].max()) + 1 if nq else 0
        st["k_table"] = o.k_table[:, :, :live]
        st["k_resid"] = o.k_resid[:, :, :n - nq]
    if L.v_kind == "plain":
        st["v_plain"] = o.v_plain[:, :, :n]
    else:
        st["v_u"] = o.v_u[:, :, :n]
        st["v_meta"] = o.v_meta[:, :, :n]
    return st


def assert_same_state(c: K.Cache, o: OracleCache, bh=None):
    """Bit-exact comparison; with bh = (b, h) the oracle cache holds only that slice."""
    assert (c.n_stored, c.n_quant, c.next_pos) == (o.n_stored, o.n_quant, o.next_pos)
    g, r = gpu_state(c, bh), oracle_state(o)
    assert set(g) == set(r)
    for name in r:
        a = np.ascontiguousarray(g[name])
        b = np.ascontiguousarray(r[name])
        assert a.shape == b.shape, (name, a.shape, b.shape)
        if a.dtype != b.dtype:
            a, b = a.view(np.uint8), b.view(np.uint8)
        if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}")


def attn_err(out_gpu: np.ndarray, out_ref: np.ndarray) -> float:
    """max |o - o_ref| / max_d |o_ref| per (b, hq) row, maximized over rows."""
    ref = out_ref.astype(np.float64)
    den = np.abs(ref).max(axis=-1, keepdims=True)
    return float((np.abs(out_gpu.astype(np.float64) - ref) / den).max())


def default_scale(D):
    return 1.0 / math.sqrt(D)

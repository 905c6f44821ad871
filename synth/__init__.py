"""Seeded synthetic inputs for the compressed-KV decode path.

This module is shared by the CPU oracle, the parity tests and the benchmark.
It draws random numbers and casts them to the storage dtype of a workload; it
holds none of the method's arithmetic (no quantization, attention, scoring or
selection).

Every (batch, kv-head) slice has its own numpy PCG64 stream
``default_rng([seed, config_id, b, h])`` so any slice can be regenerated alone.
Draw order inside a slice stream: K [T][D], then V [T][D], then the queries of
that kv-head's query-head group [G][D].  Per-kv-head parameters (the K channel
bias and the choice of outlier channels) come from a second stream
``default_rng([seed, config_id, HEAD_STREAM, h])``, drawn in that order.
The prompt's last queries (SnapKV observation windows) of slice (b, h) come
from a third stream ``default_rng([seed, config_id, QWIN_STREAM, b, h])``:
[G][n][D] for the G query heads of kv-head h.
All draws are float32 standard normals; N(0, sigma) means standard deviation
sigma.  Values are cast to the workload's dtype with round-to-nearest-even.

The five workloads mirror the shapes the source pages discuss:
  kivi_int8_tiny     tinygpt head shape (8 heads x 32), KIVI int8, StreamingLLM
                     sink 4 + window 256 over 500 generated positions
  llama3b_kivi_int4  Llama-3.2-3B layer shape, 24/8 heads x 128, T=8192, KIVI int4,
                     6 (=5%) outlier K channels per kv-head scaled x10
  snapkv_prefill     SnapKV defaults: 8 kv-heads x 128, S=8192, window 32,
                     sink 4, budget 512
  q4_0_centered      Q4_0-style K with per-(kv-head, channel) mean bias N(0,1.5),
                     32/8 heads x 128, batch 16, T=16384, int8 V
  affine4_g64        mlx-lm-style 4-bit affine g64 K and V, 32/8 heads x 128,
                     batch 64, T=32768, bf16
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 0
HEAD_STREAM = 1 << 20
QWIN_STREAM = 1 << 21


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int          # T (decode) or S (SnapKV prefill)
    dtype: str            # "f32" | "f16" | "bf16" for K/V/q
    k_bias_std: float = 0.0
    n_outlier_channels: int = 0
    outlier_scale: float = 1.0
    extra: dict = field(default_factory=dict, hash=False, compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "kivi_int8_tiny": Workload(
        "kivi_int8_tiny", 1, 1, 8, 8, 32, 500, "f32", k_bias_std=2.0,
        extra=dict(k_kind="kivi_ch", k_bits=8, k_group=32, v_bits=8, v_group=32,
                   sink=4, window=256)),
    "llama3b_kivi_int4": Workload(
        "llama3b_kivi_int4", 2, 1, 24, 8, 128, 8192, "f16",
        n_outlier_channels=6, outlier_scale=10.0,
        extra=dict(k_kind="kivi_ch", k_bits=4, k_group=32, v_bits=4, v_group=32)),
    "snapkv_prefill": Workload(
        "snapkv_prefill", 3, 1, 8, 8, 128, 8192, "f16",
        extra=dict(obs_window=32, n_sink=4, budget=512)),
    "q4_0_centered": Workload(
        "q4_0_centered", 4, 16, 32, 8, 128, 16384, "f16", k_bias_std=1.5,
        extra=dict(k_kind="tok_sym4", k_bits=4, k_group=32, v_bits=8, v_group=128)),
    "affine4_g64": Workload(
        "affine4_g64", 5, 64, 32, 8, 128, 32768, "bf16",
        extra=dict(k_kind="tok_affine", k_bits=4, k_group=64, v_bits=4, v_group=64)),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with some sizes overridden (smaller parity cases)."""
    base = WORKLOADS[name]
    if not overrides:
        return base
    kw = {k: getattr(base, k) for k in base.__dataclass_fields__}
    extra = dict(base.extra)
    extra.update(overrides.pop("extra", {}))
    kw.update(overrides)
    kw["extra"] = extra
    return Workload(**kw)


# ----------------------------------------------------------------------------
# dtype casts (storage formats of the synthetic data)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover - torch is always present here
        b = x.view(np.uint32).astype(np.uint64)
        r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
        return r.astype(np.uint16)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 draws to the storage dtype.  bf16 is returned as uint16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values back to float32 (test plumbing)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def head_params(w: Workload, h: int):
    """(bias [D] float32 or None, outlier channel indices) for kv-head h."""
    rng = np.random.default_rng([SEED, w.config_id, HEAD_STREAM, h])
    bias = None
    if w.k_bias_std:
        bias = (rng.standard_normal(w.head_dim, dtype=np.float32)
                * np.float32(w.k_bias_std)).astype(np.float32)
    outl = np.zeros(0, dtype=np.int64)
    if w.n_outlier_channels:
        outl = np.sort(rng.choice(w.head_dim, size=w.n_outlier_channels, replace=False))
    return bias, outl


def slice_f32(w: Workload, b: int, h: int, T: int | None = None):
    """float32 draws (K [T][D], V [T][D], Q [G][D]) for slice (b, h) before the cast.

    ``T`` defaults to the workload length; a shorter T yields a prefix of the
    same stream only for K (V and Q come after K in the stream), so callers
    that shrink T get a different but equally valid slice.
    """
    T = w.seq_len if T is None else T
    D = w.head_dim
    rng = np.random.default_rng([SEED, w.config_id, b, h])
    k = rng.standard_normal((T, D), dtype=np.float32)
    v = rng.standard_normal((T, D), dtype=np.float32)
    q = rng.standard_normal((w.group, D), dtype=np.float32)
    bias, outl = head_params(w, h)
    if bias is not None:
        k += bias[None, :]
    if outl.size:
        k[:, outl] *= np.float32(w.outlier_scale)
    return k, v, q


def slice_cast(w: Workload, b: int, h: int, T: int | None = None):
    """Slice (b, h) in the workload's storage dtype: (K, V, Q)."""
    k, v, q = slice_f32(w, b, h, T)
    return cast(k, w.dtype), cast(v, w.dtype), cast(q, w.dtype)


def query_window(w: Workload, b: int, h: int, n: int, group: int | None = None):
    """Observation-window queries [G][n][D] of kv-head h in storage dtype."""
    G = w.group if group is None else group
    rng = np.random.default_rng([SEED, w.config_id, QWIN_STREAM, b, h])
    return cast(rng.standard_normal((G, n, w.head_dim), dtype=np.float32), w.dtype)


def full(w: Workload, T: int | None = None, batch: int | None = None,
         threads: int = 8):
    """Whole tensors K, V [B][Hkv][T][D] and Q [B][Hq][D] in storage dtype.

    Slices are generated in parallel threads (numpy releases the GIL).
    """
    T = w.seq_len if T is None else T
    B = w.batch if batch is None else batch
    H = w.n_kv_heads
    D = w.head_dim
    npdt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[w.dtype]
    K = np.empty((B, H, T, D), dtype=npdt)
    V = np.empty((B, H, T, D), dtype=npdt)
    Q = np.empty((B, w.n_q_heads, D), dtype=npdt)

    def one(idx):
        b, h = divmod(idx, H)
        k, v, q = slice_cast(w, b, h, T)
        K[b, h] = k
        V[b, h] = v
        Q[b, h * w.group:(h + 1) * w.group] = q

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(B * H)))
    return K, V, Q

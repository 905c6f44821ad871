"""Oracle cache model -- TEST INFRASTRUCTURE ONLY.

Plain numpy bookkeeping around the C oracle's arithmetic.  It states the
semantics the HIP library must reproduce:

* Quantize-on-write ([P1] "KIVI": K per channel, V per token, computed at
  append time).  For per-channel K the scales of a token group are frozen when
  the group's last token arrives ([P1] caveats, the KIVI group-size idea;
  [P4] s.3, the residual buffer: recent keys stay in full precision and are
  attended in full precision until their block closes).  The group of a token
  is its append index divided by the group size.
* StreamingLLM compaction ([P1] "Implementation"): when more than
  sink + window slots are stored, keep slots [0, sink) and the last `window`
  slots, in order.  Only rows are dropped: kept tokens keep their codes and
  their group's frozen scales ([P1]: per-channel K scales are not sliced by
  the eviction).  Per-channel scale rows no kept token refers to are dropped;
  the remaining rows keep ascending group order.
* Decode attention over the dequantized cache ([P4] s.1: scores against the
  packed keys, softmax, weighted sum of the packed values) in fp64.
* SnapKV ([P2] "How it works"): observation-window scores, sink guarantee,
  top-k by score with lower position first on ties, ascending union, gather.
  Chunked prefill ([P2] "How it works" and "RoPE position semantics": every
  prefill call selects again, so the budget stays capped across chunks; kept
  rows keep their absolute positions) re-runs the selection over the kept
  rows followed by the new chunk.  Decode appends never pass through it.
* Kept rows stacked into a quantized cache ([P2]: the kept tokens can carry
  any quantizer) are appended at their own positions, which differ between
  kv-heads, so such a cache keeps one position row per (batch, kv-head).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import (CHANNEL, PLAIN, SYM4, TOK_AFFINE, decode_head, decode_head_rope, make_view, maxpool1d,
               quant_channel_group, quant_sym4, quant_tok_affine, snapkv_scores,
               snapkv_scores_rows, snapkv_select, widen)

_NP_STORE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


class OracleError(Exception):
    pass


@dataclass(frozen=True)
class Layout:
    batch: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    k_kind: str = "tok_affine"    # plain | kivi_ch | tok_affine | tok_sym4
    k_bits: int = 4
    k_group: int = 64             # tokens/group (kivi_ch), channels/group (tok_affine), 32 (sym4)
    v_kind: str = "tok_affine"    # plain | tok_affine
    v_bits: int = 4
    v_group: int = 64
    in_dtype: str = "f16"
    pos_per_head: bool = False    # positions [B][H][capacity] instead of [capacity]

    @property
    def table_rows(self) -> int:
        # At most two runs of consecutive positions are stored (the sinks and
        # the window); each run of L slots touches at most L/G + 2 groups.
        return self.capacity // self.k_group + 3 if self.k_kind == "kivi_ch" else 0


class OracleCache:
    def __init__(self, L: Layout, k_bias: np.ndarray | None = None):
        self.L = L
        B, H, D, C = L.batch, L.n_kv_heads, L.head_dim, L.capacity
        st = _NP_STORE[L.in_dtype]
        self.k_bias = None if k_bias is None else np.asarray(k_bias, dtype=np.float32)
        self.pos = np.zeros((B, H, C) if L.pos_per_head else C, dtype=np.int32)
        self.k_row = np.zeros(C, dtype=np.int32)
        self.k_plain = self.k_u = self.k_meta = self.k_table = self.k_resid = None
        if L.k_kind == "plain":
            self.k_plain = np.zeros((B, H, C, D), dtype=st)
        else:
            self.k_u = np.zeros((B, H, C, D), dtype=np.uint8)
        if L.k_kind == "tok_affine":
            self.k_meta = np.zeros((B, H, C, D // L.k_group, 2), dtype=np.uint16)
        elif L.k_kind == "tok_sym4":
            self.k_meta = np.zeros((B, H, C, D // 32), dtype=np.uint16)
        elif L.k_kind == "kivi_ch":
            self.k_table = np.zeros((B, H, L.table_rows, D, 2), dtype=np.uint16)
            self.k_resid = np.zeros((B, H, L.k_group, D), dtype=st)
        self.v_plain = self.v_u = self.v_meta = None
        if L.v_kind == "plain":
            self.v_plain = np.zeros((B, H, C, D), dtype=st)
        else:
            self.v_u = np.zeros((B, H, C, D), dtype=np.uint8)
            self.v_meta = np.zeros((B, H, C, D // L.v_group, 2), dtype=np.uint16)
        self.n_stored = 0
        self.n_quant = 0       # slots whose K is coded (kivi_ch); == n_stored otherwise
        self.next_pos = 0

    # ------------------------------------------------------------------ append
    def append(self, k_new: np.ndarray, v_new: np.ndarray, positions: np.ndarray | None = None,
               next_pos: int | None = None) -> None:
        """k_new, v_new: [B][H][n][D] in the layout's input dtype.

        The new slots take positions next_pos, next_pos + 1, ...; or, when
        ``positions`` is given ([B][H][n] for a per-head layout, else [n]),
        those positions, after which the generation counter becomes
        ``next_pos``."""
        L = self.L
        n = k_new.shape[2]
        if self.n_stored + n > L.capacity:
            raise OracleError("capacity")
        s0 = self.n_stored
        sl = slice(s0, s0 + n)
        if positions is None:
            self.pos[..., sl] = self.next_pos + np.arange(n, dtype=np.int32)
        else:
            self.pos[..., sl] = np.asarray(positions, dtype=np.int32)
        # V: per token, at write time ([P1] "KIVI": one (scale, zero) per token, fixed once written).
        if L.v_kind == "plain":
            self.v_plain[:, :, sl] = v_new
        else:
            u, m = quant_tok_affine(widen(v_new, L.in_dtype), L.v_group, L.v_bits)
            self.v_u[:, :, sl] = u
            self.v_meta[:, :, sl] = m
        # K
        if L.k_kind == "plain":
            self.k_plain[:, :, sl] = k_new
        elif L.k_kind == "tok_affine":
            u, m = quant_tok_affine(widen(k_new, L.in_dtype), L.k_group, L.k_bits)
            self.k_u[:, :, sl] = u
            self.k_meta[:, :, sl] = m
        elif L.k_kind == "tok_sym4":
            x = widen(k_new, L.in_dtype)
            for h in range(L.n_kv_heads):
                bias = None if self.k_bias is None else self.k_bias[h]
                u, sc = quant_sym4(x[:, h], bias)
                self.k_u[:, h, sl] = u
                self.k_meta[:, h, sl] = sc
        elif L.k_kind == "kivi_ch":
            Gt = L.k_group
            for i in range(n):
                r = self.n_stored + i - self.n_quant   # residual fill before this token
                self.k_resid[:, :, r] = k_new[:, :, i]
                if r + 1 == Gt:
                    self._close_group()
        self.n_stored += n
        self.next_pos = self.next_pos + n if positions is None else int(next_pos)
        if L.k_kind != "kivi_ch":
            self.n_quant = self.n_stored

    def _close_group(self) -> None:
        """Freeze the per-channel scales of the full residual group."""
        L = self.L
        Gt = L.k_group
        q0 = self.n_quant
        row = int(self.k_row[q0 - 1]) + 1 if q0 > 0 else 0
        if row >= L.table_rows:
            raise OracleError("table rows")
        x = widen(self.k_resid, L.in_dtype)
        for b in range(L.batch):
            for h in range(L.n_kv_heads):
                u, m = quant_channel_group(x[b, h], L.k_bits)
                self.k_u[b, h, q0:q0 + Gt] = u
                self.k_table[b, h, row] = m
        self.k_row[q0:q0 + Gt] = row
        self.n_quant += Gt

    # ------------------------------------------------------------------- evict
    def evict(self, sink: int, window: int):
        """StreamingLLM compaction.  Returns a new cache, or None when nothing is dropped."""
        L = self.L
        n = self.n_stored
        if n <= sink + window:
            return None
        if L.k_kind == "kivi_ch" and window < n - self.n_quant:
            raise OracleError("window must cover the open K group")
        keep = np.concatenate([np.arange(0, sink), np.arange(n - window, n)]).astype(np.int64)
        new = OracleCache(L, self.k_bias)
        m = keep.size
        new.pos[..., :m] = self.pos[..., keep]
        for name in ("k_plain", "k_u", "k_meta", "v_plain", "v_u", "v_meta"):
            a = getattr(self, name)
            if a is not None and not (name == "k_meta" and L.k_kind == "kivi_ch"):
                getattr(new, name)[:, :, :m] = a[:, :, keep]
        if L.k_kind == "kivi_ch":
            kq = keep[keep < self.n_quant]
            old_rows = self.k_row[kq]
            live = np.unique(old_rows)          # ascending group order
            new.k_row[:kq.size] = np.searchsorted(live, old_rows).astype(np.int32)
            new.k_table[:, :, :live.size] = self.k_table[:, :, live]
            new.k_resid[...] = self.k_resid
            new.n_quant = kq.size
        else:
            new.n_quant = m
        new.n_stored = m
        new.next_pos = self.next_pos
        return new

    # ------------------------------------------------------------------ decode
    def views(self, b: int, h: int):
        L = self.L
        D = L.head_dim
        T = self.n_stored
        if L.k_kind == "plain":
            kv = make_view(PLAIN, D, plain=widen(self.k_plain[b, h, :T], L.in_dtype))
        elif L.k_kind == "tok_affine":
            kv = make_view(TOK_AFFINE, D, L.k_group, u=self.k_u[b, h, :T], meta=self.k_meta[b, h, :T])
        elif L.k_kind == "tok_sym4":
            kv = make_view(SYM4, D, u=self.k_u[b, h, :T], meta=self.k_meta[b, h, :T])
        else:
            r = T - self.n_quant
            kv = make_view(CHANNEL, D, u=self.k_u[b, h, :T], meta=self.k_table[b, h],
                           row=self.k_row[:T],
                           plain=widen(self.k_resid[b, h, :max(r, 1)], L.in_dtype),
                           n_coded=self.n_quant)
        if L.v_kind == "plain":
            vv = make_view(PLAIN, D, plain=widen(self.v_plain[b, h, :T], L.in_dtype))
        else:
            vv = make_view(TOK_AFFINE, D, L.v_group, u=self.v_u[b, h, :T], meta=self.v_meta[b, h, :T])
        return kv, vv

    def decode(self, q: np.ndarray, q_dtype: str, sm_scale: float = 0.0,
               heads=None, threads: int = 8, rope_base: float | None = None,
               q_pos: int = 0) -> np.ndarray:
        """fp64 outputs [B][Hq][D] for queries q [B][Hq][D] (stored dtype).

        ``heads`` optionally restricts the work to a list of (b, hq) pairs;
        other rows are left as NaN.  With ``rope_base`` keys and queries are
        taken as stored before the rotary embedding: the key of slot t is
        rotated at position t (its index in the compressed cache, [P1] "RoPE
        caveat": re-positioning at the compressed slot index) and the query
        at q_pos.
        """
        L = self.L
        B, Hq, D = q.shape
        gq = Hq // L.n_kv_heads
        scale = sm_scale if sm_scale > 0 else 1.0 / math.sqrt(D)
        qf = widen(q, q_dtype)
        out = np.full((B, Hq, D), np.nan, dtype=np.float64)
        todo = heads if heads is not None else [(b, hq) for b in range(B) for hq in range(Hq)]

        def one(bh):
            b, hq = bh
            kv, vv = self.views(b, hq // gq)
            if rope_base is None:
                out[b, hq] = decode_head(kv, vv, self.n_stored, qf[b, hq], scale)
            else:
                out[b, hq] = decode_head_rope(kv, vv, self.n_stored, qf[b, hq], scale, rope_base, q_pos)

        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(one, todo))
        return out


def prefill_attention(cache: "OracleCache", q: np.ndarray, q_dtype: str, sm_scale: float = 0.0,
                      causal: bool = False, threads: int = 8) -> np.ndarray:
    """Attention of n_q queries per head over the cache (a prefill chunk, [P4]
    s.5's multi-query microbenchmark shape): fp64 outputs [B][Hq][n_q][D] for
    q [B][Hq][n_q][D].  Each row is the decode of that query over the first T
    slots, or with ``causal`` -- the chunk being the cache's last n_q slots --
    over the first T - n_q + i + 1 slots for query i."""
    L = cache.L
    B, Hq, n_q, D = q.shape
    T = cache.n_stored
    gq = Hq // L.n_kv_heads
    scale = sm_scale if sm_scale > 0 else 1.0 / math.sqrt(D)
    qf = widen(q, q_dtype)
    out = np.zeros((B, Hq, n_q, D), dtype=np.float64)

    def one(bh):
        b, hq = divmod(bh, Hq)
        kv, vv = cache.views(b, hq // gq)
        for i in range(n_q):
            Ti = T - n_q + i + 1 if causal else T
            out[b, hq, i] = decode_head(kv, vv, Ti, qf[b, hq, i], scale)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(B * Hq)))
    return out


def snapkv(K: np.ndarray, V: np.ndarray, obs_window: int, n_sink: int, budget: int,
           threads: int = 8):
    """SnapKV over K, V [B][H][S][D] fp16.

    Returns (scores fp64 [B][H][S], kept int32 [B][H][n_keep], K_out, V_out fp16),
    with the selection taken on the fp32-rounded scores.
    """
    B, H, S, D = K.shape
    n_keep = max(0, min(budget, S))
    scores = np.zeros((B, H, S), dtype=np.float64)
    kept = np.zeros((B, H, n_keep), dtype=np.int32)
    Kf = K.astype(np.float32)

    def one(bh):
        b, h = divmod(bh, H)
        scores[b, h] = snapkv_scores(Kf[b, h], obs_window)
        kept[b, h] = snapkv_select(scores[b, h].astype(np.float32), n_sink, budget)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(B * H)))
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    return scores, kept, K[bi, hi, kept], V[bi, hi, kept]


@dataclass
class SnapState:
    """Rows kept by SnapKV so far: k, v [B][H][n][D] fp16 in ascending
    position order, their absolute positions pos [B][H][n], and the position
    of the next prefill token."""
    k: np.ndarray
    v: np.ndarray
    pos: np.ndarray
    next_pos: int

    @staticmethod
    def empty(B: int, H: int, D: int) -> "SnapState":
        z = np.zeros((B, H, 0, D), dtype=np.float16)
        return SnapState(z, z.copy(), np.zeros((B, H, 0), dtype=np.int32), 0)


def snapkv_chunk(state: SnapState, k_chunk: np.ndarray, v_chunk: np.ndarray, obs_window: int,
                 n_sink: int, budget: int, q_window: np.ndarray | None = None, pool_kernel: int = 1,
                 threads: int = 8):
    """One prefill call of SnapKV over the kept rows followed by a new chunk.

    The candidates are state.k (positions state.pos) then k_chunk (positions
    state.next_pos, +1, ...).  Observation rows: the last min(w, n) candidate
    key rows, or with q_window [B][Hq][w][D] the w query rows of every query
    head of the kv-head's group.  Scores per [P2] "How it works" step 1 (fp64),
    rounded to fp32, max-pooled when pool_kernel > 1, then the sinks plus the
    top (budget - sinks) as in steps 2-3; the kept rows and positions are
    gathered in candidate order (ascending position).

    Returns (new SnapState, scores fp64 [B][H][n], kept candidate indices
    int32 [B][H][min(budget, n)]).
    """
    B, H, _, D = state.k.shape
    S_c = k_chunk.shape[2]
    K = np.concatenate([state.k, np.asarray(k_chunk, dtype=np.float16)], axis=2)
    V = np.concatenate([state.v, np.asarray(v_chunk, dtype=np.float16)], axis=2)
    new_pos = np.broadcast_to(state.next_pos + np.arange(S_c, dtype=np.int32), (B, H, S_c))
    P = np.concatenate([state.pos, new_pos], axis=2)
    n = K.shape[2]
    n_keep = min(budget, n)
    scores = np.zeros((B, H, n), dtype=np.float64)
    kept = np.zeros((B, H, n_keep), dtype=np.int32)
    Kf = K.astype(np.float32)

    def one(bh):
        b, h = divmod(bh, H)
        if q_window is None:
            rows = Kf[b, h, n - min(obs_window, n):]
        else:
            G = q_window.shape[1] // H
            rows = q_window[b, h * G:(h + 1) * G].reshape(G * q_window.shape[2], D).astype(np.float32)
        scores[b, h] = snapkv_scores_rows(rows, Kf[b, h])
        rank = scores[b, h].astype(np.float32)
        if pool_kernel > 1:
            rank = maxpool1d(rank, pool_kernel)
        kept[b, h] = snapkv_select(rank, n_sink, budget)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(B * H)))
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    new = SnapState(K[bi, hi, kept], V[bi, hi, kept], P[bi, hi, kept].astype(np.int32),
                    state.next_pos + S_c)
    return new, scores, kept

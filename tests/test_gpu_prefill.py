"""GPU parity for multi-query (prefill-chunk) attention over the packed cache
([P4] s.5: the fused-attention microbenchmark shape -- 128 queries per head,
GQA 4:1 -- where attention is a dense contraction on the matrix cores).

Row (b, hq, i) is the oracle's fp64 decode of query i over the whole cache
or, causally, over the slots up to the chunk's own row.  The kernel feeds the
matrix cores fp16 keys, values, queries and probabilities with fp32
accumulation; the bar is the attention tolerance, 2e-3 relative to each
row's largest output.
"""
import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K
import synth
from oracle.cache import OracleCache, prefill_attention

from _gpu import attn_err, layouts, say, to_dev
from test_gpu_parity import build_pair, make_case

pytestmark = pytest.mark.gpu
TOL = 2e-3


def gen_q(w, B, Hq, Hkv, n_q, seed):
    """Queries [B][Hq][n_q][D] in the workload dtype, from the window-query streams."""
    G = Hq // Hkv
    wl = synth.workload(w.name, head_dim=w.head_dim, n_kv_heads=Hkv, n_q_heads=Hq, config_id=700 + seed)
    npdt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[w.dtype]
    q = np.empty((B, Hq, n_q, w.head_dim), npdt)
    for b in range(B):
        for h in range(Hkv):
            q[b, h * G:(h + 1) * G] = synth.query_window(wl, b, h, n_q, G)
    return q


@pytest.mark.parametrize("name,n_q,causal", [
    ("affine4_g64_bf16", 37, False),     # ragged row block, two heads per block
    ("affine4_g64_bf16", 128, True),     # the microbenchmark row count, causal chunk
    ("kivi4_llama3b", 128, True),        # KIVI keys with an open residual group
    ("sym4_centered", 64, False),
    ("affine8_d64", 5, True),            # head_dim 64, GQA 2
    ("plain_f32", 200, False),           # head_dim 32, fp32 cache
    ("kivi2_llama3b", 33, True),
])
def test_prefill_attention_parity(name, n_q, causal):
    w, pl, ol, k, v, _q, bias, cfg = make_case(name)
    say("prefill attention", name, n_q, causal)
    c, o = build_pair(pl, ol, k, v, w.dtype, cfg.get("chunks"), k_bias=bias)
    Hq = cfg.get("Hq", pl.n_kv_heads * w.group)
    q = gen_q(w, pl.batch, Hq, pl.n_kv_heads, n_q, seed=n_q)
    out = K.kvq_prefill_attention(pl, c, to_dev(q, w.dtype), causal=causal)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = prefill_attention(o, q, w.dtype, causal=causal)
    err = attn_err(got, ref)
    say(f"  prefill attention error {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL, err


def test_prefill_single_query_is_the_decode():
    w, pl, ol, k, v, _q, bias, cfg = make_case("affine4_g64_bf16")
    c, o = build_pair(pl, ol, k, v, w.dtype, cfg.get("chunks"))
    q = gen_q(w, pl.batch, 32, 8, 1, seed=3)
    say("prefill single query")
    a = K.kvq_prefill_attention(pl, c, to_dev(q, w.dtype)).cpu().numpy()[:, :, 0]
    d = K.kvq_decode_attention(pl, c, to_dev(np.ascontiguousarray(q[:, :, 0]), w.dtype)).cpu().numpy()
    ref = o.decode(np.ascontiguousarray(q[:, :, 0]), w.dtype)
    assert attn_err(a, ref) <= TOL and attn_err(d, ref) <= TOL


def test_prefill_microbenchmark_shape_sampled():
    """B = 1, 32 query / 8 kv-heads x 128, T = 32768 (4-bit affine g64 K and V,
    bf16), 128 causal queries: sampled rows against the oracle."""
    w = synth.workload("affine4_g64")
    B, T, n_q = 1, 32768, 128
    k, v, _ = synth.full(w, batch=B, threads=16)
    pl, ol = layouts(batch=B, n_kv_heads=8, head_dim=128, capacity=T, k_kind="tok_affine", k_bits=4,
                     k_group=64, v_kind="tok_affine", v_bits=4, v_group=64, in_dtype="bf16")
    say("prefill attention full size", B, T, n_q)
    c, o = build_pair(pl, ol, k, v, "bf16")
    q = gen_q(w, B, 32, 8, n_q, seed=9)
    out = K.kvq_prefill_attention(pl, c, to_dev(q, "bf16"), causal=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    from oracle import decode_head, widen
    qf = widen(q, "bf16")
    for hq, i in [(0, 0), (5, 17), (13, 64), (22, 100), (31, 127)]:
        kv, vv = o.views(0, hq // 4)
        ref = decode_head(kv, vv, T - n_q + i + 1, qf[0, hq, i], 1.0 / np.sqrt(128))
        err = float(np.abs(got[0, hq, i] - ref).max() / np.abs(ref).max())
        say(f"  row ({hq}, {i}) error {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("D,dtype,k_bits,T", [
    (128, "bf16", 4, 8192),      # 64 splits: 32 past the combine's prefetch (two split phases)
    (64, "bf16", 8, 12000),      # 93 splits, four phases
    (32, "f32", 4, 20000),       # 156 splits, eight phases, fp32 queries
])
def test_prefill_many_splits(D, dtype, k_bits, T):
    """One kv-head and four query rows over a long cache: the split plan then
    takes many short splits, and the fp16 split combine reads the splits past
    its prefetch in its tail loop.  Every row against the oracle."""
    B, H, G, n_q = 1, 1, 2, 2
    w = synth.workload("affine4_g64", head_dim=D, seq_len=T, batch=B, n_kv_heads=H, n_q_heads=H * G,
                       dtype=dtype)
    k, v, _ = synth.full(w, threads=16)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind="tok_affine", k_bits=k_bits,
                     k_group=32, v_kind="tok_affine", v_bits=k_bits, v_group=32, in_dtype=dtype)
    say("prefill many splits", D, dtype, k_bits, T)
    c, o = build_pair(pl, ol, k, v, dtype)
    q = gen_q(w, B, H * G, H, n_q, seed=T)
    out = K.kvq_prefill_attention(pl, c, to_dev(q, dtype), causal=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = prefill_attention(o, q, dtype, causal=True)
    err = attn_err(got, ref)
    say(f"  error {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL, err


@pytest.mark.parametrize("kg,vg,dtype,stress", [
    (64, 32, "bf16", "outliers"), (64, 64, "bf16", "outliers"), (64, 128, "bf16", "offset"),
    (128, 32, "bf16", "outliers"), (128, 64, "f16", "outliers"), (128, 128, "bf16", "offset"),
    (64, 64, "f16", "offset"), (64, 32, "f16", "outliers"),
])
def test_prefill_factored_key_groups(kg, vg, dtype, stress):
    """4-bit per-token affine keys in groups of 64 or 128 channels at head_dim
    128 take the factored scores (codes as exact operands, per-group scales
    applied to the sums, zero points as one more product).  Keys with x10
    outlier channels, or with a large per-channel offset (big zero points whose
    term cancels most of the code term), against the oracle: causal rows over
    a ragged cache, two batches x two kv-heads x four query heads."""
    B, H, G, T, n_q = 2, 2, 4, 1500, 40
    over = dict(n_outlier_channels=6, outlier_scale=10.0) if stress == "outliers" else dict(k_bias_std=8.0)
    w = synth.workload("affine4_g64", head_dim=128, seq_len=T, batch=B, n_kv_heads=H, n_q_heads=H * G,
                       dtype=dtype, **over)
    k, v, _ = synth.full(w, threads=8)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind="tok_affine", k_bits=4,
                     k_group=kg, v_kind="tok_affine", v_bits=4, v_group=vg, in_dtype=dtype)
    say("prefill factored scores", kg, vg, dtype, stress)
    c, o = build_pair(pl, ol, k, v, dtype)
    rng = np.random.default_rng([0, 701, kg, vg])
    q = synth.cast(rng.standard_normal((B, H * G, n_q, 128), dtype=np.float32), dtype)
    out = K.kvq_prefill_attention(pl, c, to_dev(q, dtype), causal=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = prefill_attention(o, q, dtype, causal=True)
    err = attn_err(got, ref)
    say(f"  error {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL, err


@pytest.mark.parametrize("T,kg,dtype", [(1, 64, "bf16"), (63, 128, "f16"), (65, 64, "f16"), (200, 128, "bf16")])
def test_prefill_factored_edges(T, kg, dtype):
    """Factored scores on short caches (one slot, one partial tile, a tile
    plus one slot) with some all-zero query rows (their logits are all zero:
    the output is the mean of the visible values), causal and not."""
    B, H, G, n_q = 1, 2, 4, 1 if T == 1 else min(T, 24)
    w = synth.workload("affine4_g64", head_dim=128, seq_len=T, batch=B, n_kv_heads=H, n_q_heads=H * G,
                       dtype=dtype, n_outlier_channels=6, outlier_scale=10.0)
    k, v, _ = synth.full(w, threads=8)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind="tok_affine", k_bits=4,
                     k_group=kg, v_kind="tok_affine", v_bits=4, v_group=64, in_dtype=dtype)
    say("prefill factored edges", T, kg, dtype)
    c, o = build_pair(pl, ol, k, v, dtype)
    rng = np.random.default_rng([0, 702, T, kg])
    qf = rng.standard_normal((B, H * G, n_q, 128), dtype=np.float32)
    qf[:, 1] = 0.0                        # a whole query head of zero rows
    qf[:, 4:, n_q // 2] = 0.0             # and one row in each later head
    q = synth.cast(qf, dtype)
    for causal in (False, True):
        out = K.kvq_prefill_attention(pl, c, to_dev(q, dtype), causal=causal)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = prefill_attention(o, q, dtype, causal=causal)
        err = attn_err(got, ref)
        say(f"  causal={causal} error {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= TOL, err


@pytest.mark.parametrize("kg,dtype", [(64, "bf16"), (128, "f16")])
def test_prefill_reference_moves_inside_splits(kg, dtype):
    """Key norms that grow along the cache in steps (x1 up to x9, plus single
    spike tokens at x14): each row's largest logit keeps rising from tile to
    tile inside a split, so the softmax reference point has to move (and the
    output accumulators be rescaled) after the first tile, also on tiles that
    need no mask.  Against the oracle, causal and not."""
    B, H, G, T, n_q = 1, 2, 4, 3000, 24
    rng = np.random.default_rng([0, 703, kg])
    k = rng.standard_normal((B, H, T, 128), dtype=np.float32)
    v = rng.standard_normal((B, H, T, 128), dtype=np.float32)
    k *= (1.0 + np.floor(np.arange(T) / 375.0))[None, None, :, None].astype(np.float32)
    spikes = rng.choice(T, size=12, replace=False)
    k[:, :, spikes] *= 14.0 / (1.0 + np.floor(spikes / 375.0))[None, None, :, None]
    k, v = synth.cast(k, dtype), synth.cast(v, dtype)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind="tok_affine", k_bits=4,
                     k_group=kg, v_kind="tok_affine", v_bits=4, v_group=64, in_dtype=dtype)
    say("prefill reference moves", kg, dtype)
    c, o = build_pair(pl, ol, k, v, dtype)
    q = synth.cast(rng.standard_normal((B, H * G, n_q, 128), dtype=np.float32), dtype)
    for causal in (False, True):
        out = K.kvq_prefill_attention(pl, c, to_dev(q, dtype), causal=causal)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = prefill_attention(o, q, dtype, causal=causal)
        err = attn_err(got, ref)
        say(f"  causal={causal} error {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= TOL, err

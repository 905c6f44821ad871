"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Codes, scales, zeros, positions, table rows and residual keys must match
bit-for-bit; attention outputs within 2e-3 of the fp64 oracle, measured as
max |o - o_ref| / max_d |o_ref| per (batch, query-head) row over the same
dequantized cache.  Sizes span several tiles and splits with ragged tails.
"""
import dataclasses

import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K
import oracle
import synth
from oracle.cache import OracleCache

from _gpu import (DEV, assert_same_state, attn_err, layouts, say, to_dev)

pytestmark = pytest.mark.gpu
TOL = 2e-3


def gen(w, B, H, T, Hq=None):
    """Seeded K, V [B][H][T][D] and q [B][Hq][D] in the workload dtype."""
    Hq = Hq or w.n_q_heads
    D = w.head_dim
    np_dt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[w.dtype]
    k = np.empty((B, H, T, D), np_dt)
    v = np.empty((B, H, T, D), np_dt)
    q = np.empty((B, Hq, D), np_dt)
    g = Hq // H
    ww = dataclasses.replace(w, n_q_heads=Hq, n_kv_heads=H)
    for b in range(B):
        for h in range(H):
            kk, vv, qq = synth.slice_cast(ww, b, h, T)
            k[b, h], v[b, h], q[b, h * g:(h + 1) * g] = kk, vv, qq
    return k, v, q


def build_pair(pl, ol, k, v, dtype, chunks=None, k_bias=None):
    """Append the same chunks to a product and an oracle cache."""
    c = K.Cache(pl, k_bias=None if k_bias is None else torch.from_numpy(k_bias))
    o = OracleCache(ol, k_bias=k_bias)
    T = k.shape[2]
    chunks = chunks or [(0, T)]
    for s, e in chunks:
        kd = to_dev(np.ascontiguousarray(k[:, :, s:e]), dtype)
        vd = to_dev(np.ascontiguousarray(v[:, :, s:e]), dtype)
        K.kvq_quantize_append(pl, c, kd, vd)
        o.append(k[:, :, s:e], v[:, :, s:e])
    torch.cuda.synchronize()
    return c, o


def check_decode(pl, c, o, q, qdt, sm_scale=0.0, tol=TOL):
    out = K.kvq_decode_attention(pl, c, to_dev(q, qdt), sm_scale=sm_scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = o.decode(q, qdt, sm_scale)
    err = attn_err(got, ref)
    say(f"  attention error {err:.3e} (tolerance {tol:.0e})")
    assert np.all(np.isfinite(got))
    assert err <= tol, err
    return got, err


# ---------------------------------------------------------------- per format

CASES = {
    # mlx-style 4-bit affine g64 K and V, bf16 (headline format), 2 x 8 heads
    "affine4_g64_bf16": dict(w="affine4_g64", B=2, H=8, T=1500,
                             lay=dict(k_kind="tok_affine", k_bits=4, k_group=64, v_kind="tok_affine",
                                      v_bits=4, v_group=64, in_dtype="bf16"),
                             chunks=[(0, 1), (1, 700), (700, 1500)]),
    # KIVI int4, per-channel K over 32-token groups + residual, outlier channels
    "kivi4_llama3b": dict(w="llama3b_kivi_int4", B=1, H=8, T=1000,
                          lay=dict(k_kind="kivi_ch", k_bits=4, k_group=32, v_kind="tok_affine",
                                   v_bits=4, v_group=32, in_dtype="f16"),
                          chunks=[(0, 1), (1, 300), (300, 1000)]),
    # KIVI int8, tinygpt shape, fp32
    "kivi8_tiny": dict(w="kivi_int8_tiny", B=1, H=8, T=450,
                       lay=dict(k_kind="kivi_ch", k_bits=8, k_group=32, v_kind="tok_affine",
                                v_bits=8, v_group=32, in_dtype="f32"),
                       chunks=[(0, 17), (17, 450)]),
    # symmetric 4-bit K with mean-centering, int8 per-token V
    "sym4_centered": dict(w="q4_0_centered", B=2, H=8, T=777,
                          lay=dict(k_kind="tok_sym4", k_bits=4, k_group=32, v_kind="tok_affine",
                                   v_bits=8, v_group=128, in_dtype="f16"),
                          center=True, chunks=[(0, 400), (400, 777)]),
    # 8-bit affine K g32 with 4-bit V g32 at head_dim 64, GQA 2
    "affine8_d64": dict(w="affine4_g64", B=3, H=2, T=600, Hq=4, D=64,
                        lay=dict(k_kind="tok_affine", k_bits=8, k_group=32, v_kind="tok_affine",
                                 v_bits=4, v_group=32, in_dtype="bf16")),
    # KIVI int4 with 8 query heads per kv-head (both head slots of the scores)
    "kivi4_gqa8": dict(w="llama3b_kivi_int4", B=1, H=2, T=700, Hq=16,
                       lay=dict(k_kind="kivi_ch", k_bits=4, k_group=32, v_kind="tok_affine",
                                v_bits=4, v_group=32, in_dtype="f16"),
                       chunks=[(0, 100), (100, 700)]),
    # 4-bit affine K and V at head_dim 64 with 6 query heads per kv-head
    "affine4_d64_gqa6": dict(w="affine4_g64", B=2, H=2, T=333, Hq=12, D=64,
                             lay=dict(k_kind="tok_affine", k_bits=4, k_group=64, v_kind="tok_affine",
                                      v_bits=4, v_group=32, in_dtype="bf16")),
    # KIVI-2bit: per-channel 2-bit K over 32-token groups, 2-bit V groups of 32
    "kivi2_llama3b": dict(w="llama3b_kivi_int4", B=1, H=8, T=1000,
                          lay=dict(k_kind="kivi_ch", k_bits=2, k_group=32, v_kind="tok_affine",
                                   v_bits=2, v_group=32, in_dtype="f16"),
                          chunks=[(0, 1), (1, 300), (300, 1000)]),
    # 2-bit per-token K and V at head_dim 32 (rows of 8 bytes), fp32 inputs
    "affine2_d32": dict(w="kivi_int8_tiny", B=2, H=8, T=333,
                        lay=dict(k_kind="tok_affine", k_bits=2, k_group=32, v_kind="tok_affine",
                                 v_bits=2, v_group=32, in_dtype="f32"),
                        chunks=[(0, 100), (100, 333)]),
    # full-precision cache
    "plain_f32": dict(w="kivi_int8_tiny", B=1, H=8, T=300,
                      lay=dict(k_kind="plain", k_bits=4, k_group=32, v_kind="plain", v_bits=4,
                               v_group=32, in_dtype="f32")),
}


def make_case(name):
    cfg = CASES[name]
    w = synth.workload(cfg["w"])
    if "D" in cfg:
        w = synth.workload(cfg["w"], head_dim=cfg["D"])
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    Hq = cfg.get("Hq", H * w.group)
    k, v, q = gen(w, B, H, T, Hq)
    bias = None
    flags = 0
    if cfg.get("center"):
        bias = np.stack([synth.head_params(w, h)[0] for h in range(H)]).astype(np.float32)
        flags = K.KVQ_CENTER_K
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=w.head_dim, capacity=T + 37, flags=flags,
                     **cfg["lay"])
    return w, pl, ol, k, v, q, bias, cfg


@pytest.mark.parametrize("name", sorted(CASES))
def test_quantize_and_decode_parity(name):
    w, pl, ol, k, v, q, bias, cfg = make_case(name)
    say("quantize+decode", name, pl)
    c, o = build_pair(pl, ol, k, v, w.dtype, cfg.get("chunks"), k_bias=bias)
    assert_same_state(c, o)
    got, err = check_decode(pl, c, o, q, w.dtype)
    # deterministic: a second run gives the same bytes
    again = K.kvq_decode_attention(pl, c, to_dev(q, w.dtype)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    # explicit softmax scale
    check_decode(pl, c, o, q, w.dtype, sm_scale=0.05)


def test_decode_query_dtypes_and_single_slot():
    w, pl, ol, k, v, q, bias, cfg = make_case("affine4_g64_bf16")
    say("decode q dtypes / T=1")
    c, o = build_pair(pl, ol, k[:, :, :1], v[:, :, :1], w.dtype)
    out = K.kvq_decode_attention(pl, c, to_dev(q, w.dtype)).cpu().numpy()
    ref = o.decode(q, w.dtype)
    assert attn_err(out, ref) <= 1e-6      # one slot: the value row itself
    c, o = build_pair(pl, ol, k, v, w.dtype)
    qf = synth.widen(q, "bf16")
    for qdt in ("f32", "f16"):
        qq = synth.cast(qf, qdt)
        check_decode(pl, c, o, qq, qdt)


@pytest.mark.parametrize("kg,vg", [(kg, vg) for kg in (32, 64, 128) for vg in (32, 64, 128)])
def test_fast_decode_group_combinations(kg, vg):
    """4-bit affine K and V at head_dim 128 with 4 query heads per kv-head, for
    every K / V group size pair: a ragged length split over T (batch 1 x 2
    kv-heads), so splits hold odd and even tile counts and a partial tile."""
    w = synth.workload("affine4_g64")
    B, H, T = 1, 2, 2224
    k, v, q = gen(w, B, H, T, Hq=8)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind="tok_affine", k_bits=4,
                     k_group=kg, v_kind="tok_affine", v_bits=4, v_group=vg, in_dtype="bf16")
    say("fast decode groups", kg, vg)
    c, o = build_pair(pl, ol, k, v, "bf16", chunks=[(0, 1000), (1000, T)])
    assert_same_state(c, o)
    check_decode(pl, c, o, q, "bf16")
    check_decode(pl, c, o, synth.cast(synth.widen(q, "bf16"), "f16"), "f16")


@pytest.mark.parametrize("k_kind,kg,vb,vg", [
    ("tok_sym4", 32, 4, 64), ("tok_sym4", 32, 8, 32), ("tok_sym4", 32, 8, 128),
    ("tok_affine", 64, 8, 64), ("tok_affine", 128, 8, 128), ("tok_affine", 32, 8, 64),
])
def test_fast_decode_k_formats_and_8bit_v(k_kind, kg, vb, vg):
    """Symmetric (Q4_0-style) or affine 4-bit K with 4- or 8-bit per-token V at
    head_dim 128, 4 query heads per kv-head: ragged length split over T."""
    w = synth.workload("q4_0_centered")
    B, H, T = 1, 2, 2000
    k, v, q = gen(w, B, H, T, Hq=8)
    bias = np.stack([synth.head_params(w, h)[0] for h in range(H)]).astype(np.float32)
    flags = K.KVQ_CENTER_K if k_kind == "tok_sym4" else 0
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind=k_kind, k_bits=4, k_group=kg,
                     v_kind="tok_affine", v_bits=vb, v_group=vg, in_dtype="f16", flags=flags)
    say("fast decode formats", k_kind, kg, vb, vg)
    c, o = build_pair(pl, ol, k, v, "f16", chunks=[(0, 1333), (1333, T)],
                      k_bias=bias if flags else None)
    assert_same_state(c, o)
    check_decode(pl, c, o, q, "f16")
    check_decode(pl, c, o, synth.cast(synth.widen(q, "f16"), "bf16"), "bf16")


@pytest.mark.parametrize("B,H", [(8, 8), (9, 7)])
def test_8bit_value_decode_at_the_split_plan_boundary(B, H):
    """Q4_0-style centered keys with 8-bit values: from 64 (batch, kv-head)
    units the split plan aims at 256 workgroups instead of 512 (B=8 x 8
    kv-heads: 4 splits of a ragged cache; 9 x 7 = 63 units: 6).  Every row
    against the oracle."""
    w = synth.workload("q4_0_centered")
    T = 1500
    k, v, q = gen(w, B, H, T, Hq=4 * H)
    bias = np.stack([synth.head_params(w, h)[0] for h in range(H)]).astype(np.float32)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind="tok_sym4", k_bits=4,
                     k_group=32, v_kind="tok_affine", v_bits=8, v_group=32, in_dtype="f16",
                     flags=K.KVQ_CENTER_K)
    say("8-bit value decode, split plan boundary", B, H)
    c, o = build_pair(pl, ol, k, v, "f16", k_bias=bias)
    check_decode(pl, c, o, q, "f16")


@pytest.mark.parametrize("k_kind,kg,vb,vg,dt", [
    ("tok_affine", 32, 4, 128, "bf16"), ("tok_affine", 64, 4, 64, "f16"), ("tok_sym4", 32, 8, 64, "f16"),
])
def test_matrix_core_decode_extremes(k_kind, kg, vb, vg, dt):
    """Per-token 4-bit K with 4 query heads per kv-head (the matrix-core
    decode) on inputs at the edges of its exactness argument: keys with x100
    outlier channels and a constant block, values with constant rows and a
    channel at +-4, query heads that span 2^-24 .. 2^4, are zero, or hold one
    large element among tiny ones, and a kv-head whose whole query group is
    zero.  T = 97: three full tiles and a partial one."""
    rng = np.random.default_rng(1234)
    B, H, T, D, Hq = 1, 2, 97, 128, 8
    k = rng.standard_normal((B, H, T, D)).astype(np.float32)
    k[..., 5] *= 100.0
    k[..., 70] *= 100.0
    k[..., 96:] = 0.75
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    v[:, :, ::7, :] = 3.0
    v[..., 0] = np.where(np.arange(T) % 2 == 0, -4.0, 4.0)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    q[0, 1] = np.ldexp(np.where(rng.random(D) < 0.5, -1.0, 1.0), rng.integers(-24, 5, D))
    q[0, 2] = 0.0
    q[0, 3] *= 1e-6
    q[0, 3, 17] = 8.0
    q[0, 4:8] = 0.0
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind=k_kind, k_bits=4, k_group=kg,
                     v_kind="tok_affine", v_bits=vb, v_group=vg, in_dtype=dt)
    say("matrix-core decode extremes", k_kind, kg, vb, vg, dt)
    c, o = build_pair(pl, ol, synth.cast(k, dt), synth.cast(v, dt), dt)
    assert_same_state(c, o)
    for qdt in ("bf16", "f16"):
        check_decode(pl, c, o, synth.cast(q, qdt), qdt)


def test_empty_cache_decodes_to_zeros():
    pl, ol = layouts(batch=2, n_kv_heads=2, head_dim=64, capacity=10, in_dtype="f16",
                     k_group=64, v_group=64)
    c = K.Cache(pl)
    q = torch.randn(2, 4, 64, device=DEV, dtype=torch.float16)
    out = torch.full((2, 4, 64), 7.0, device=DEV)
    K.kvq_decode_attention(pl, c, q, out=out)
    assert torch.count_nonzero(out).item() == 0


def test_constant_channels_use_subnormal_eps_scale():
    """[P1] bug class 1: constant slices quantize with scale fp16(1e-5), a subnormal."""
    pl, ol = layouts(batch=1, n_kv_heads=2, head_dim=32, capacity=64, k_kind="kivi_ch", k_bits=8,
                     k_group=32, v_kind="tok_affine", v_bits=4, v_group=32, in_dtype="f16")
    k = np.full((1, 2, 40, 32), 0.1, np.float16)
    v = np.full((1, 2, 40, 32), -3.5, np.float16)
    k[0, 1, :, 5] = np.float16(6.1e-5)
    say("constant channels")
    c, o = build_pair(pl, ol, k, v, "f16")
    assert_same_state(c, o)
    table = c.k_meta.cpu().numpy().view(np.uint16)
    assert 168 in table        # fp16 bit pattern of the eps scale


def test_centering_disabled_is_a_byte_noop():
    """[P3] regression safety: centering off, or an all-zero bias, leaves every byte unchanged."""
    w = synth.workload("q4_0_centered")
    k, v, q = gen(w, 2, 8, 300)
    pl0, ol0 = layouts(batch=2, n_kv_heads=8, head_dim=128, capacity=300, k_kind="tok_sym4",
                       k_bits=4, k_group=32, v_kind="tok_affine", v_bits=8, v_group=128, in_dtype="f16")
    plz, _ = layouts(batch=2, n_kv_heads=8, head_dim=128, capacity=300, k_kind="tok_sym4",
                     k_bits=4, k_group=32, v_kind="tok_affine", v_bits=8, v_group=128,
                     in_dtype="f16", flags=K.KVQ_CENTER_K)
    say("centering no-op")
    c0, o0 = build_pair(pl0, ol0, k, v, "f16")
    cz = K.Cache(plz, k_bias=torch.zeros(8, 128))
    K.kvq_quantize_append(plz, cz, to_dev(k, "f16"), to_dev(v, "f16"))
    torch.cuda.synchronize()
    for name in ("k_codes", "k_meta", "v_codes", "v_meta", "pos"):
        assert torch.equal(getattr(c0, name), getattr(cz, name)), name
    assert_same_state(c0, o0)


def test_shift_invariance_on_gpu():
    """[P3] "Why this is safe": a full-precision fp32 K cache centered through the
    test seam attends exactly like the uncentered one (to fp32 rounding)."""
    rng = np.random.default_rng(77)
    B, H, T, D = 2, 4, 900, 128
    k = (rng.standard_normal((B, H, T, D)) + rng.standard_normal((1, H, 1, D)) * 1.5).astype(np.float32)
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    q = rng.standard_normal((B, 4 * H, D)).astype(np.float32)
    kbar = (rng.standard_normal((H, D)) * 1.5).astype(np.float32)
    base = dict(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind="plain", k_bits=4,
                k_group=32, v_kind="plain", v_bits=4, v_group=32, in_dtype="f32")
    pl, ol = layouts(**base)
    plc, _ = layouts(flags=K.KVQ_CENTER_K | K.KVQ_TEST_CENTER_ANY, **base)
    say("shift invariance")
    c, o = build_pair(pl, ol, k, v, "f32")
    cc = K.Cache(plc, k_bias=torch.from_numpy(kbar))
    K.kvq_quantize_append(plc, cc, to_dev(k, "f32"), to_dev(v, "f32"))
    a = K.kvq_decode_attention(pl, c, to_dev(q, "f32")).cpu().numpy().astype(np.float64)
    b = K.kvq_decode_attention(plc, cc, to_dev(q, "f32")).cpu().numpy().astype(np.float64)
    nmse = np.sum((a - b) ** 2) / np.sum(a ** 2)
    assert nmse < 1e-9, nmse
    assert attn_err(b, a) < 1e-4
    assert attn_err(a, o.decode(q, "f32")) <= TOL


def test_append_past_capacity_raises_and_keeps_state():
    pl, ol = layouts(batch=1, n_kv_heads=2, head_dim=64, capacity=50, in_dtype="f16",
                     k_group=64, v_group=64)
    c = K.Cache(pl)
    x = torch.randn(1, 2, 40, 64, device=DEV, dtype=torch.float16)
    K.kvq_quantize_append(pl, c, x, x)
    with pytest.raises(K.KvqError) as e:
        K.kvq_quantize_append(pl, c, x, x)
    assert e.value.status == K.KVQ_ERR_CAPACITY
    assert c.n_stored == 40


# ---------------------------------------------------------------- eviction

def stream_pair(pl, ol, k, v, dtype, sink, window, evict_every=1):
    """Append token by token, evicting when the cap is exceeded; product caches ping-pong."""
    cur, spare = K.Cache(pl), K.Cache(pl)
    o = OracleCache(ol)
    T = k.shape[2]
    for t in range(T):
        K.kvq_quantize_append(pl, cur, to_dev(np.ascontiguousarray(k[:, :, t:t + 1]), dtype),
                              to_dev(np.ascontiguousarray(v[:, :, t:t + 1]), dtype))
        o.append(k[:, :, t:t + 1], v[:, :, t:t + 1])
        if (t + 1) % evict_every == 0:
            st = K.kvq_evict_streaming(pl, cur, spare, sink, window)
            e = o.evict(sink, window)
            assert (st == K.KVQ_NOOP) == (e is None)
            if st == K.KVQ_OK:
                cur, spare = spare, cur
                o = e
    torch.cuda.synchronize()
    return cur, o


def test_streaming_kivi_int8_tinygpt_500_positions():
    """[P1] smoke-test shape: sink 4 + window 256 over 500 positions; KIVI int8
    keys, per-channel tables compacted; state and decode match the oracle."""
    w = synth.workload("kivi_int8_tiny")
    k, v, q = gen(w, 1, 8, 500)
    pl, ol = layouts(batch=1, n_kv_heads=8, head_dim=32, capacity=261, k_kind="kivi_ch", k_bits=8,
                     k_group=32, v_kind="tok_affine", v_bits=8, v_group=32, in_dtype="f32")
    say("stream kivi int8 500")
    c, o = stream_pair(pl, ol, k, v, "f32", 4, 256)
    assert c.n_stored == 260 and c.next_pos == 500
    assert_same_state(c, o)
    assert np.array_equal(c.pos.cpu().numpy().view(np.int32)[:260], np.r_[0:4, 244:500])
    check_decode(pl, c, o, q, "f32")


@pytest.mark.parametrize("name", ["affine4_g64_bf16", "sym4_centered", "kivi4_llama3b", "plain_f32",
                                  "kivi2_llama3b", "affine2_d32"])
def test_batch_evict_parity(name):
    w, pl, ol, k, v, q, bias, cfg = make_case(name)
    say("batch evict", name)
    c, o = build_pair(pl, ol, k, v, w.dtype, k_bias=bias)
    dst = K.Cache(pl, k_bias=None if bias is None else torch.from_numpy(bias))
    T = k.shape[2]
    sink, window = 5, 256 + 7
    assert K.kvq_evict_streaming(pl, c, dst, sink, window) == K.KVQ_OK
    e = o.evict(sink, window)
    torch.cuda.synchronize()
    assert_same_state(dst, e)
    check_decode(pl, dst, e, q, w.dtype)
    # idempotent: nothing more to drop
    assert K.kvq_evict_streaming(pl, dst, c, sink, window) == K.KVQ_NOOP
    # append after eviction continues positions and groups
    k2, v2, _ = gen(w, pl.batch, pl.n_kv_heads, 45)
    K.kvq_quantize_append(pl, dst, to_dev(k2, w.dtype), to_dev(v2, w.dtype))
    e.append(k2, v2)
    torch.cuda.synchronize()
    assert_same_state(dst, e)
    check_decode(pl, dst, e, q, w.dtype)


def test_periodic_eviction_and_batch_eviction_kivi4():
    w = synth.workload("llama3b_kivi_int4")
    k, v, q = gen(w, 1, 8, 200)
    pl, ol = layouts(batch=1, n_kv_heads=8, head_dim=128, capacity=200, k_kind="kivi_ch", k_bits=4,
                     k_group=32, v_kind="tok_affine", v_bits=4, v_group=32, in_dtype="f16")
    say("stream vs batch kivi4")
    cs, os_ = stream_pair(pl, ol, k, v, "f16", 3, 64, evict_every=7)
    cb, ob = build_pair(pl, ol, k, v, "f16")
    dst = K.Cache(pl)
    assert K.kvq_evict_streaming(pl, cb, dst, 3, 64) == K.KVQ_OK
    torch.cuda.synchronize()
    # streaming state: slots [0,3) + last window after the final eviction point
    assert_same_state(cs, os_)
    assert_same_state(dst, ob.evict(3, 64))


@pytest.mark.parametrize("G,vb,vg,qdt", [(3, 4, 32, "f16"), (1, 8, 128, "bf16"), (4, 4, 64, "f16"),
                                          (2, 4, 128, "bf16")])
def test_kivi_fast_decode(G, vb, vg, qdt):
    """KIVI 4-bit keys at head_dim 128 with 1-4 query heads per kv-head (the
    fast decode's KIVI path): a ragged cache whose last group is still open,
    then the same cache after StreamingLLM compaction (sink 5, window 700),
    whose tiles mix table rows and read some rows per lane."""
    w = synth.workload("llama3b_kivi_int4")
    B, H, T = 1, 2, 2221
    k, v, q = gen(w, B, H, T, H * G)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind="kivi_ch", k_bits=4, k_group=32,
                     v_kind="tok_affine", v_bits=vb, v_group=vg, in_dtype="f16")
    say("kivi fast decode", G, vb, vg, qdt)
    c, o = build_pair(pl, ol, k, v, "f16", chunks=[(0, 1000), (1000, T)])
    qq = q if qdt == "f16" else synth.cast(synth.widen(q, "f16"), "bf16")
    check_decode(pl, c, o, qq, qdt)
    dst = K.Cache(pl)
    assert K.kvq_evict_streaming(pl, c, dst, 5, 700) == K.KVQ_OK
    torch.cuda.synchronize()
    check_decode(pl, dst, o.evict(5, 700), qq, qdt)


def test_quantize_codes_on_rounding_boundaries():
    """Quotients exactly on, and one ulp either side of, half-integers (where a
    reciprocal-based quotient could round differently): codes stay bit-exact."""
    rng = np.random.default_rng(99)
    B, H, T, D = 1, 2, 64, 64
    # groups of 32 with min 0 and max 15/8 -> scale 1/8, zero 0 (4-bit); interior
    # values (k + 0.5)/8 nudged by -1, 0, +1 ulp
    k = rng.integers(0, 15, size=(B, H, T, D)).astype(np.float32)
    x = (k + 0.5) / 8
    nudge = rng.integers(-1, 2, size=x.shape)
    x = np.where(nudge < 0, np.nextafter(x, -np.inf), np.where(nudge > 0, np.nextafter(x, np.inf), x))
    x = x.astype(np.float32)
    x[..., 0::32] = 0.0
    x[..., 1::32] = 15 / 8
    v = x.copy()
    for k_kind, k_bits, k_group in (("tok_affine", 4, 32), ("tok_affine", 8, 32), ("tok_sym4", 4, 32),
                                    ("kivi_ch", 4, 32)):
        pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind=k_kind, k_bits=k_bits,
                         k_group=k_group, v_kind="tok_affine", v_bits=4, v_group=32, in_dtype="f32")
        say("rounding boundaries", k_kind, k_bits)
        c, o = build_pair(pl, ol, x, v, "f32")
        assert_same_state(c, o)


@pytest.mark.parametrize("offset", [48.0, 1024.0])
def test_quantize_codes_with_offset_zero_points(offset):
    """4-bit codes of groups whose zero point sits `offset` away from 0: 48
    (|z| / s = 384, the fused-quotient path) and 1024 (|z| / s = 8192, where
    every element goes to the exact quotient).  Quotients on, and one ulp
    either side of, half-integers stay bit-exact."""
    rng = np.random.default_rng(int(offset))
    B, H, T, D = 1, 2, 64, 128
    k = rng.integers(0, 15, size=(B, H, T, D)).astype(np.float32)
    x = (np.float32(offset) + (k + 0.5) / 8).astype(np.float32)
    nudge = rng.integers(-1, 2, size=x.shape)
    x = np.where(nudge < 0, np.nextafter(x, -np.inf), np.where(nudge > 0, np.nextafter(x, np.inf), x))
    x = x.astype(np.float32)
    x[..., 0::64] = offset                  # group min: zero = offset exactly
    x[..., 1::64] = offset + 15 / 8         # group max: scale = 1/8
    # odd tokens: the offset only on some groups, so fused and exact lanes share waves
    x[:, :, 1::2, 64:] -= np.float32(offset)
    v = x.copy()
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind="tok_affine", k_bits=4,
                     k_group=64, v_kind="tok_affine", v_bits=4, v_group=32, in_dtype="f32")
    say("offset zero points", offset)
    c, o = build_pair(pl, ol, x, v, "f32")
    assert_same_state(c, o)


def test_quantize_codes_random_offsets_bf16():
    """Random per-group offsets up to +-2000 and spreads from 1e-3 to 1 (bf16
    inputs): lanes of one wave take both quotient forms; codes bit-exact."""
    rng = np.random.default_rng(7)
    B, H, T, D = 2, 2, 96, 128
    off = rng.uniform(-2000, 2000, size=(B, H, T, D // 64, 1))
    spread = 10.0 ** rng.uniform(-3, 0, size=(B, H, T, D // 64, 1))
    x = (off + spread * rng.standard_normal((B, H, T, D // 64, 64))).reshape(B, H, T, D).astype(np.float32)
    x[:, :, ::3] = rng.standard_normal((B, H, (T + 2) // 3, D)).astype(np.float32)
    xb = synth.cast(x, "bf16")
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind="tok_affine", k_bits=4,
                     k_group=64, v_kind="tok_affine", v_bits=4, v_group=64, in_dtype="bf16")
    say("random offsets bf16")
    c, o = build_pair(pl, ol, xb, xb, "bf16")
    assert_same_state(c, o)


# ------------------------------------------------ RoPE on read (re-positioning)

def check_decode_rope(pl, c, o, q, qdt, table, q_pos, tol=TOL):
    out = K.kvq_decode_attention_rope(pl, c, to_dev(q, qdt), table, q_pos)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = o.decode(q, qdt, rope_base=10000.0, q_pos=q_pos)
    err = attn_err(got, ref)
    say(f"  rope attention error {err:.3e} (q_pos {q_pos})")
    assert np.all(np.isfinite(got)) and err <= tol, err


def test_rope_table_matches_oracle_rotation():
    """(cos, sin) of pos * base^(-2j/D) in fp32: each entry is the oracle's
    rotation of the unit vector e_j at that position, to fp32 rounding."""
    D, n = 128, 5000
    say("rope table", D, n)
    t = K.kvq_rope_table(n, D).cpu().numpy()
    for p in (0, 1, 2, 77, 1023, 4999):
        for j in (0, 1, 5, 31, 63):
            e = np.zeros(D)
            e[j] = 1.0
            r = oracle.rope_rotate(e, 10000.0, p)
            assert abs(t[p, j, 0] - r[j]) <= 1.2e-7 and abs(t[p, j, 1] - r[j + D // 2]) <= 1.2e-7, (p, j)


@pytest.mark.parametrize("name", ["affine4_g64_bf16", "kivi4_llama3b", "sym4_centered", "affine8_d64", "plain_f32"])
def test_decode_rope_on_read(name):
    """Keys stored before the rotation, rotated at their slot index on read,
    the query at the newest slot ([P1] "RoPE caveat", re-positioning)."""
    w, pl, ol, k, v, q, bias, cfg = make_case(name)
    say("rope decode", name)
    c, o = build_pair(pl, ol, k, v, w.dtype, chunks=cfg.get("chunks"), k_bias=bias)
    table = K.kvq_rope_table(pl.capacity + 8, pl.head_dim)
    for q_pos in (c.n_stored - 1, c.n_stored + 3, 0):
        check_decode_rope(pl, c, o, q, w.dtype, table, q_pos)


def test_streaming_rope_repositioning_kivi_int8_tiny():
    """StreamingLLM over 500 positions (sink 4 + window 256, KIVI int8): with
    RoPE on read the sink and window keys sit at slots 0..259, the query at
    the newest slot, so attention never sees a distance beyond the cache."""
    w = synth.workload("kivi_int8_tiny")
    k, v, q = gen(w, 1, 8, 500)
    pl, ol = layouts(batch=1, n_kv_heads=8, head_dim=32, capacity=261, k_kind="kivi_ch", k_bits=8,
                     k_group=32, v_kind="tok_affine", v_bits=8, v_group=32, in_dtype="f32")
    say("stream rope kivi int8 500")
    c, o = stream_pair(pl, ol, k, v, "f32", 4, 256)
    table = K.kvq_rope_table(261, 32)
    check_decode_rope(pl, c, o, q, "f32", table, c.n_stored - 1)


@pytest.mark.parametrize("gt,G,dt,qdt,vb,vg", [(16, 4, "f16", "f16", 4, 32), (64, 2, "bf16", "bf16", 8, 128),
                                              (8, 3, "f32", "f16", 4, 64), (128, 1, "f16", "bf16", 8, 32),
                                              (32, 4, "f32", "bf16", 4, 32)])
def test_kivi_matrix_core_group_sizes(gt, G, dt, qdt, vb, vg):
    """KIVI 4-bit keys on the matrix-core decode with token groups of 8 to
    128: a 32-token tile then holds one group, two (the second staged row)
    or four (rows beyond the two staged ones take the per-lane path); the
    open group is read from an fp16, bf16 or fp32 residual.  Then the same
    cache after StreamingLLM compaction (sink 5, window 700), whose tiles
    mix table rows of the sink and window runs."""
    rng = np.random.default_rng(gt * 10 + G)
    B, H, T, D = 1, 2, 1333, 128
    k = (rng.standard_normal((B, H, T, D)) * np.where(rng.random(D) < 0.05, 10.0, 1.0)).astype(np.float32)
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    q = rng.standard_normal((B, H * G, D)).astype(np.float32)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind="kivi_ch", k_bits=4, k_group=gt,
                     v_kind="tok_affine", v_bits=vb, v_group=vg, in_dtype=dt)
    say("kivi matrix-core groups", gt, G, dt, qdt, vb, vg)
    c, o = build_pair(pl, ol, synth.cast(k, dt), synth.cast(v, dt), dt, chunks=[(0, 1), (1, 600), (600, T)])
    assert_same_state(c, o)
    qq = synth.cast(q, qdt)
    check_decode(pl, c, o, qq, qdt)
    dst = K.Cache(pl)
    assert K.kvq_evict_streaming(pl, c, dst, 5, 700) == K.KVQ_OK
    torch.cuda.synchronize()
    check_decode(pl, dst, o.evict(5, 700), qq, qdt)


@pytest.mark.parametrize("k_kind,kg,G,vb,vg", [("tok_affine", 64, 1, 4, 64), ("tok_sym4", 32, 2, 8, 128),
                                               ("tok_affine", 32, 3, 4, 32)])
def test_matrix_core_decode_fewer_query_heads(k_kind, kg, G, vb, vg):
    """Per-token 4-bit keys with 1-3 query heads per kv-head on the
    matrix-core decode (the rows of the missing heads are zero and never
    written): ragged length, split over T."""
    w = synth.workload("q4_0_centered")
    B, H, T = 2, 2, 1555
    k, v, q = gen(w, B, H, T, Hq=H * G)
    bias = np.stack([synth.head_params(w, h)[0] for h in range(H)]).astype(np.float32)
    flags = K.KVQ_CENTER_K if k_kind == "tok_sym4" else 0
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind=k_kind, k_bits=4, k_group=kg,
                     v_kind="tok_affine", v_bits=vb, v_group=vg, in_dtype="f16", flags=flags)
    say("matrix-core fewer heads", k_kind, kg, G, vb, vg)
    c, o = build_pair(pl, ol, k, v, "f16", chunks=[(0, 700), (700, T)], k_bias=bias if flags else None)
    out = torch.full((B, H * G, 128), 9.0, device=DEV)
    K.kvq_decode_attention(pl, c, to_dev(q, "f16"), out=out)
    torch.cuda.synchronize()
    err = attn_err(out.cpu().numpy(), o.decode(q, "f16"))
    say(f"  attention error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("k_kind,G", [("kivi_ch", 3), ("tok_affine", 4)])
def test_split_decode_repeats_bit_identically(k_kind, G):
    """A decode split over T (partials merged by log-sum-exp): thirty
    back-to-back calls, queued without synchronization, give bit-identical
    outputs that match the oracle."""
    w = synth.workload("llama3b_kivi_int4")
    B, H, T = 1, 8, 3001
    k, v, q = gen(w, B, H, T, Hq=H * G)
    kg = 32 if k_kind == "kivi_ch" else 64
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=128, capacity=T, k_kind=k_kind, k_bits=4, k_group=kg,
                     v_kind="tok_affine", v_bits=4, v_group=32, in_dtype="f16")
    say("split merge repeats", k_kind, G)
    c, o = build_pair(pl, ol, k, v, "f16")
    qd = to_dev(q, "f16")
    outs = [K.kvq_decode_attention(pl, c, qd) for _ in range(30)]
    torch.cuda.synchronize()
    first = outs[0].cpu().numpy()
    for x in outs[1:]:
        assert np.array_equal(x.cpu().numpy().view(np.uint32), first.view(np.uint32))
    err = attn_err(first, o.decode(q, "f16"))
    say(f"  attention error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("wname,D,lay,T", [
    # matrix-core decode: 64 splits of 256 tokens
    ("affine4_g64", 128, dict(k_kind="tok_affine", k_bits=4, k_group=64, v_kind="tok_affine", v_bits=4,
                              v_group=64), 16384),
    # KIVI keys: 64 splits of 8 tiles, workgroups of 8 waves
    ("llama3b_kivi_int4", 128, dict(k_kind="kivi_ch", k_bits=4, k_group=32, v_kind="tok_affine", v_bits=4,
                                    v_group=64), 16384),
    # generic decode (8-bit codes at head_dim 64)
    ("affine4_g64", 64, dict(k_kind="tok_affine", k_bits=8, k_group=32, v_kind="tok_affine", v_bits=8,
                             v_group=32), 6000),
])
def test_decode_many_splits(wname, D, lay, T):
    """One kv-head of four query heads over a long cache: the split plans take
    many splits, and the combine reads the splits past its prefetch in its
    tail loop."""
    B, H, Hq = 1, 1, 4
    w = synth.workload(wname, head_dim=D)
    k, v, q = gen(w, B, H, T, Hq)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T + 37, in_dtype=w.dtype, **lay)
    say("decode many splits", wname, D, lay["k_kind"], T)
    c, o = build_pair(pl, ol, k, v, w.dtype)
    check_decode(pl, c, o, q, w.dtype)

"""Pins of the CPU oracle to facts the source pages and mathematics fix.

Each test names what it pins and why a plausible mistake would fail it.
Nothing here retypes an oracle formula: expected values come from closed
forms, library routines (numpy / scipy), brute force on tiny inputs, or the
pages' own numbers (tests/golden/*.json).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.cache import Layout, OracleCache, snapkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_f16_rounding_matches_numpy_on_random_bit_patterns():
    """fp32 -> fp16 round-to-nearest-even incl. subnormals, overflow and ties
    (pinned to numpy's independent conversion)."""
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # concentrate on the fp16 range, subnormals and exact ties
    near = (rng.standard_normal(200_000) * 10.0 ** rng.integers(-9, 5, 200_000)).astype(np.float32)
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    h = h[np.isfinite(h)]
    ties = ((h[:-1] + h[1:]) / 2).astype(np.float32)     # exact midpoints
    x = np.concatenate([x, near, ties, np.float32([65504, 65519.99, 65520, -65520, 1e-5, 6e-8, 3e-8])])
    got = oracle.f32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_f16_widening_is_exact_for_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_bits_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.all(np.isnan(got[~fin]) == np.isnan(want[~fin]))


def test_eps_is_an_fp16_subnormal():
    """[P1] eps = 1e-5 stored as fp16 is the subnormal 168 * 2^-24 (must not flush)."""
    assert int(oracle.f32_to_f16_bits(np.float32([1e-5]))[0]) == 168
    assert oracle.f16_bits_to_f32(np.uint16([168]))[0] == np.float32(168 * 2.0 ** -24)


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def test_affine_int4_grid_is_lossless():
    """Values zero + j/8 with range exactly 15/8: scale 1/8, zero = min, codes = j."""
    rng = np.random.default_rng(1)
    j = rng.integers(0, 16, size=(50, 64))
    j[:, 0], j[:, 1] = 0, 15
    m0 = np.float32(-1.25)
    x = (m0 + j.astype(np.float32) / 8).astype(np.float32)
    u, meta = oracle.quant_tok_affine(x, G=64, bits=4)
    assert np.array_equal(u, j.astype(np.uint8))
    assert np.all(oracle.f16_bits_to_f32(meta[..., 0]) == 0.125)
    assert np.all(oracle.f16_bits_to_f32(meta[..., 1]) == m0)
    # dequantization of a lossless code grid gives the input back exactly
    v = oracle.make_view(oracle.TOK_AFFINE, 64, 64, u=u, meta=meta)
    assert np.array_equal(oracle.dequant(v, 50, 64), x.astype(np.float64))


def test_affine_int8_channel_group_grid():
    """Per-channel over 32 tokens: min and max at 255/64 apart -> scale 1/64, codes = j."""
    rng = np.random.default_rng(2)
    D = 32
    j = rng.integers(0, 256, size=(32, D))
    j[3, :], j[17, :] = 0, 255
    base = np.float32(0.5) * np.arange(D, dtype=np.float32)  # per-channel offset, exact in fp16
    x = (base[None, :] + j.astype(np.float32) / 64).astype(np.float32)
    u, meta = oracle.quant_channel_group(x, bits=8)
    assert np.array_equal(u, j.astype(np.uint8))
    assert np.all(oracle.f16_bits_to_f32(meta[:, 0]) == np.float32(1 / 64))
    assert np.array_equal(oracle.f16_bits_to_f32(meta[:, 1]), base)
    # transposing the group (per-token instead of per-channel) must not pass
    u_t, _ = oracle.quant_tok_affine(x, G=D, bits=8)
    assert not np.array_equal(u_t, u)


def test_constant_channel_uses_eps_scale():
    """[P1] bug class 1: a constant slice gets scale max(eps, 0) = fp16(1e-5)."""
    x = np.full((1, 32), 0.1, dtype=np.float32)
    u, meta = oracle.quant_tok_affine(x, G=32, bits=8)
    s = oracle.f16_bits_to_f32(meta[..., 0])[0, 0]
    z = oracle.f16_bits_to_f32(meta[..., 1])[0, 0]
    assert s == np.float32(168 * 2.0 ** -24)
    assert z == np.float16(0.1).astype(np.float32)
    # (0.1 - fp16(0.1)) / s = 2.43.. -> code 2; reconstruction within s/2
    assert np.all(u == 2)
    assert abs(2 * float(s) + float(z) - 0.1) <= float(s) / 2


def test_rounding_is_half_even_and_not_offset_first():
    """Codes use rint((x - zero) / scale) (ties to even), not round(... + qMin).

    With scale 1/8, zero 0: (x - z)/s = 2.5 -> 2, 3.5 -> 4.  With
    (x - z)/s = 0.5 + 2^-20 the code is 1; adding qMin = -128 first would round
    -127.49999905 to -127.5 in fp32 and then to -128, i.e. code 0."""
    g = np.zeros(64, dtype=np.float32)
    g[1] = 15 / 8                      # range 15/8 -> scale 1/8 at int4
    g[2], g[3] = 2.5 / 8, 3.5 / 8
    u, _ = oracle.quant_tok_affine(g[None], G=64, bits=4)
    assert (u[0, 2], u[0, 3]) == (2, 4)
    g8 = np.zeros(32, dtype=np.float32)
    g8[1] = np.float32(255 / 8)        # int8 range 255/8 -> scale 1/8
    g8[2] = np.float32(2.0 ** -4 + 2.0 ** -23)
    u8, _ = oracle.quant_tok_affine(g8[None], G=32, bits=8)
    assert u8[0, 2] == 1
    literal = np.float32(np.float32(g8[2] / np.float32(0.125)) + np.float32(-128))
    assert np.rint(literal) + 128 == 0   # the rejected order gives a different code


def test_affine_error_bound_random():
    """|x - xhat| <= s/2 + |z - min| + 4 ulp(max|x|) for every element (int4 and int8)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((400, 128)) * rng.uniform(0.01, 20, (400, 1))).astype(np.float32)
    for bits, G in ((4, 64), (4, 32), (8, 128)):
        u, meta = oracle.quant_tok_affine(x, G=G, bits=bits)
        s = oracle.f16_bits_to_f32(meta[..., 0]).astype(np.float64)
        z = oracle.f16_bits_to_f32(meta[..., 1]).astype(np.float64)
        xg = x.reshape(400, 128 // G, G).astype(np.float64)
        xhat = u.reshape(400, 128 // G, G) * s[..., None] + z[..., None]
        mn = xg.min(-1)
        ulp = np.spacing(np.abs(xg).max(-1).astype(np.float32)).astype(np.float64)
        bound = s / 2 + np.abs(z - mn) + 4 * ulp
        assert np.all(np.abs(xg - xhat) <= bound[..., None])
        assert u.max() <= 2 ** bits - 1


def test_sym4_grid_and_centering_noop():
    """[P3]: symmetric blocks; grid k/8 with |k| <= 7 and one |k| = 7 gives d = 1/8,
    codes k + 8; centering by an exactly representable bias gives the same
    codes; a NULL bias and an all-zero bias are byte-identical."""
    rng = np.random.default_rng(4)
    k = rng.integers(-7, 8, size=(40, 128))
    k[:, ::32] = 7
    x = (k / 8).astype(np.float32)
    u, sc = oracle.quant_sym4(x, None)
    assert np.array_equal(u, (k + 8).astype(np.uint8))
    assert np.all(oracle.f16_bits_to_f32(sc) == 0.125)
    bias = (rng.integers(-64, 64, size=128) / 4).astype(np.float32)
    uc, scc = oracle.quant_sym4((x + bias).astype(np.float32), bias)
    assert np.array_equal(uc, u) and np.array_equal(scc, sc)
    xr = (rng.standard_normal((40, 128)) * 3).astype(np.float32)
    a = oracle.quant_sym4(xr, None)
    b = oracle.quant_sym4(xr, np.zeros(128, np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    v = oracle.make_view(oracle.SYM4, 128, u=u, meta=sc)
    assert np.array_equal(oracle.dequant(v, 40, 128), x.astype(np.float64))


def test_sym4_error_bound_and_range():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 128)) * 2 + 1).astype(np.float32)
    bias = rng.standard_normal(128).astype(np.float32)
    u, sc = oracle.quant_sym4(x, bias)
    d = oracle.f16_bits_to_f32(sc).astype(np.float64)
    xc = (x - bias).astype(np.float32).astype(np.float64).reshape(300, 4, 32)
    xhat = (u.reshape(300, 4, 32).astype(np.float64) - 8) * d[..., None]
    amax = np.abs(xc).max(-1)
    # |x' - xhat| <= d/2 except where rounding to fp16 made d*7 < amax (clamp at +7);
    # the clamp error is at most amax - 7d + d/2.
    lim = d / 2 + np.maximum(0.0, amax - 7 * d) + 4 * np.spacing(amax.astype(np.float32))
    assert np.all(np.abs(xc - xhat) <= lim[..., None])
    assert u.min() >= 0 and u.max() <= 15


# Half-even rounding of k + 1/2, written out: the even one of k and k + 1
# (the ties that fit under max |x'/d| = 7).
SYM4_TIES = {-7: -6, -6: -6, -5: -4, -4: -4, -3: -2, -2: -2, -1: 0,
             0: 0, 1: 2, 2: 2, 3: 4, 4: 4, 5: 6, 6: 6}


def test_sym4_ties_round_half_even():
    """[P3] "The idea" (symmetric, no zero point) with the rint of the
    specification: a block whose max |x'| is 7/8 has d = 1/8 exactly, so
    x' = (k + 1/2)/8 is a tie k + 1/2 and must go to the even neighbour
    (round-half-away would give k + 1 for k >= 0 and k for k < 0).  The same
    ties after centering by a bias on the 1/16 grid (x - bias exact)."""
    ks = sorted(SYM4_TIES)                                      # -7 .. 6
    vals = [7.0, -7.0, 0.0, 0.0] + [k + 0.5 for k in ks] + [k + 0.5 for k in ks[::-1]]
    want = [7, -7, 0, 0] + [SYM4_TIES[k] for k in ks] + [SYM4_TIES[k] for k in ks[::-1]]
    assert len(vals) == 32
    x = np.tile(np.array(vals) / 8, 4)[None].astype(np.float32)   # one row, 4 blocks
    u, sc = oracle.quant_sym4(x, None)
    assert np.all(sc == 0x3000)                                 # fp16 bits of 1/8
    assert np.array_equal(u[0], np.tile(np.array(want) + 8, 4).astype(np.uint8))
    bias = (np.arange(128) % 37 - 18).astype(np.float32) / 16
    xb = (x + bias).astype(np.float32)
    assert np.array_equal((xb - bias).astype(np.float32), x)     # exact on this grid
    ub, scb = oracle.quant_sym4(xb, bias)
    assert np.array_equal(ub, u) and np.array_equal(scb, sc)


def test_sym4_zero_block_takes_eps_scale():
    """[P1] "The bug class the previous attempt hit" (class 1: a degenerate
    range must not divide by zero) reached through [P3]'s subtraction: a key
    equal to the bias is an all-zero centered block, so d = fp16(1e-5) (the
    subnormal 168 * 2^-24) and every code is 8 (q = 0).  Blocks with
    max |x'| below 7e-5 also take the eps scale; their codes follow x'/d."""
    bias = (np.arange(128, dtype=np.float32) - 60) / 8
    x = np.tile(bias, (3, 1)).astype(np.float32)
    x[1, 32:64] += np.float32(2.0 ** -20)     # one tiny block: x'/d = 2^-20 / (168 * 2^-24) = 16/168
    x[2, 64:96] += np.float32(2.0 ** -14)     # max |x'| / 7 = 8.7e-6 < eps; x'/d = 1024/168 = 6.1 -> 6
    u, sc = oracle.quant_sym4(x, bias)
    assert sc.shape == (3, 4)
    assert np.all(sc == 168)
    want = np.full((3, 128), 8, np.uint8)
    want[2, 64:96] = 14
    assert np.array_equal(u, want)
    u0, sc0 = oracle.quant_sym4(np.zeros((2, 64), np.float32), None)
    assert np.all(sc0 == 168) and np.all(u0 == 8)


def test_quant_codes_use_the_stored_fp16_scale():
    """O3/O9: codes are taken against the scale as stored (fp16), not the fp32
    value before rounding.  Each input below sits between the two quotients'
    rounding boundary, so the two readings give different codes.

    Affine int4: range 1.5 -> s32 = 0.1, stored s = fp16(0.1) = 0.0999755859375
    (below s32); x = 1.4498 gives x/s = 14.5015 against the stored scale
    (code 15) but 14.498 against s32 (code 14).
    Q4_0: max |x'| = 1 -> d32 = 1/7, stored d = 1170/8192 = 0.142822265625;
    x' = 2.5 * (d + d32)/2 gives x'/d just above 2.5 (q = 3, code 11) and
    x'/d32 just below (q = 2, code 10)."""
    g = np.zeros(32, np.float32)
    g[1] = 1.5
    g[2] = np.float32(1.4498)
    s16 = np.float64(np.float16(0.1))
    assert s16 == 0.0999755859375
    assert float(g[2]) / s16 > 14.5 > float(g[2]) / 0.1
    u, meta = oracle.quant_tok_affine(g[None], G=32, bits=4)
    assert meta[0, 0, 0] == np.float16(0.1).view(np.uint16)
    assert u[0, 2] == 15
    d16 = 1170 / 8192
    assert np.float64(np.float16(np.float32(1) / np.float32(7))) == d16
    blk = np.zeros(32, np.float32)
    blk[0] = 1.0
    blk[1] = np.float32(2.5 * (d16 + 1 / 7) / 2)
    assert float(blk[1]) / d16 > 2.5 > float(blk[1]) * 7
    us, ss = oracle.quant_sym4(blk[None], None)
    assert oracle.f16_bits_to_f32(ss)[0, 0] == np.float32(d16)
    assert us[0, 0] == 15 and us[0, 1] == 11


# --------------------------------------------------------------------------
# decode attention
# --------------------------------------------------------------------------

def _softmax_attention(q, K, V, scale):
    p = scipy.special.softmax(scale * (K @ q))
    return p @ V


def test_decode_matches_brute_force_softmax_attention():
    """kvo_decode_head equals scipy softmax attention over the same dequantized K, V."""
    rng = np.random.default_rng(6)
    T, D = 37, 32
    x = rng.standard_normal((T, D)).astype(np.float32)
    ku, km = oracle.quant_tok_affine(x, G=32, bits=4)
    vu, vm = oracle.quant_tok_affine(rng.standard_normal((T, D)).astype(np.float32), G=16, bits=8)
    kv = oracle.make_view(oracle.TOK_AFFINE, D, 32, u=ku, meta=km)
    vv = oracle.make_view(oracle.TOK_AFFINE, D, 16, u=vu, meta=vm)
    Kd, Vd = oracle.dequant(kv, T, D), oracle.dequant(vv, T, D)
    q = rng.standard_normal(D).astype(np.float32)
    for scale in (1 / math.sqrt(D), 0.3):
        got = oracle.decode_head(kv, vv, T, q, scale)
        want = _softmax_attention(q.astype(np.float64), Kd, Vd, scale)
        assert np.allclose(got, want, rtol=0, atol=1e-12)
    # swapping K and V (a transposed-operand mistake) changes the answer
    swapped = oracle.decode_head(vv, kv, T, q, 1 / math.sqrt(D))
    assert not np.allclose(swapped, oracle.decode_head(kv, vv, T, q, 1 / math.sqrt(D)))


def test_decode_special_cases():
    rng = np.random.default_rng(7)
    D = 32
    K = rng.standard_normal((9, D)).astype(np.float32)
    V = rng.standard_normal((9, D)).astype(np.float32)
    q = rng.standard_normal(D).astype(np.float32)
    kv = oracle.make_view(oracle.PLAIN, D, plain=K)
    vv = oracle.make_view(oracle.PLAIN, D, plain=V)
    # T = 1: the only value row
    assert np.array_equal(oracle.decode_head(kv, vv, 1, q, 0.2), V[0].astype(np.float64))
    # identical keys: uniform weights -> mean of values
    Ks = np.repeat(K[:1], 9, axis=0)
    out = oracle.decode_head(oracle.make_view(oracle.PLAIN, D, plain=Ks), vv, 9, q, 0.2)
    assert np.allclose(out, V.astype(np.float64).mean(0), atol=1e-15)
    # empty cache -> zeros
    assert np.all(oracle.decode_head(kv, vv, 0, q, 0.2) == 0)


def test_decode_shift_invariance():
    """[P3] "Why this is safe": subtracting the same k_bar from every key adds the
    constant q.k_bar to every logit of the row; softmax does not see it."""
    rng = np.random.default_rng(8)
    T, D = 64, 32
    K = rng.standard_normal((T, D)).astype(np.float32)
    V = rng.standard_normal((T, D)).astype(np.float32)
    kbar = (rng.standard_normal(D) * 1.5).astype(np.float32)
    q = rng.standard_normal(D).astype(np.float32)
    a = oracle.decode_head(oracle.make_view(oracle.PLAIN, D, plain=K),
                           oracle.make_view(oracle.PLAIN, D, plain=V), T, q, 0.2)
    Kc = (K.astype(np.float64) - kbar).astype(np.float32)
    b = oracle.decode_head(oracle.make_view(oracle.PLAIN, D, plain=Kc),
                           oracle.make_view(oracle.PLAIN, D, plain=V), T, q, 0.2)
    nmse = np.sum((a - b) ** 2) / np.sum(a ** 2)
    assert nmse < 1e-9, nmse
    # a bias that differs per key is NOT invariant (the pin would catch a per-token shift)
    Kp = (K.astype(np.float64) - rng.standard_normal((T, 1))).astype(np.float32)
    c = oracle.decode_head(oracle.make_view(oracle.PLAIN, D, plain=Kp),
                           oracle.make_view(oracle.PLAIN, D, plain=V), T, q, 0.2)
    assert np.sum((a - c) ** 2) / np.sum(a ** 2) > 1e-4


def test_channel_view_reads_residual_and_rows():
    """Per-channel K: coded slots use their row's scales, later slots the fp residual."""
    rng = np.random.default_rng(9)
    D, Gt = 32, 8
    j = rng.integers(0, 16, size=(16, D))
    j[0], j[1] = 0, 15
    j[8], j[9] = 0, 15
    offs = np.float32([0.5, -2.0])
    x = np.concatenate([offs[0] + j[:8] / 8, offs[1] + j[8:] / 4]).astype(np.float32)
    u0, m0 = oracle.quant_channel_group(x[:8], 4)
    u1, m1 = oracle.quant_channel_group(x[8:], 4)
    resid = rng.standard_normal((3, D)).astype(np.float32)
    view = oracle.make_view(oracle.CHANNEL, D, u=np.concatenate([u0, u1, np.zeros((3, D), np.uint8)]),
                            meta=np.stack([m0, m1]), row=np.int32([0] * 8 + [1] * 8 + [0] * 3),
                            plain=resid, n_coded=16)
    got = oracle.dequant(view, 19, D)
    assert np.array_equal(got[:16], x.astype(np.float64))
    assert np.array_equal(got[16:], resid.astype(np.float64))


# --------------------------------------------------------------------------
# cache model: append, residual groups, eviction
# --------------------------------------------------------------------------

def _c1_stream(L, k, v, evict_each=True, sink=4, window=256):
    c = OracleCache(L)
    for t in range(k.shape[2]):
        c.append(k[:, :, t:t + 1], v[:, :, t:t + 1])
        if evict_each:
            e = c.evict(sink, window)
            if e is not None:
                c = e
    return c


def test_streaming_cap_and_positions_tinygpt_shape():
    """[P1] smoke test: sink 4 + window 256 over 500 positions stores exactly 260,
    positions [0,4) U [244,500); K groups of 32: 240 coded slots + 20 residual,
    9 live scale rows (groups 0 and 7..14)."""
    g = golden("p1_streaming_kivi.json")["streaming"]
    rng = np.random.default_rng(10)
    B, H, D, N = 1, 8, 32, g["generated"]
    k = rng.standard_normal((B, H, N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    L = Layout(B, H, D, capacity=g["stored_cap"] + 1, k_kind="kivi_ch", k_bits=8, k_group=32,
               v_kind="tok_affine", v_bits=8, v_group=32, in_dtype="f32")
    c = _c1_stream(L, k, v, sink=g["sink"], window=g["window"])
    assert c.n_stored == g["stored_cap"]
    assert np.array_equal(c.pos[:260], np.r_[0:4, 244:500])
    assert c.n_quant == 240 and c.next_pos == 500
    rows = c.k_row[:240]
    assert np.array_equal(np.unique(rows), np.arange(9))
    # groups of the kept slots: pos // 32 -> rank among {0, 7, ..., 14}
    grp = c.pos[:240] // 32
    live = np.r_[0, 7:15]
    assert np.array_equal(rows, np.searchsorted(live, grp))
    # streaming eviction == append everything, then evict once
    Lb = Layout(B, H, D, capacity=N, k_kind="kivi_ch", k_bits=8, k_group=32,
                v_kind="tok_affine", v_bits=8, v_group=32, in_dtype="f32")
    cb = _c1_stream(Lb, k, v, evict_each=False).evict(4, 256)
    for name in ("pos", "k_row"):
        assert np.array_equal(getattr(c, name)[:260], getattr(cb, name)[:260])
    assert np.array_equal(c.k_u[:, :, :240], cb.k_u[:, :, :240])
    assert np.array_equal(c.v_u[:, :, :260], cb.v_u[:, :, :260])
    assert np.array_equal(c.v_meta[:, :, :260], cb.v_meta[:, :, :260])
    assert np.array_equal(c.k_table[:, :, :9], cb.k_table[:, :, :9])
    assert np.array_equal(c.k_resid, cb.k_resid)
    # idempotent: a second eviction drops nothing
    assert c.evict(4, 256) is None


def test_chunked_append_equals_token_by_token():
    rng = np.random.default_rng(11)
    B, H, D, N = 2, 2, 64, 150
    for k_kind, kb, kg in (("kivi_ch", 4, 32), ("tok_affine", 4, 64), ("tok_sym4", 4, 32)):
        L = Layout(B, H, D, N, k_kind=k_kind, k_bits=kb, k_group=kg,
                   v_kind="tok_affine", v_bits=4, v_group=32, in_dtype="f16")
        k = rng.standard_normal((B, H, N, D)).astype(np.float16)
        v = rng.standard_normal((B, H, N, D)).astype(np.float16)
        a = OracleCache(L)
        a.append(k, v)
        b = OracleCache(L)
        for s, e in ((0, 1), (1, 40), (40, 41), (41, 100), (100, 150)):
            b.append(k[:, :, s:e], v[:, :, s:e])
        for name in ("k_u", "k_meta", "k_table", "k_resid", "v_u", "v_meta", "pos", "k_row"):
            x, y = getattr(a, name), getattr(b, name)
            assert (x is None and y is None) or np.array_equal(x, y), (k_kind, name)
        assert (a.n_stored, a.n_quant) == (b.n_stored, b.n_quant)


def test_eviction_keeps_rows_bit_identical():
    rng = np.random.default_rng(12)
    B, H, D = 1, 3, 32
    L = Layout(B, H, D, 100, k_kind="tok_affine", k_bits=4, k_group=32,
               v_kind="tok_affine", v_bits=8, v_group=32, in_dtype="f32")
    c = OracleCache(L)
    c.append(rng.standard_normal((B, H, 90, D)).astype(np.float32),
             rng.standard_normal((B, H, 90, D)).astype(np.float32))
    e = c.evict(5, 20)
    keep = np.r_[0:5, 70:90]
    assert e.n_stored == 25
    assert np.array_equal(e.k_u[:, :, :25], c.k_u[:, :, keep])
    assert np.array_equal(e.v_meta[:, :, :25], c.v_meta[:, :, keep])
    assert np.array_equal(e.pos[:25], keep)
    assert c.evict(60, 30) is None


# --------------------------------------------------------------------------
# SnapKV
# --------------------------------------------------------------------------

def test_snapkv_scores_brute_force_and_invariants():
    """[P2] step 1 against scipy: mean over the last w rows of softmax(K_w K^T / sqrt(D))."""
    rng = np.random.default_rng(13)
    S, D = 70, 32
    K = rng.standard_normal((S, D)).astype(np.float16).astype(np.float32)
    for w in (1, 8, 70, 500):
        got = oracle.snapkv_scores(K, w)
        wc = min(w, S)
        P = scipy.special.softmax(K[S - wc:].astype(np.float64) @ K.T.astype(np.float64) / math.sqrt(D), axis=1)
        assert np.allclose(got, P.mean(0), rtol=0, atol=1e-14)
        assert abs(got.sum() - 1) < 1e-12
        assert got.min() >= 0 and got.max() <= 1
    # identical keys -> uniform scores
    same = np.repeat(K[:1], S, axis=0)
    assert np.allclose(oracle.snapkv_scores(same, 8), 1 / S, atol=1e-15)


def test_snapkv_select_invariants():
    """[P2] Evidence list: count, order, sinks with zero scores, known top, budget >= S."""
    g = golden("p2_snapkv_defaults.json")
    S = 2000
    rng = np.random.default_rng(14)
    sc = rng.random(S).astype(np.float32)
    kept = oracle.snapkv_select(sc, g["n_sink"], g["budget"])
    assert kept.size == g["budget"] and np.all(np.diff(kept) > 0)
    assert set(range(g["n_sink"])) <= set(kept.tolist())
    # brute force: lexsort by (-score, index) over the non-sink candidates
    cand = np.arange(g["n_sink"], S)
    order = cand[np.lexsort((cand, -sc[cand].astype(np.float64)))]
    want = np.sort(np.r_[0:g["n_sink"], order[:g["budget"] - g["n_sink"]]])
    assert np.array_equal(kept, want)
    # zero scores: sinks still kept; remaining ties go to the lowest positions
    z = oracle.snapkv_select(np.zeros(S, np.float32), 4, 10)
    assert np.array_equal(z, np.arange(10))
    # known high-score keys are selected
    sc2 = np.zeros(S, np.float32)
    top = rng.choice(np.arange(4, S), size=6, replace=False)
    sc2[top] = 1.0
    assert set(top.tolist()) <= set(oracle.snapkv_select(sc2, 4, 10).tolist())
    # budget >= S keeps everything; n_sink > budget is clamped
    assert np.array_equal(oracle.snapkv_select(sc[:50], 4, 512), np.arange(50))
    assert np.array_equal(oracle.snapkv_select(sc, 30, 10), np.arange(10))


def test_snapkv_end_to_end_shapes_and_coverage():
    """Gathered rows are the kept rows; the kept set maximizes the score mass among
    sets that contain the sinks ([P2] coverage harness, by construction)."""
    rng = np.random.default_rng(15)
    B, H, S, D = 1, 2, 300, 32
    K = rng.standard_normal((B, H, S, D)).astype(np.float16)
    V = rng.standard_normal((B, H, S, D)).astype(np.float16)
    scores, kept, Ko, Vo = snapkv(K, V, obs_window=16, n_sink=4, budget=40)
    assert kept.shape == (B, H, 40) and Ko.shape == (B, H, 40, D) and Ko.dtype == np.float16
    for h in range(H):
        assert np.array_equal(Ko[0, h], K[0, h, kept[0, h]])
        assert np.array_equal(Vo[0, h], V[0, h, kept[0, h]])
        s = scores[0, h]
        rand = np.r_[0:4, rng.choice(np.arange(4, S), 36, replace=False)]
        assert s[kept[0, h]].sum() >= s[rand].sum()


def test_snapkv_query_rows_pins():
    """[P2] "Proxy limitation" variant: observation rows given explicitly.
    Pinned to the key-proxy scorer (same rows), to the uniform closed form for
    zero queries, and to a closed form for a one-hot query over one-hot keys."""
    rng = np.random.default_rng(11)
    K = rng.standard_normal((90, 32)).astype(np.float32)
    # the trailing key rows as explicit rows reproduce the proxy scores exactly
    assert np.array_equal(oracle.snapkv_scores_rows(K[-12:], K), oracle.snapkv_scores(K, 12))
    # zero queries: every logit 0, so every score is 1/S
    z = oracle.snapkv_scores_rows(np.zeros((5, 32), np.float32), K)
    assert np.allclose(z, 1.0 / 90, rtol=0, atol=1e-15)
    # one-hot keys e_(j mod D), query c e_0: logit c/sqrt(D) for j = 0 and 32, else 0
    D, S, c = 32, 40, 6.0
    Kh = np.zeros((S, D), np.float32)
    Kh[np.arange(S), np.arange(S) % D] = 1.0
    q = np.zeros((1, D), np.float32)
    q[0, 0] = c
    sc = oracle.snapkv_scores_rows(q, Kh)
    e = math.exp(c / math.sqrt(D))
    hot = e / (2 * e + (S - 2))
    cold = 1.0 / (2 * e + (S - 2))
    assert abs(sc[0] - hot) < 1e-15 and abs(sc[32] - hot) < 1e-15
    assert np.allclose(np.delete(sc, [0, 32]), cold, rtol=1e-14, atol=0)
    # rows are averaged: permuting them changes nothing, duplicating all of them neither
    Q = rng.standard_normal((7, 32)).astype(np.float32)
    a = oracle.snapkv_scores_rows(Q, K)
    assert np.allclose(oracle.snapkv_scores_rows(Q[::-1], K), a, rtol=1e-13, atol=0)
    assert np.allclose(oracle.snapkv_scores_rows(np.concatenate([Q, Q]), K), a, rtol=1e-13, atol=0)
    assert abs(a.sum() - 1.0) < 1e-12


def test_maxpool_pins():
    """[P2] "Proxy limitation": max-pool smoothing of width k before ranking.
    Pinned to scipy's maximum filter (edge clamping adds no new values), the
    identity at k = 1 and the global max at k >= 2S - 1."""
    from scipy.ndimage import maximum_filter1d
    rng = np.random.default_rng(12)
    for S in (1, 2, 7, 100):
        x = rng.random(S).astype(np.float32)
        x[S // 2] = x[0]                      # ties
        for k in (1, 3, 5, 7, 31):
            got = oracle.maxpool1d(x, k)
            assert np.array_equal(got, maximum_filter1d(x, size=k, mode="nearest")), (S, k)
        assert np.array_equal(oracle.maxpool1d(x, 1), x)
        assert np.all(oracle.maxpool1d(x, 2 * S + 1) == x.max())


def test_bits_per_element_accounting():
    """[P4] s.2 / s.4: 4-bit g64 with fp16 scale+bias is 4.5 bits/elt, g32 is 5.0."""
    for case in golden("p4_bits_per_element.json")["cases"]:
        G, bits = case["group"], case["bits"]
        per_group_bits = G * bits + 2 * 16
        assert per_group_bits / G == case["bits_per_element"]


def test_snapkv_chunked_single_chunk_is_one_shot():
    """[P2] "How it works": one prefill call over an empty state is the
    one-shot selection; kept rows keep their absolute positions."""
    from oracle.cache import SnapState, snapkv, snapkv_chunk
    rng = np.random.default_rng(21)
    K = rng.standard_normal((1, 2, 300, 32)).astype(np.float16)
    V = rng.standard_normal((1, 2, 300, 32)).astype(np.float16)
    st, sc, kept = snapkv_chunk(SnapState.empty(1, 2, 32), K, V, 16, 4, 40)
    ref_sc, ref_kept, ref_k, ref_v = snapkv(K, V, 16, 4, 40)
    assert np.array_equal(sc, ref_sc) and np.array_equal(kept, ref_kept)
    assert np.array_equal(st.k, ref_k) and np.array_equal(st.v, ref_v)
    assert np.array_equal(st.pos, ref_kept) and st.next_pos == 300


def test_snapkv_chunked_closed_form():
    """Two prefill chunks whose scores are known in closed form.  Keys are
    c e_0 ("hot") at positions divisible by 4 and at the chunk's last two
    positions, e_1 otherwise; the last two rows (hot) are the observation
    rows.  Hot keys score higher; equal scores go to the lower position.
    The second chunk's hot keys are 2 c e_0, so they outscore the first
    chunk's survivors and displace them (budget re-enforced, sinks kept)."""
    from oracle.cache import SnapState, snapkv_chunk
    D, c, w, sink, budget = 8, 3.0, 2, 2, 6

    def chunk(p0, mag):
        k = np.zeros((1, 1, 16, D), np.float16)
        for i in range(16):
            hot = (p0 + i) % 4 == 0 or i >= 14
            k[0, 0, i, 0 if hot else 1] = mag if hot else 1.0
        return k

    k1 = chunk(0, c)
    st, sc1, _ = snapkv_chunk(SnapState.empty(1, 1, D), k1, k1, w, sink, budget)
    assert st.pos[0, 0].tolist() == [0, 1, 4, 8, 12, 14]
    # scores: both observation rows see hot logit c^2/sqrt(D) at 6 keys, 0 at 10
    e = math.exp(c * c / math.sqrt(D))
    hot = e / (6 * e + 10)
    assert abs(sc1[0, 0, 4] - hot) < 1e-15 and abs(sc1[0, 0, 3] - 1 / (6 * e + 10)) < 1e-15
    k2 = chunk(16, 2 * c)
    st2, sc2, _ = snapkv_chunk(st, k2, k2, w, sink, budget)
    assert st2.pos[0, 0].tolist() == [0, 1, 16, 20, 24, 28] and st2.next_pos == 32
    assert np.array_equal(st2.k[0, 0, 2:], k2[0, 0, [0, 4, 8, 12]])
    # candidates: 6 survivors (hot at 0, 4, 8, 12, 14 with c; cold 1), 16 new (hot: 6 with 2c)
    e1, e2 = math.exp(2 * c * c / math.sqrt(D)), math.exp(4 * c * c / math.sqrt(D))
    Z = 5 * e1 + 6 * e2 + 11
    assert abs(sc2[0, 0, 6] - e2 / Z) < 1e-14 and abs(sc2[0, 0, 2] - e1 / Z) < 1e-14


def test_snapkv_chunked_invariants():
    """Across uneven chunks: the budget stays capped (n_kept = min(budget,
    tokens so far)), positions are ascending, absolute and include the sinks,
    every kept row is the source row of its position, and while the prompt
    fits the budget nothing is dropped."""
    from oracle.cache import SnapState, snapkv_chunk
    rng = np.random.default_rng(22)
    B, H, D, w, sink, budget = 2, 2, 32, 8, 4, 64
    sizes = [50, 1, 7, 130, 64, 3]
    total = sum(sizes)
    K = rng.standard_normal((B, H, total, D)).astype(np.float16)
    V = rng.standard_normal((B, H, total, D)).astype(np.float16)
    st = SnapState.empty(B, H, D)
    t = 0
    for S_c in sizes:
        st, _, _ = snapkv_chunk(st, K[:, :, t:t + S_c], V[:, :, t:t + S_c], w, sink, budget)
        t += S_c
        assert st.next_pos == t and st.k.shape[2] == min(budget, t)
        for b in range(B):
            for h in range(H):
                p = st.pos[b, h]
                assert np.all(np.diff(p) > 0) and p[0] >= 0 and p[-1] < t
                assert np.array_equal(p[:sink], np.arange(sink))
                assert np.array_equal(st.k[b, h], K[b, h, p]) and np.array_equal(st.v[b, h], V[b, h, p])
        if t <= budget:
            assert np.array_equal(st.pos, np.broadcast_to(np.arange(t), (B, H, t)))


def test_cache_positions_per_head_and_decode_appends():
    """Kept rows appended at their own per-head positions; later decode
    appends continue from the prompt length and are never evicted by
    SnapKV (they bypass it); positions do not change attention."""
    from oracle.cache import Layout, OracleCache
    rng = np.random.default_rng(23)
    B, H, D = 1, 2, 32
    L = Layout(B, H, D, 16, k_kind="tok_affine", k_group=32, v_group=32, in_dtype="f16", pos_per_head=True)
    Lp = Layout(B, H, D, 16, k_kind="tok_affine", k_group=32, v_group=32, in_dtype="f16")
    k = rng.standard_normal((B, H, 5, D)).astype(np.float16)
    v = rng.standard_normal((B, H, 5, D)).astype(np.float16)
    pos = np.array([[[0, 1, 7, 9, 30], [0, 1, 2, 20, 31]]], np.int32)
    c = OracleCache(L)
    c.append(k, v, positions=pos, next_pos=40)
    c.append(k[:, :, :1], v[:, :, :1])
    assert c.next_pos == 41 and c.n_stored == 6
    assert c.pos[0, 0].tolist()[:6] == [0, 1, 7, 9, 30, 40] and c.pos[0, 1].tolist()[:6] == [0, 1, 2, 20, 31, 40]
    p = OracleCache(Lp)
    p.append(k, v)
    p.append(k[:, :, :1], v[:, :, :1])
    q = rng.standard_normal((B, 2 * H, D)).astype(np.float16)
    assert np.array_equal(c.decode(q, "f16"), p.decode(q, "f16"))


def test_rope_rotation_pins():
    """RoPE on read ([P1] "RoPE caveat"): half-split pairs (x_j, x_{j+D/2})
    turned by pos * base^(-2j/D).  Pinned to closed forms for unit vectors,
    to the same rotation written as complex multiplication, to the identity
    at position 0, to norm preservation and to the relative-position
    identity <rot(q, m), rot(k, n)> = <rot(q, m + c), rot(k, n + c)>."""
    base = 10000.0
    e0, e1 = np.eye(4)[0], np.eye(4)[1]
    for p in (0, 1, 3, 17, 1000):
        assert np.allclose(oracle.rope_rotate(e0, base, p), [math.cos(p), 0, math.sin(p), 0], rtol=0, atol=1e-15)
        t1 = p * base ** -0.5
        assert np.allclose(oracle.rope_rotate(e1, base, p), [0, math.cos(t1), 0, math.sin(t1)], rtol=0, atol=1e-15)
    rng = np.random.default_rng(31)
    D = 64
    x = rng.standard_normal(D)
    assert np.array_equal(oracle.rope_rotate(x, base, 0), x)
    for p in (5, 123, 4095):
        z = (x[:D // 2] + 1j * x[D // 2:]) * np.exp(1j * p * base ** (-2.0 * np.arange(D // 2) / D))
        r = oracle.rope_rotate(x, base, p)
        assert np.allclose(r, np.concatenate([z.real, z.imag]), rtol=0, atol=1e-12)
        assert abs(np.linalg.norm(r) - np.linalg.norm(x)) < 1e-12
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    ref = oracle.rope_rotate(q, base, 40) @ oracle.rope_rotate(k, base, 7)
    for c in (1, 13, 500):
        assert abs(oracle.rope_rotate(q, base, 40 + c) @ oracle.rope_rotate(k, base, 7 + c) - ref) < 1e-11


def test_decode_rope_pins():
    """Decode with keys rotated at their slot index and the query at q_pos.
    Closed form: keys e_0 at every slot and query e_0 give logits
    scale * cos(q_pos - t); one-hot values return the softmax weights.  Also
    equal to the plain decode over keys and query rotated beforehand."""
    from oracle.cache import Layout, OracleCache
    D, T, base = 4, 4, 10000.0
    L = Layout(1, 1, D, T, k_kind="plain", v_kind="plain", in_dtype="f32")
    c = OracleCache(L)
    k = np.zeros((1, 1, T, D), np.float32)
    k[..., 0] = 1.0
    v = np.eye(D, dtype=np.float32)[None, None]
    c.append(k, v)
    q = np.zeros((1, 1, D), np.float32)
    q[..., 0] = 1.0
    for q_pos in (3, 10):
        out = c.decode(q, "f32", rope_base=base, q_pos=q_pos)[0, 0]
        lg = np.array([math.cos(q_pos - t) for t in range(T)]) / math.sqrt(D)
        w = np.exp(lg - lg.max())
        assert np.allclose(out, w / w.sum(), rtol=0, atol=1e-15)
    # against the plain decode of pre-rotated keys and query (fp32 storage of the rotation)
    rng = np.random.default_rng(32)
    D, T = 32, 50
    L2 = Layout(1, 1, D, T, k_kind="plain", v_kind="plain", in_dtype="f32")
    k = rng.standard_normal((1, 1, T, D)).astype(np.float32)
    v = rng.standard_normal((1, 1, T, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    a = OracleCache(L2)
    a.append(k, v)
    kr = np.stack([oracle.rope_rotate(k[0, 0, t], base, t) for t in range(T)]).astype(np.float32)
    b = OracleCache(L2)
    b.append(kr[None, None], v)
    qr = oracle.rope_rotate(q[0, 0], base, 60).astype(np.float32)[None, None]
    ra = a.decode(q, "f32", rope_base=base, q_pos=60)
    rb = b.decode(qr, "f32")
    assert np.allclose(ra, rb, rtol=0, atol=1e-5)


def test_two_bit_grids_and_error_bound():
    """KIVI-2bit ([P2] "SnapKV-adapted" table; 2 bits per element): four
    levels.  Lossless grids per token (groups of 32) and per channel (groups
    of 32 tokens) give codes j with scale = range / 3 and zero = min; random
    data stays within the O5 bound s/2 + |z - min| + 4 ulp."""
    rng = np.random.default_rng(41)
    j = rng.integers(0, 4, size=(40, 64))
    j[:, 0], j[:, 1], j[:, 32], j[:, 33] = 0, 3, 0, 3
    m0 = np.float32(-0.75)
    x = (m0 + j.astype(np.float32) * np.float32(0.25)).astype(np.float32)
    u, meta = oracle.quant_tok_affine(x, G=32, bits=2)
    assert np.array_equal(u, j.astype(np.uint8))
    assert np.all(oracle.f16_bits_to_f32(meta[..., 0]) == 0.25)
    assert np.all(oracle.f16_bits_to_f32(meta[..., 1]) == m0)
    xc = x[:32].copy()
    xc[5, :], xc[9, :] = m0, m0 + np.float32(0.75)
    uc, mc = oracle.quant_channel_group(xc, bits=2)
    jc = np.round((xc - m0) / np.float32(0.25)).astype(np.uint8)
    assert np.array_equal(uc, jc) and np.all(oracle.f16_bits_to_f32(mc[:, 0]) == 0.25)
    y = rng.standard_normal((64, 32)).astype(np.float32)
    u2, m2 = oracle.quant_tok_affine(y, G=32, bits=2)
    assert u2.max() <= 3
    s = oracle.f16_bits_to_f32(m2[..., 0]).astype(np.float64)[:, 0]
    z = oracle.f16_bits_to_f32(m2[..., 1]).astype(np.float64)[:, 0]
    xh = u2 * s[:, None] + z[:, None]
    bound = s / 2 + np.abs(z - y.min(1)) + 4 * np.spacing(np.abs(y).max(1))
    assert np.all(np.abs(xh - y).max(1) <= bound)


def test_prefill_attention_pins():
    """Multi-query attention over the cache ([P4] s.5 prefill shape): brute
    force with scipy's softmax and an explicit causal mask on the dequantized
    values; one query reduces to the decode; the first causal row attends to
    the prefix alone."""
    from oracle.cache import Layout, OracleCache, prefill_attention
    rng = np.random.default_rng(51)
    B, H, G, T, D, n_q = 1, 2, 2, 40, 32, 6
    L = Layout(B, H, D, T, k_kind="tok_affine", k_bits=4, k_group=32, v_kind="tok_affine", v_bits=8,
               v_group=32, in_dtype="f32")
    c = OracleCache(L)
    k = rng.standard_normal((B, H, T, D)).astype(np.float32)
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    c.append(k, v)
    q = rng.standard_normal((B, H * G, n_q, D)).astype(np.float32)
    for causal in (False, True):
        out = prefill_attention(c, q, "f32", causal=causal)
        for hq in range(H * G):
            kv, vv = c.views(0, hq // G)
            Kd, Vd = oracle.dequant(kv, T, D), oracle.dequant(vv, T, D)
            lg = (q[0, hq].astype(np.float64) @ Kd.T) / math.sqrt(D)
            if causal:
                lg = np.where(np.arange(T)[None, :] <= (T - n_q + np.arange(n_q))[:, None], lg, -np.inf)
            ref = scipy.special.softmax(lg, axis=-1) @ Vd
            assert np.allclose(out[0, hq], ref, rtol=1e-12, atol=1e-12)
    one = prefill_attention(c, q[:, :, :1], "f32")
    assert np.array_equal(one[:, :, 0], c.decode(q[:, :, 0], "f32"))

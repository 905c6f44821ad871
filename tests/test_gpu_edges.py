"""GPU parity at the edges of the quantizers' and the decodes' arithmetic.

* Q4_0-style symmetric keys ("kv-cache: optional per-channel K-cache
  mean-centering for Q4_0", The idea): quotients x'/d exactly on half-integers
  and one ulp either side (the kernel's reciprocal fast path must hand ties
  to the exact divide and round them half to even), all-zero centered blocks
  (x == k_bar, the degenerate range of "StreamingLLM + KIVI", The bug class
  the previous attempt hit, class 1: d = fp16(1e-5), codes 8) and blocks
  below the eps floor, with and without centering.  Codes and scales must
  match the oracle bit for bit.
* Values of small magnitude (V ~ N(0, sigma) with sigma 3e-3 .. 1e-2, so
  per-token scales of 1e-5 .. 1e-4): the decodes' fp16 softmax weights
  p * s must keep their relative precision; attention within 2e-3 of the
  fp64 oracle on every kernel that serves these layouts.
"""
import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K
import synth

from _gpu import assert_same_state, attn_err, layouts, say, to_dev
from test_gpu_parity import TOL, build_pair, check_decode

pytestmark = pytest.mark.gpu

# tie quotients k + 1/2 that fit under max |x'/d| = 7
_TIE_K = np.arange(-7, 7)


def sym4_edge_keys(rng, B, H, T, D, nudge):
    """Centered keys x' [B][H][T][D] fp32 built block by block (32 channels):
    kind 0: max |x'| = 7/8 (d = 1/8) and the rest (k + 1/2)/8 ties, each
            optionally moved one fp32 ulp down or up;
    kind 1: all zero (x == k_bar after centering);
    kind 2: max |x'| below 7e-5 (d at the eps floor), values on 2^-18 steps;
    kind 3: N(0, 1) values."""
    xc = np.empty((B, H, T, D), np.float32)
    kinds = rng.integers(0, 4, size=(B, H, T, D // 32))
    kinds[..., 0, :] = np.arange(D // 32) % 4            # every kind occurs
    for idx in np.ndindex(*kinds.shape):
        kind = kinds[idx]
        b, h, t, blk = idx
        if kind == 0:
            vals = rng.choice(_TIE_K, size=32) + 0.5
            vals[rng.integers(0, 32)] = 7.0 * rng.choice([-1.0, 1.0])
            blkv = (vals / 8).astype(np.float32)
            if nudge:
                n = rng.integers(-1, 2, size=32)
                n[np.abs(vals) == 7.0] = 0
                blkv = np.where(n < 0, np.nextafter(blkv, -np.inf),
                                np.where(n > 0, np.nextafter(blkv, np.inf), blkv)).astype(np.float32)
        elif kind == 1:
            blkv = np.zeros(32, np.float32)
        elif kind == 2:
            blkv = (rng.integers(-15, 16, size=32) * 2.0 ** -18).astype(np.float32)
        else:
            blkv = rng.standard_normal(32).astype(np.float32)
        xc[b, h, t, 32 * blk:32 * blk + 32] = blkv
    return xc


@pytest.mark.parametrize("center,dt", [(False, "f32"), (True, "f32"), (False, "f16"), (True, "f16")])
def test_sym4_ties_zero_blocks_and_eps_floor(center, dt):
    rng = np.random.default_rng(2024 + 2 * center + (dt == "f16"))
    B, H, T, D = 1, 2, 97, 128
    nudge = dt == "f32"
    xc = sym4_edge_keys(rng, B, H, T, D, nudge)
    if dt == "f16":
        # fp16 inputs: ties and tiny steps are fp16 values already; the
        # normal blocks are rounded
        xc = xc.astype(np.float16).astype(np.float32)
    bias = None
    x = xc
    if center:
        # bias on the 1/16 grid: x = x' + bias, and x - bias gives x' back in fp32
        bias = ((rng.integers(-40, 41, size=(H, D))) / 16).astype(np.float32)
        if dt == "f16":
            keep = np.abs(xc) >= 2.0 ** -10          # tiny steps do not survive + bias in fp16
            xc = np.where(keep, xc, 0.0).astype(np.float32)
        x = (xc + bias[None, :, None, :]).astype(np.float32)
        # tie and zero blocks survive the cast and the subtraction exactly
        # (1/16 grid); the scale checks below confirm they occur
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    q = rng.standard_normal((B, 4 * H, D)).astype(np.float32)
    flags = K.KVQ_CENTER_K if center else 0
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind="tok_sym4", k_bits=4, k_group=32,
                     v_kind="tok_affine", v_bits=8, v_group=128, in_dtype=dt, flags=flags)
    say("sym4 ties / zero blocks / eps floor", "center" if center else "plain", dt)
    xs, vs = synth.cast(x, dt), synth.cast(v, dt)
    c, o = build_pair(pl, ol, xs, vs, dt, chunks=[(0, 40), (40, T)], k_bias=bias)
    assert_same_state(c, o)
    meta = c.k_meta.cpu().numpy().view(np.uint16).reshape(B, H, T, D // 32)
    assert np.any(meta == 168) and np.any(meta == 0x3000)   # eps-floor and d = 1/8 blocks occur
    for qdt in ("f16", "bf16"):
        check_decode(pl, c, o, synth.cast(q, qdt), qdt)


def test_sym4_key_equal_to_bias_everywhere():
    """Every key equals k_bar: every block is all zero after centering, so
    every scale is fp16(1e-5) (bits 168) and every code 8 (value 0); the
    decode then sees equal logits and returns the mean of the values."""
    rng = np.random.default_rng(5)
    B, H, T, D = 2, 2, 70, 128
    bias = (rng.standard_normal((H, D)) * 1.5).astype(np.float16).astype(np.float32)
    x = np.broadcast_to(bias[None, :, None, :], (B, H, T, D)).astype(np.float32)
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, k_kind="tok_sym4", k_bits=4, k_group=32,
                     v_kind="tok_affine", v_bits=8, v_group=128, in_dtype="f16", flags=K.KVQ_CENTER_K)
    say("sym4 key == bias")
    c, o = build_pair(pl, ol, synth.cast(x, "f16"), synth.cast(v, "f16"), "f16", k_bias=bias)
    assert_same_state(c, o)
    assert np.all(c.k_meta.cpu().numpy().view(np.uint16)[:B * H * T * 4] == 168)
    codes = c.k_codes.cpu().numpy().reshape(B, H, T, D // 2)
    assert np.all(codes == 0x88)
    q = rng.standard_normal((B, 4 * H, D)).astype(np.float16)
    got, _ = check_decode(pl, c, o, q, "f16")
    vmean = o.decode(np.zeros_like(q), "f16")        # equal logits: the mean of the values
    assert attn_err(got, vmean) <= TOL


# ----------------------------------------------------------- small values

SMALL_V = [
    # (label, k layout, v bits, v group)           kernel serving it
    ("affine4 K", dict(k_kind="tok_affine", k_bits=4, k_group=64), 8, 32),    # matrix-core decode
    ("affine4 K", dict(k_kind="tok_affine", k_bits=4, k_group=64), 8, 128),
    ("affine4 K", dict(k_kind="tok_affine", k_bits=4, k_group=64), 4, 64),
    ("q4_0 K", dict(k_kind="tok_sym4", k_bits=4, k_group=32), 8, 128),
    ("kivi4 K", dict(k_kind="kivi_ch", k_bits=4, k_group=32), 8, 32),          # KIVI decode
    ("kivi4 K", dict(k_kind="kivi_ch", k_bits=4, k_group=32), 8, 128),
    ("kivi4 K", dict(k_kind="kivi_ch", k_bits=4, k_group=32), 4, 32),
    ("affine8 K", dict(k_kind="tok_affine", k_bits=8, k_group=32), 8, 32),     # generic decode
]


@pytest.mark.parametrize("sigma", [3e-3, 1e-2])
@pytest.mark.parametrize("case", range(len(SMALL_V)))
def test_decode_small_magnitude_values(case, sigma):
    label, klay, vb, vg = SMALL_V[case]
    rng = np.random.default_rng(100 + case)
    B, H, T, D, G = 1, 2, 2077, 128, 4
    k = rng.standard_normal((B, H, T, D)).astype(np.float32)
    v = (rng.standard_normal((B, H, T, D)) * sigma).astype(np.float32)
    q = rng.standard_normal((B, G * H, D)).astype(np.float32)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=D, capacity=T, v_kind="tok_affine", v_bits=vb,
                     v_group=vg, in_dtype="f16", **klay)
    say("small values", label, f"V{vb} g{vg}", f"sigma {sigma}")
    c, o = build_pair(pl, ol, synth.cast(k, "f16"), synth.cast(v, "f16"), "f16", chunks=[(0, 1000), (1000, T)])
    for qdt in ("f16", "bf16"):
        check_decode(pl, c, o, synth.cast(q, qdt), qdt)
    # sharper attention: scaled logits concentrate the weights on a few tokens
    check_decode(pl, c, o, synth.cast(q, "f16"), "f16", sm_scale=0.5)

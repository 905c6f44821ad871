"""GPU parity at the workloads' full sizes, on outputs the oracle computes one
by one: sampled (batch, kv-head) slices are regenerated from their seeded
streams, quantized by the oracle and compared bit-for-bit with the GPU cache;
their query heads' attention outputs are compared within 2e-3.  The decode
runs in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K
import synth
from oracle.cache import Layout as OLayout
from oracle.cache import OracleCache

from _gpu import assert_same_state, attn_err, say, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-3


def layout_for(w, capacity=None, flags=0):
    e = w.extra
    return K.Layout(batch=w.batch, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                    capacity=capacity or w.seq_len, k_kind=e["k_kind"], k_bits=e["k_bits"],
                    k_group=e["k_group"], v_kind="tok_affine", v_bits=e["v_bits"],
                    v_group=e["v_group"], in_dtype=w.dtype, flags=flags)


def sampled_parity(w, pl, c, out, samples, k_bias=None):
    g = w.group
    for b, h in samples:
        say("full-size sample", w.name, b, h)
        k, v, q = synth.slice_cast(w, b, h)
        ol = OLayout(batch=1, n_kv_heads=1, head_dim=pl.head_dim, capacity=pl.capacity,
                     k_kind=pl.k_kind, k_bits=pl.k_bits, k_group=pl.k_group, v_kind=pl.v_kind,
                     v_bits=pl.v_bits, v_group=pl.v_group, in_dtype=pl.in_dtype)
        o = OracleCache(ol, k_bias=None if k_bias is None else k_bias[h:h + 1])
        o.append(k[None, None], v[None, None])
        assert_same_state(c, o, bh=(b, h))
        ref = o.decode(q[None], w.dtype)[0]
        got = out[b, h * g:(h + 1) * g]
        err = attn_err(got, ref)
        say(f"  attention error {err:.3e} (tolerance {TOL:.0e})")
        assert err <= TOL, (b, h, err)


def test_affine4_g64_full_size():
    """mlx-style 4-bit g64 K and V, bf16, B=64, 32/8 heads, T=32768 (2.4 GB cache)."""
    w = synth.workload("affine4_g64")
    say("generate", w.name)
    Kh, Vh, Qh = synth.full(w, threads=16)
    pl = layout_for(w)
    c = K.Cache(pl)
    kd, vd = to_dev(Kh, "bf16"), to_dev(Vh, "bf16")
    say("quantize", w.name)
    K.kvq_quantize_append(pl, c, kd, vd)
    del kd, vd
    say("decode", w.name)
    out = K.kvq_decode_attention(pl, c, to_dev(Qh, "bf16"))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    sampled_parity(w, pl, c, out, [(0, 0), (13, 5), (40, 2), (63, 7)])


def test_q4_0_centered_full_size():
    """Symmetric 4-bit K with per-(kv-head, channel) mean-centering, int8 V,
    B=16, 32/8 heads, T=16384."""
    w = synth.workload("q4_0_centered")
    say("generate", w.name)
    Kh, Vh, Qh = synth.full(w, threads=16)
    bias = np.stack([synth.head_params(w, h)[0] for h in range(w.n_kv_heads)]).astype(np.float32)
    pl = layout_for(w, flags=K.KVQ_CENTER_K)
    c = K.Cache(pl, k_bias=torch.from_numpy(bias))
    K.kvq_quantize_append(pl, c, to_dev(Kh, "f16"), to_dev(Vh, "f16"))
    out = K.kvq_decode_attention(pl, c, to_dev(Qh, "f16"))
    torch.cuda.synchronize()
    sampled_parity(w, pl, c, out.cpu().numpy(), [(0, 0), (7, 3), (15, 7)], k_bias=bias)


def test_llama3b_kivi_int4_full_size():
    """KIVI int4 (per-channel K over 32-token groups), 24/8 heads, T=8192, with
    outlier channels; every slice and every query head checked."""
    w = synth.workload("llama3b_kivi_int4")
    Kh, Vh, Qh = synth.full(w, threads=16)
    pl = layout_for(w)
    c = K.Cache(pl)
    K.kvq_quantize_append(pl, c, to_dev(Kh, "f16"), to_dev(Vh, "f16"))
    out = K.kvq_decode_attention(pl, c, to_dev(Qh, "f16"))
    torch.cuda.synchronize()
    sampled_parity(w, pl, c, out.cpu().numpy(), [(0, h) for h in range(w.n_kv_heads)])

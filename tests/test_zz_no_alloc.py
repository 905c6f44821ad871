"""kvq_decode_attention_noalloc against kvq_decode_attention.

The no-allocation entry point runs the same kernels with the same split
plan; only the partials' buffer differs (the library's fixed per-GPU
scratch instead of a caller workspace), so its output must equal the
workspace entry point's bit for bit.  Each case makes two calls in a row,
the second with a smaller input, so the second reads a scratch that still
holds the first call's partials.  Also checked against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K

from _gpu import layouts, say, to_dev
from test_gpu_parity import TOL, build_pair, gen
import synth

pytestmark = pytest.mark.gpu

CASES = [
    # per-token 4-bit K (matrix-core decode), split over T
    dict(w="affine4_g64", lay=dict(k_kind="tok_affine", k_bits=4, k_group=64, v_kind="tok_affine", v_bits=4,
                                   v_group=64, in_dtype="bf16"), H=4, G=4,
         first=(2, 3000), second=(1, 1111)),
    # KIVI 4-bit K (VALU decode), split over T, open residual group
    dict(w="llama3b_kivi_int4", lay=dict(k_kind="kivi_ch", k_bits=4, k_group=32, v_kind="tok_affine",
                                         v_bits=4, v_group=32, in_dtype="f16"), H=8, G=3,
         first=(1, 2500), second=(1, 700)),
    # KIVI 8-bit K at head_dim 32 (LDS-tiled decode, partials always written)
    dict(w="kivi_int8_tiny", lay=dict(k_kind="kivi_ch", k_bits=8, k_group=32, v_kind="tok_affine", v_bits=8,
                                      v_group=32, in_dtype="f32"), H=8, G=1, D=32,
         first=(3, 900), second=(2, 333)),
]


def run_pair(cfg, B, T):
    w = synth.workload(cfg["w"], head_dim=cfg.get("D", 128)) if "D" in cfg else synth.workload(cfg["w"])
    H, G = cfg["H"], cfg["G"]
    k, v, q = gen(w, B, H, T, Hq=H * G)
    pl, ol = layouts(batch=B, n_kv_heads=H, head_dim=w.head_dim, capacity=T, **cfg["lay"])
    c, o = build_pair(pl, ol, k, v, w.dtype, chunks=[(0, T // 3), (T // 3, T)])
    qd = to_dev(q, w.dtype)
    ref = K.kvq_decode_attention(pl, c, qd).cpu().numpy()
    got = K.kvq_decode_attention_noalloc(pl, c, qd)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    ora = o.decode(q, w.dtype)
    err = float((np.abs(got.astype(np.float64) - ora) / np.abs(ora).max(-1, keepdims=True)).max())
    say(f"  noalloc vs oracle {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("i", range(len(CASES)))
def test_noalloc_decode_equals_workspace_decode(i):
    cfg = CASES[i]
    for B, T in (cfg["first"], cfg["second"]):
        say("noalloc decode", cfg["w"], cfg["lay"]["k_kind"], f"B={B} T={T}")
        run_pair(cfg, B, T)


def test_noalloc_rejects_beyond_scratch_and_empty_cache():
    """Partials beyond the fixed scratch: KVQ_ERR_SCRATCH before any launch;
    an empty cache decodes to zeros."""
    pl, _ = layouts(batch=4096, n_kv_heads=8, head_dim=128, capacity=64, k_kind="kivi_ch", k_bits=8,
                    k_group=32, v_kind="tok_affine", v_bits=8, v_group=128, in_dtype="f16")
    c = K.Cache(pl)
    x = torch.zeros(4096, 8, 40, 128, device="cuda", dtype=torch.float16)
    K.kvq_quantize_append(pl, c, x, x)
    q = torch.zeros(4096, 64, 128, device="cuda", dtype=torch.float16)
    say("noalloc rejects beyond scratch")
    with pytest.raises(K.KvqError) as e:
        K.kvq_decode_attention_noalloc(pl, c, q)
    assert e.value.status == K.KVQ_ERR_SCRATCH
    pe, _ = layouts(batch=2, n_kv_heads=2, head_dim=64, capacity=10, in_dtype="f16", k_group=64, v_group=64)
    ce = K.Cache(pe)
    out = torch.full((2, 4, 64), 3.0, device="cuda")
    K.kvq_decode_attention_noalloc(pe, ce, torch.randn(2, 4, 64, device="cuda", dtype=torch.float16), out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0

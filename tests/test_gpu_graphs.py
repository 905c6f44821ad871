"""Decode attention (split partials and their combine) and multi-query
attention captured in a HIP graph: replays over changing queries, with eager
work between them, give the same bits as eager calls on the same inputs
(the kernels clear nothing by memset, so a replay depends on nothing a
previous replay left in the workspace)."""
import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K
import synth

from _gpu import layouts, say, to_dev

pytestmark = pytest.mark.gpu


def build_cache(kw, T, seed):
    w = synth.workload("affine4_g64", head_dim=128, seq_len=T, batch=kw["batch"],
                       n_kv_heads=kw["n_kv_heads"], n_q_heads=4 * kw["n_kv_heads"], dtype="bf16")
    k, v, _ = synth.full(w, threads=8)
    L, _ = layouts(capacity=T, **kw)
    c = K.Cache(L)
    K.kvq_quantize_append(L, c, to_dev(k, "bf16"), to_dev(v, "bf16"))
    torch.cuda.synchronize()
    return L, c


def queries(shape, seeds):
    return [to_dev(synth.cast(np.random.default_rng([0, 801, s]).standard_normal(shape, dtype=np.float32),
                              "bf16"), "bf16") for s in seeds]


KW = dict(batch=2, n_kv_heads=2, head_dim=128, k_kind="tok_affine", k_bits=4, k_group=64,
          v_kind="tok_affine", v_bits=4, v_group=64, in_dtype="bf16")


def test_decode_graph_replays():
    """Batch 2 x 2 kv-heads over 5000 slots: the plan splits T, so a call is
    the decode launch plus the split combine."""
    L, c = build_cache(KW, 5000, 1)
    Hq = 8
    qs = queries((2, Hq, 128), range(4))
    q = qs[0].clone()
    out = torch.empty((2, Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(K.kvq_decode_workspace_bytes(L, Hq), 16), dtype=torch.uint8, device="cuda")
    K.kvq_decode_attention(L, c, q, out=out, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvq_decode_attention(L, c, q, out=out, ws=ws)
    for rep in range(6):
        qi = qs[rep % 4]
        q.copy_(qi)
        ref = K.kvq_decode_attention(L, c, qi.clone()).clone()     # eager, its own workspace
        torch.cuda.synchronize()
        say("decode graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), rep


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_attention_graph_replays(causal):
    """64 queries per head (4 query heads per kv-head) over 3000 slots: the
    multi-query launch over token splits plus the fp16 split combine."""
    L, c = build_cache(KW, 3000, 2)
    Hq, n_q = 8, 64
    qs = queries((2, Hq, n_q, 128), range(10, 13))
    q = qs[0].clone()
    out = torch.empty((2, Hq, n_q, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(K.kvq_prefill_workspace_bytes(L, Hq, n_q), 16), dtype=torch.uint8, device="cuda")
    K.kvq_prefill_attention(L, c, q, causal=causal, out=out, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvq_prefill_attention(L, c, q, causal=causal, out=out, ws=ws)
    for rep in range(5):
        qi = qs[rep % 3]
        q.copy_(qi)
        ref = K.kvq_prefill_attention(L, c, qi.clone(), causal=causal).clone()
        torch.cuda.synchronize()
        say("prefill attention graph replay", causal, rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), rep

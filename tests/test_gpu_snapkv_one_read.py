"""The one-read SnapKV scores ([P2] "How it works", step 1): each workgroup
keeps its key chunk's logits in registers while the chunks of a head exchange
their softmax row statistics, and the select launch clears the exchange
flags.  Its numerics against the fp64 oracle are covered by
test_gpu_snapkv.py (every shape there with S <= 32768 and at most 4096 kept
rows takes this path).  Here:

* a workgroup that stops waiting recomputes its head's statistics with the
  same code: with the wait bound at 0 the outputs are the same bits;
* the flags are cleared between calls: repeated calls on one workspace, and
  a captured graph replayed over changing inputs, match fresh eager calls.
"""
import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K

from _gpu import say, to_dev
from test_gpu_snapkv import gen_kv, gen_q

pytestmark = pytest.mark.gpu


def run(k, v, w, sink, budget, q=None, ws=None, outs=None):
    B, H, S, D = k.shape
    if q is None and ws is None and outs is None:
        return [t.clone() for t in K.kvq_snapkv_select(k, v, w, sink, budget)]
    if q is None:
        sc, kept, ko, vo = outs if outs else (None,) * 4
        return K.kvq_snapkv_select(k, v, w, sink, budget, scores=sc, kept=kept, k_out=ko, v_out=vo, ws=ws)
    return [t.clone() for t in K.kvq_snapkv_select_ex(k, v, w, sink, budget, q_window=q)]


def same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("B,H,S,D,w,sink,budget,G", [
    (1, 8, 8192, 128, 32, 4, 512, 0),       # the page's defaults: 32 chunks of 256 keys per head
    (2, 3, 300, 64, 16, 4, 40, 0),          # ragged last chunk
    (1, 2, 1000, 128, 64, 4, 100, 0),       # two row tiles, chunks of 128 keys
    (1, 2, 777, 64, 16, 4, 60, 8),          # 128 query rows per kv-head
    (1, 1, 129, 32, 8, 0, 64, 0),           # one key past the first chunk
])
def test_late_workgroups_give_the_same_bits(B, H, S, D, w, sink, budget, G):
    k, v = gen_kv(B, H, S, D, seed=S + w)
    kd, vd = to_dev(k, "f16"), to_dev(v, "f16")
    q = to_dev(gen_q(B, H, G, w, D, seed=S), "f16") if G else None
    say("one-read late path", B, H, S, D, w, sink, budget, G)
    ref = run(kd, vd, w, sink, budget, q)
    prev = K.kvq_snapkv_set_wait_us(0)
    try:
        late = run(kd, vd, w, sink, budget, q)
        torch.cuda.synchronize()
    finally:
        K.kvq_snapkv_set_wait_us(prev)
    assert prev == 200
    assert same(ref, late)


def test_repeated_calls_on_one_workspace():
    B, H, S, D, w, sink, budget = 1, 4, 3000, 128, 32, 4, 256
    ins = [gen_kv(B, H, S, D, seed=s) for s in (1, 2)]
    dev = [(to_dev(k, "f16"), to_dev(v, "f16")) for k, v in ins]
    ref = [run(kd, vd, w, sink, budget) for kd, vd in dev]
    assert not torch.equal(ref[0][0], ref[1][0])
    ws = torch.empty(K.kvq_snapkv_workspace_bytes(B, H, S, D, w), dtype=torch.uint8, device="cuda")
    for i in (0, 1, 0, 1, 1, 0):
        say("one-read repeated call, input", i)
        got = run(*dev[i], w, sink, budget, ws=ws)
        assert same(got, ref[i])


def test_graph_replays_over_changing_inputs():
    B, H, S, D, w, sink, budget = 1, 8, 4096, 128, 32, 4, 300
    srcs = [gen_kv(B, H, S, D, seed=10 + s) for s in range(3)]
    kd, vd = to_dev(srcs[0][0], "f16"), to_dev(srcs[0][1], "f16")
    n_keep = min(budget, S)
    outs = (torch.empty((B, H, S), dtype=torch.float32, device="cuda"),
            torch.empty((B, H, n_keep), dtype=torch.int32, device="cuda"),
            torch.empty((B, H, n_keep, D), dtype=torch.float16, device="cuda"),
            torch.empty((B, H, n_keep, D), dtype=torch.float16, device="cuda"))
    ws = torch.empty(K.kvq_snapkv_workspace_bytes(B, H, S, D, w), dtype=torch.uint8, device="cuda")
    run(kd, vd, w, sink, budget, ws=ws, outs=outs)       # eager first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(kd, vd, w, sink, budget, ws=ws, outs=outs)
    for rep in range(6):
        k, v = srcs[rep % 3]
        kd.copy_(to_dev(k, "f16"))
        vd.copy_(to_dev(v, "f16"))
        torch.cuda.synchronize()
        say("one-read graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        ref = run(kd.clone(), vd.clone(), w, sink, budget)
        torch.cuda.synchronize()
        assert same(got, ref), rep

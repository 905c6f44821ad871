"""GPU parity for SnapKV prefill selection ([P2] "How it works").

* Scores (MFMA logits, fp32 softmax, window mean) against the fp64 oracle:
  |s - s_ref| <= 1e-4 s_ref + 1e-12, and each head's scores sum to 1.
* Selection from given scores: bit-exact against the oracle (same fp32 input,
  ties broken by the lower position).
* End to end the kept sets may differ only where the oracle's scores are
  within twice the score tolerance of its selection threshold (fp32 versus
  fp64 near-ties); the gathered rows are exactly the kept rows.
"""
import numpy as np
import pytest
import torch

import evicted_kv_cache_amd as K
import oracle
import synth
from oracle.cache import snapkv as oracle_snapkv

from _gpu import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def tol(s):
    return 1e-4 * np.abs(s) + 1e-12


def gen_kv(B, H, S, D, seed):
    w = synth.workload("snapkv_prefill", batch=B, n_kv_heads=H, n_q_heads=H, seq_len=S,
                       head_dim=D, config_id=300 + seed)
    k = np.empty((B, H, S, D), np.float16)
    v = np.empty((B, H, S, D), np.float16)
    for b in range(B):
        for h in range(H):
            k[b, h], v[b, h], _ = synth.slice_cast(w, b, h)
    return k, v


def check_end_to_end(k, v, w, sink, budget):
    B, H, S, D = k.shape
    say("snapkv", B, H, S, D, w, sink, budget)
    sc, kept, ko, vo = K.kvq_snapkv_select(to_dev(k, "f16"), to_dev(v, "f16"), w, sink, budget)
    torch.cuda.synchronize()
    sc, kept, ko, vo = (t.cpu().numpy() for t in (sc, kept, ko, vo))
    ref_sc, ref_kept, _, _ = oracle_snapkv(k, v, w, sink, budget)
    n_keep = min(budget, S)
    n_s = min(sink, n_keep)
    assert kept.shape == (B, H, n_keep) and ko.shape == (B, H, n_keep, D) and ko.dtype == np.float16
    assert np.all(np.abs(sc - ref_sc) <= tol(ref_sc)), np.abs(sc - ref_sc).max()
    assert np.all(np.abs(sc.astype(np.float64).sum(-1) - 1) <= 1e-5)
    assert sc.min() >= 0 and sc.max() <= 1
    for b in range(B):
        for h in range(H):
            g, r = kept[b, h], ref_kept[b, h]
            assert np.all(np.diff(g) > 0), "kept positions ascending"
            assert np.array_equal(g[:n_s], np.arange(n_s)), "sinks always kept"
            s = ref_sc[b, h]
            diff = np.setxor1d(g, r)
            if diff.size:
                cand = r[n_s:]
                thr = s[cand].min()
                assert np.all(np.abs(s[diff] - thr) <= 2 * tol(thr)), (b, h, diff, s[diff], thr)
                assert s[g].sum() >= s[r].sum() - diff.size * 2 * tol(thr)
            assert np.array_equal(ko[b, h], k[b, h, g])
            assert np.array_equal(vo[b, h], v[b, h, g])
    return sc, kept


def test_snapkv_defaults_full_size():
    """The SnapKV page's defaults (budget 512, window 32, sink 4) at S = 8192,
    8 kv-heads x 128, fp16 keys ~ N(0,1)."""
    w = synth.workload("snapkv_prefill")
    k, v, _ = synth.full(w, threads=16)
    e = w.extra
    check_end_to_end(k, v, e["obs_window"], e["n_sink"], e["budget"])


@pytest.mark.parametrize("B,H,S,D,w,sink,budget", [
    (2, 3, 300, 64, 16, 4, 40),       # ragged chunk tail
    (1, 2, 20, 128, 32, 4, 8),        # obs_window > S (clamped)
    (1, 2, 50, 32, 8, 4, 512),        # budget >= S keeps everything
    (1, 2, 100, 64, 8, 30, 10),       # n_sink > budget
    (1, 2, 129, 64, 128, 0, 64),      # no sinks, widest window, one key past a chunk
    (1, 1, 1, 64, 4, 4, 4),           # a single key
    (3, 2, 1000, 128, 64, 4, 100),    # two MFMA row tiles
    (1, 2, 10000, 128, 32, 4, 512),   # stats: 2 chunks of 128 keys per workgroup
    (1, 1, 20000, 64, 40, 4, 512),    # stats: 4 chunks per workgroup, two row tiles
    (1, 1, 40000, 32, 16, 4, 512),    # stats: two steps of 4 chunks; radix select
])
def test_snapkv_edge_shapes(B, H, S, D, w, sink, budget):
    k, v = gen_kv(B, H, S, D, seed=S + D + w)
    check_end_to_end(k, v, w, sink, budget)


def test_snapkv_identical_keys_keep_the_first_positions():
    k = np.repeat(gen_kv(1, 2, 1, 64, 5)[0], 200, axis=2)
    v = gen_kv(1, 2, 200, 64, 6)[1]
    sc, kept, _, _ = K.kvq_snapkv_select(to_dev(k, "f16"), to_dev(v, "f16"), 8, 4, 30)
    assert torch.allclose(sc, torch.full_like(sc, 1 / 200), rtol=1e-5, atol=0)
    assert np.array_equal(kept.cpu().numpy()[0, 0], np.arange(30))


@pytest.mark.parametrize("S,sink,budget,levels", [
    (8192, 4, 512, 7),        # heavy ties at the threshold
    (8192, 4, 512, 0),        # continuous scores
    (3000, 0, 1, 3),
    (5000, 17, 4999, 5),
    (777, 4, 100, 1),         # all candidates tie
    (8193, 4, 512, 0),        # 16 keys per thread
    (12000, 4, 700, 5),
    (16384, 4, 512, 0),
    (20000, 4, 512, 0),       # 32 keys per thread
    (20000, 0, 1000, 9),
    (20001, 4, 512, 0),       # 32 keys per thread, 4-byte loads
    (32768, 4, 512, 3),
    (40000, 4, 512, 0),       # radix select over global keys
    (40001, 0, 1000, 9),
])
def test_select_from_scores_bit_exact(S, sink, budget, levels):
    rng = np.random.default_rng(S + budget + levels)
    B, H = 2, 3
    if levels:
        sc = (rng.integers(0, levels, (B, H, S)) / 8).astype(np.float32)
    else:
        sc = rng.random((B, H, S)).astype(np.float32)
    sc[0, 0, :5] = -0.0                       # signed zeros rank as +0
    sc[1, 2, 10:20] = -1.0                    # negative scores are ordered too
    say("select_from_scores", S, sink, budget, levels)
    kept = K.kvq_snapkv_select_from_scores(to_dev(sc, "f32"), sink, budget).cpu().numpy()
    for b in range(B):
        for h in range(H):
            ref = oracle.snapkv_select(np.where(sc[b, h] == 0, np.float32(0), sc[b, h]), sink, budget)
            assert np.array_equal(kept[b, h], ref), (b, h)


# ---- SnapKV with the prompt's own queries and max-pool smoothing -----------
# (the paper's scoring, which the SnapKV page replaces by the key proxy:
# [P2] "Proxy limitation").  Readings: a kv-head's score is the mean over the
# G * w query rows of its group; pooling clips at the sequence ends and only
# ranks, the returned scores stay unpooled.

def gen_q(B, H, G, w, D, seed):
    wl = synth.workload("snapkv_prefill", batch=B, n_kv_heads=H, n_q_heads=H * G, head_dim=D,
                        config_id=400 + seed)
    q = np.empty((B, H * G, w, D), np.float16)
    for b in range(B):
        for h in range(H):
            q[b, h * G:(h + 1) * G] = synth.query_window(wl, b, h, w)
    return q


def oracle_snapkv_ex(k, q, w, sink, budget, pool):
    """(scores fp64, ranking scores fp32, kept) per the oracle; q None = key proxy."""
    B, H, S, D = k.shape
    sc = np.zeros((B, H, S))
    rank = np.zeros((B, H, S), np.float32)
    kept = np.zeros((B, H, min(budget, S)), np.int32)
    for b in range(B):
        for h in range(H):
            kk = k[b, h].astype(np.float32)
            if q is None:
                rows = kk[S - min(w, S):]
            else:
                G = q.shape[1] // H
                rows = q[b, h * G:(h + 1) * G].reshape(G * w, D).astype(np.float32)
            sc[b, h] = oracle.snapkv_scores_rows(rows, kk)
            r = sc[b, h].astype(np.float32)
            rank[b, h] = oracle.maxpool1d(r, pool) if pool > 1 else r
            kept[b, h] = oracle.snapkv_select(rank[b, h], sink, budget)
    return sc, rank, kept


def check_ex(k, v, q, w, sink, budget, pool):
    B, H, S, D = k.shape
    say("snapkv_ex", B, H, S, D, None if q is None else q.shape[1], w, sink, budget, pool)
    qd = None if q is None else to_dev(q, "f16")
    sc, kept, ko, vo = K.kvq_snapkv_select_ex(to_dev(k, "f16"), to_dev(v, "f16"), w, sink, budget,
                                              q_window=qd, pool_kernel=pool)
    torch.cuda.synchronize()
    sc, kept, ko, vo = (t.cpu().numpy() for t in (sc, kept, ko, vo))
    ref_sc, ref_rank, ref_kept = oracle_snapkv_ex(k, q, w, sink, budget, pool)
    n_s = min(sink, min(budget, S))
    assert np.all(np.abs(sc - ref_sc) <= tol(ref_sc)), np.abs(sc - ref_sc).max()
    assert np.all(np.abs(sc.astype(np.float64).sum(-1) - 1) <= 1e-5)
    n_diff = 0
    for b in range(B):
        for h in range(H):
            g, r = kept[b, h], ref_kept[b, h]
            assert np.all(np.diff(g) > 0) and np.array_equal(g[:n_s], np.arange(n_s))
            s = ref_rank[b, h].astype(np.float64)
            diff = np.setxor1d(g, r)
            n_diff += diff.size
            if diff.size:
                thr = s[r[n_s:]].min()
                assert np.all(np.abs(s[diff] - thr) <= 2 * tol(thr)), (b, h, diff, s[diff], thr)
            assert np.array_equal(ko[b, h], k[b, h, g])
            assert np.array_equal(vo[b, h], v[b, h, g])
    say("snapkv_ex kept-set differences (near-ties):", n_diff)
    return sc, kept


@pytest.mark.parametrize("B,H,G,S,D,w,sink,budget,pool", [
    (2, 2, 4, 1000, 128, 16, 4, 100, 1),      # GQA group of 4: 64 rows per kv-head
    (1, 2, 8, 777, 64, 16, 4, 60, 7),         # 128 rows, pooled
    (1, 3, 1, 50, 32, 8, 2, 20, 31),          # pool wider than half the prompt
    (2, 1, 2, 129, 128, 1, 0, 16, 3),         # one query per head, ragged chunk
    (1, 2, 3, 5, 64, 5, 1, 3, 5),             # window = whole prompt
])
def test_snapkv_query_window(B, H, G, S, D, w, sink, budget, pool):
    k, v = gen_kv(B, H, S, D, seed=S + G)
    q = gen_q(B, H, G, w, D, seed=S + D)
    check_ex(k, v, q, w, sink, budget, pool)


@pytest.mark.parametrize("S,D,w,sink,budget,pool", [
    (300, 64, 16, 4, 40, 7),
    (1000, 128, 64, 4, 100, 31),
    (20, 128, 32, 4, 8, 3),                   # window clamps to S
])
def test_snapkv_proxy_pooled(S, D, w, sink, budget, pool):
    k, v = gen_kv(2, 2, S, D, seed=S + pool)
    check_ex(k, v, None, w, sink, budget, pool)


def test_snapkv_query_window_full_size():
    """SnapKV defaults (S = 8192, 8 kv-heads x 128, window 32, sink 4, budget
    512) scored by 32 query heads (G = 4: 128 rows per kv-head), pooled over 7."""
    wl = synth.workload("snapkv_prefill")
    k, v, _ = synth.full(wl, threads=16)
    q = gen_q(1, 8, 4, 32, 128, seed=0)
    e = wl.extra
    check_ex(k, v, q, e["obs_window"], e["n_sink"], e["budget"], 7)


def test_snapkv_key_rows_as_queries_match_proxy():
    """Passing the last w key rows as a G = 1 query window reproduces the proxy exactly."""
    k, v = gen_kv(2, 3, 1500, 128, seed=77)
    w = 32
    kd, vd = to_dev(k, "f16"), to_dev(v, "f16")
    q = kd[:, :, -w:, :].contiguous()
    say("snapkv_ex key rows as queries")
    a = K.kvq_snapkv_select(kd, vd, w, 4, 200)
    b = K.kvq_snapkv_select_ex(kd, vd, w, 4, 200, q_window=q)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("S,pool,levels", [
    (1, 3, 0), (5, 31, 0), (300, 3, 4), (1000, 7, 0), (8192, 7, 6), (8193, 31, 0), (777, 1, 0),
])
def test_pool_scores_bit_exact(S, pool, levels):
    rng = np.random.default_rng(S * 31 + pool)
    B, H = 2, 3
    if levels:
        sc = (rng.integers(0, levels, (B, H, S)) / 8).astype(np.float32)
    else:
        sc = rng.random((B, H, S)).astype(np.float32)
    say("pool_scores", S, pool, levels)
    out = K.kvq_snapkv_pool_scores(to_dev(sc, "f32"), pool).cpu().numpy()
    for b in range(B):
        for h in range(H):
            assert np.array_equal(out[b, h], oracle.maxpool1d(sc[b, h], pool)), (b, h)

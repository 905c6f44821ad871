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
    (20000, 4, 512, 0),       # radix select over global keys
    (20000, 0, 1000, 9),
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

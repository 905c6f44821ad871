#!/usr/bin/env python3
"""Benchmark of the compressed-KV decode path on one MI355X.

A timed step is one decode-attention call over the whole batch of the
headline workload (mlx-style 4-bit affine g64 K and V, bf16, batch 64,
32 query / 8 kv heads x 128, T = 32768): every cached byte is read once.
The other rows of the hot path are timed in the same run on their own
workloads and reported under "rows":
  A  quantize-on-write: prefill of the whole cache (n_new = T) and the
     per-step append of one token per sequence
  C  StreamingLLM compaction of the headline cache to sink 4 + window 16380
  D  SnapKV prefill selection (8 kv-heads x 128, S = 8192, window 32,
     sink 4, budget 512): scores/s
  B  decode on the other cache formats: Q4_0-style centered K + int8 V
     (batch 16, T = 16384), a KIVI int4 Llama-3.2-3B layer (T = 8192) and
     the same layer shape at batch 16, T = 16384
  E  multi-query (prefill-chunk) attention: 128 causal queries per head,
     32 / 8 heads x 128, T = 2048 and 32768 (matrix-core bound)
Inputs are seeded synthetic data (synth) already resident in HBM when the
timed region starts.  Times come from HIP events on the stream the kernels
run on; every row other than the step is the median of five trials.  The
CPU oracle is timed on a bounded sample as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps 300] [--warmup 200] [--no-cpu-baseline]
                       [--rows ACDBE] [--e-lengths 2048,32768]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0      # dense fp16 matrix-core peak
# source of the kernel the step launches (the traffic counters are only
# reported while they were taken on this source)
DECODE_SRC = os.path.join(ROOT, "evicted_kv_cache_amd", "csrc", "decode_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_affine4_g64_traffic.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_algorithmic_bytes(B, Hkv, Hq, D, T, bits, group, q_bytes=2):
    """Bytes a decode step must move: K and V codes and (scale, zero) fp16 per
    group for T slots, the queries, and the fp32 outputs."""
    per_token_head = 2 * (D * bits // 8 + (D // group) * 4)
    return B * Hkv * T * per_token_head + B * Hq * D * q_bytes + B * Hq * D * 4


MALL_BYTES = 256 << 20
ROTATE_BYTES = 512 << 20           # input copies cycled by the cold timings: twice the MALL
# Sustained load: for the first tens of ms of heavy work after an idle spell
# the power manager pulls the shader clock down (on an MI355X under the decode:
# 2.4 GHz to about 1.1 GHz within 5 ms, back to about 2.2 GHz after some 40 ms,
# flat from then on), so every row first runs its own work untimed for
# SUSTAIN_MS of device time and is then timed over at least MIN_TIMED_MS.
SUSTAIN_MS = 80.0
MIN_TIMED_MS = 30.0


def time_rotating(fns, reps, torch):
    """Per-call ms of calls whose inputs are distinct copies (fns[i] reads copy
    i), replayed from one captured HIP graph: a copy comes round again only
    after ROTATE_BYTES (> 2x the 256 MB MALL) of other inputs were read, so
    each call reads its inputs from HBM ("cold")."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    ms = time_stream(g.replay, reps, 2, torch) / len(fns)
    LAST_TRIALS[:] = [t / len(fns) for t in LAST_TRIALS]
    del g
    return ms


def n_copies(nbytes):
    return max(2, math.ceil(ROTATE_BYTES / nbytes))


def host_cpu():
    """(os.cpu_count(), CPUs this process may run on, /proc/cpuinfo model name)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return os.cpu_count() or 1, avail, model


def sustain(fn, torch, ms_min=SUSTAIN_MS):
    """Run fn untimed until at least ms_min of device time has passed; return
    the last batch's ms per call."""
    s = torch.cuda.current_stream()
    done, n, per = 0.0, 1, 0.0
    while done < ms_min:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(n):
            fn()
        b.record(s)
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        done += t
        per = t / n
        n = min(2 * n, 4096)
    return per


TRIALS = 5
LAST_TRIALS = []                   # ms per call of each trial of the last time_stream


def time_stream(fn, steps, warmup, torch, sustain_ms=SUSTAIN_MS, min_timed_ms=MIN_TIMED_MS):
    """Median over TRIALS trials of the average ms per call of fn, with HIP
    events on the current stream: `warmup` calls, then sustain_ms of device
    time untimed, then TRIALS trials of max(steps, as many as fill
    min_timed_ms) timed calls each (the trials are kept in LAST_TRIALS)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    per = sustain(fn, torch, sustain_ms) if sustain_ms > 0 else 0.0
    if per > 0:
        steps = max(steps, math.ceil(min_timed_ms / per))
    s = torch.cuda.current_stream()
    trials = []
    for _ in range(TRIALS):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(s)
        for _ in range(steps):
            fn()
        end.record(s)
        torch.cuda.synchronize()
        trials.append(start.elapsed_time(end) / steps)
    LAST_TRIALS[:] = trials
    return sorted(trials)[TRIALS // 2]


def trials_note(scale):
    """The last time_stream's trials, times scale (e.g. 1e3 for us per call)."""
    return [round(t * scale, 4) for t in LAST_TRIALS]


def time_steps(fn, steps, warmup, torch):
    """The timed step: exactly `warmup` untimed calls (each bracketed by events,
    so the clock's settling shows), then exactly `steps` timed calls. Returns
    (ms per timed call, ms of each warm-up call)."""
    s = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(warmup + 1)]
    evs[0].record(s)
    for i in range(warmup):
        fn()
        evs[i + 1].record(s)
    torch.cuda.synchronize()
    warm = [evs[i].elapsed_time(evs[i + 1]) for i in range(warmup)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(steps):
        fn()
    end.record(s)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, warm


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(path=TRAFFIC_FILE, src=DECODE_SRC):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source. The sum over the file's kernels
    when it holds several (one launch of each per call)."""
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_sha256_16") != source_hash(src):
        return None
    return t.get("bytes_per_launch") or sum(k["bytes_per_launch"] for k in t["kernels"].values())


def cpu_baseline(w, target_s=12.0):
    """Time the CPU oracle's decode on a bounded sample of (batch, kv-head) slices."""
    import numpy as np

    import synth
    from oracle.cache import Layout as OLayout
    from oracle.cache import OracleCache

    host_cpus, avail, model = host_cpu()
    threads = max(1, min(16, avail))
    e = w.extra

    def slice_cache(b, h):
        k, v, q = synth.slice_cast(w, b, h)
        ol = OLayout(batch=1, n_kv_heads=1, head_dim=w.head_dim, capacity=w.seq_len,
                     k_kind=e["k_kind"], k_bits=e["k_bits"], k_group=e["k_group"],
                     v_kind="tok_affine", v_bits=e["v_bits"], v_group=e["v_group"], in_dtype=w.dtype)
        o = OracleCache(ol)
        o.append(k[None, None], v[None, None])
        return o, q[None]

    # probe one slice to size the sample
    o, q = slice_cache(0, 0)
    t0 = time.perf_counter()
    o.decode(q, w.dtype, threads=1)
    one = time.perf_counter() - t0          # single-thread seconds per kv-head slice (4 q-heads)
    n = max(threads, int(target_s * threads / max(one, 1e-3)))
    n = min(n, w.batch * w.n_kv_heads)
    slices = [(i // w.n_kv_heads, i % w.n_kv_heads) for i in range(n)]
    caches = [slice_cache(b, h) for b, h in slices]
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda oc: oc[0].decode(oc[1], w.dtype, threads=1), caches))
    dt = time.perf_counter() - t0
    per_slice = decode_algorithmic_bytes(1, 1, w.group, w.head_dim, w.seq_len, e["k_bits"], e["k_group"])
    nbytes = per_slice * n
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single_thread_value": round(per_slice / one / 1e9, 5),
            "host_cpus": host_cpus, "cpus_available": avail, "cpu_model": model,
            "sample": f"{n} of {w.batch * w.n_kv_heads} (batch, kv-head) slices of the headline "
                      f"workload ({n * w.group} query heads over T={w.seq_len}), fp64 decode, "
                      f"{dt:.1f} s wall on {threads} threads (one thread: {one:.2f} s per slice)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (about 75 ms of decode: the clock has settled)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows", default="ACDBE", help="extra rows to time (subset of ACDBE)")
    ap.add_argument("--e-lengths", default="2048,32768",
                    help="cache lengths of row E (comma-separated; one length gives its own counters)")
    ap.add_argument("--mode", default="full", choices=["full", "decode", "copy"],
                    help="decode: only the timed decode steps (for counter runs); "
                         "copy: a plain 2 GiB device copy (bandwidth probe / counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import evicted_kv_cache_amd as K
    import synth

    dev = "cuda"
    if args.mode == "copy":
        n = 1 << 31
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms = time_stream(lambda: dst.copy_(src), args.steps, args.warmup, torch)
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                          "ms": round(ms, 4), "GB/s": round(2 * n / ms / 1e6, 1)}), flush=True)
        return
    if args.mode == "decode":
        args.rows = ""
        args.no_cpu_baseline = True
    w = synth.workload("affine4_g64")
    e = w.extra
    B, Hkv, Hq, D, T = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.seq_len
    log("generating", w.name)
    t0 = time.time()
    Kh, Vh, Qh = synth.full(w, threads=max(1, min(16, os.cpu_count() or 1)))
    log(f"generated in {time.time() - t0:.1f}s")

    def bf16(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    L = K.Layout(batch=B, n_kv_heads=Hkv, head_dim=D, capacity=T, k_kind=e["k_kind"],
                 k_bits=e["k_bits"], k_group=e["k_group"], v_kind="tok_affine",
                 v_bits=e["v_bits"], v_group=e["v_group"], in_dtype="bf16")
    cache = K.Cache(L)
    kd, vd = bf16(Kh), bf16(Vh)
    q = bf16(Qh)
    del Kh, Vh
    rows = {}

    # ---- row A: prefill quantize-on-write (n_new = T) into an emptied cache
    if "A" in args.rows:
        def prefill():
            K.kvq_cache_reset(cache)               # host counters only: an empty cache
            K.kvq_quantize_append(L, cache, kd, vd)
        ms = time_stream(prefill, 1, 1, torch)
        trials_a = trials_note(1.0)
        nbytes = 2 * kd.numel() * 2 + 2 * (cache.sizes.k_codes + cache.sizes.k_meta) + T * 4
        rows["A_quantize_prefill"] = {"workload": f"{w.name} prefill n_new={T}", "ms": round(ms, 4),
                                      "trials_ms": trials_a,
                                      "GB/s": round(nbytes / ms / 1e6, 1),
                                      "frac_hbm": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}
    else:
        K.kvq_quantize_append(L, cache, kd, vd)
    torch.cuda.synchronize()
    del kd, vd

    # ---- row B (the step): decode attention over the full cache
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(K.kvq_decode_workspace_bytes(L, Hq), 16), dtype=torch.uint8, device=dev)

    def step():
        K.kvq_decode_attention(L, cache, q, out=out, ws=ws)

    log("timing decode")
    ms, warm = time_steps(step, args.steps, args.warmup, torch)
    nbytes = decode_algorithmic_bytes(B, Hkv, Hq, D, T, e["k_bits"], e["k_group"])
    gbs = nbytes / ms / 1e6
    log(f"decode {ms * 1e3:.1f} us/step  {gbs:.1f} GB/s  {gbs / PEAK_HBM_GBS:.3f} of HBM peak")
    traffic = load_traffic()

    # ---- row A (decode-time append of one token per sequence) on a cache with room
    if "A" in args.rows:
        L1 = K.Layout(**{**L.__dict__, "capacity": 4096})
        c1 = K.Cache(L1)
        one_k = torch.randn(B, Hkv, 1, D, device=dev).to(torch.bfloat16)
        ms1 = time_stream(lambda: (K.kvq_cache_reset(c1) if c1.n_stored >= 4000 else None,
                                   K.kvq_quantize_append(L1, c1, one_k, one_k)), 200, 10, torch)
        # device time per append: 64 appends captured in one HIP graph and
        # replayed, so host marshalling is out of the timed region
        K.kvq_cache_reset(c1)
        n_cap = 64
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_cap):
                K.kvq_quantize_append(L1, c1, one_k, one_k)
        msg = time_stream(g.replay, 20, 3, torch) / n_cap
        rows["A_append_one_token"] = {"workload": f"{w.name} append n_new=1 (B={B}, Hkv={Hkv})",
                                      "us": round(msg * 1e3, 2),
                                      "us_host_inclusive": round(ms1 * 1e3, 2)}
        del g

    # ---- row C: StreamingLLM compaction of the headline cache
    if "C" in args.rows:
        dst = K.Cache(L)
        sink, window = 4, T // 2 - 4
        def evict():
            st = K.kvq_evict_streaming(L, cache, dst, sink, window)
            assert st == K.KVQ_OK
        msc = time_stream(evict, 10, 2, torch)
        trials_c = trials_note(1.0)
        row_bytes = 2 * (D * e["k_bits"] // 8 + (D // e["k_group"]) * 4)
        cbytes = 2 * B * Hkv * (sink + window) * row_bytes + 2 * (sink + window) * 4
        rows["C_evict"] = {"workload": f"{w.name} T={T} -> sink {sink} + window {window}",
                           "ms": round(msc, 4), "trials_ms": trials_c,
                           "GB/s": round(cbytes / msc / 1e6, 1),
                           "frac_hbm": round(cbytes / msc / 1e6 / PEAK_HBM_GBS, 4),
                           "algorithmic_bytes": cbytes,
                           "traffic": load_traffic(
                               os.path.join(ROOT, "profiles", "evict_gather_affine4_g64_traffic.json"),
                               os.path.join(ROOT, "evicted_kv_cache_amd", "csrc", "evict.hip"))}
        del dst

    # ---- row D: SnapKV prefill selection
    if "D" in args.rows:
        ws_ = synth.workload("snapkv_prefill")
        ks, vs, _ = synth.full(ws_, threads=16)
        ksd = torch.from_numpy(ks).to(dev)
        vsd = torch.from_numpy(vs).to(dev)
        ex = ws_.extra
        Bs, Hs, Ss, Ds = ks.shape
        n_keep = min(ex["budget"], Ss)
        sc = torch.empty((Bs, Hs, Ss), dtype=torch.float32, device=dev)
        kept = torch.empty((Bs, Hs, n_keep), dtype=torch.int32, device=dev)
        ko = torch.empty((Bs, Hs, n_keep, Ds), dtype=torch.float16, device=dev)
        vo = torch.empty_like(ko)
        wsb = torch.empty(K.kvq_snapkv_workspace_bytes(Bs, Hs, Ss, Ds, ex["obs_window"]),
                          dtype=torch.uint8, device=dev)
        def snap(kk, vv):
            return lambda: K.kvq_snapkv_select(kk, vv, ex["obs_window"], ex["n_sink"], ex["budget"],
                                               sc, kept, ko, vo, wsb)
        msw = time_stream(snap(ksd, vsd), 200, 10, torch)
        ncp = n_copies(ks.nbytes + vs.nbytes)
        copies = [(ksd.clone(), vsd.clone()) for _ in range(ncp)]
        msd = time_rotating([snap(a, b) for a, b in copies], 20, torch)
        trials_d = trials_note(1e3)
        del copies
        sbytes = ks.nbytes + 2 * n_keep * Hs * Ds * 2 * 2 + sc.numel() * 4 + kept.numel() * 4
        rows["D_snapkv"] = {"workload": f"{ws_.name} S={Ss} w={ex['obs_window']} sink={ex['n_sink']} "
                                        f"budget={ex['budget']} Hkv={Hs} D={Ds}",
                            "us": round(msd * 1e3, 2), "trials_us": trials_d,
                            "scores/s": round(Hs * Ss / (msd * 1e-3), 1),
                            "logits/s": round(Bs * Hs * ex["obs_window"] * Ss / (msd * 1e-3), 1),
                            "algorithmic_bytes": sbytes,
                            "traffic": load_traffic(
                                os.path.join(ROOT, "profiles", "snapkv_s8192_traffic.json"),
                                os.path.join(ROOT, "evicted_kv_cache_amd", "csrc", "snapkv.hip")),
                            "GB/s": round(sbytes / msd / 1e6, 1),
                            "frac_hbm": round(sbytes / msd / 1e6 / PEAK_HBM_GBS, 4),
                            "timing": f"cold: graph replay over {ncp} copies of K and V "
                                      f"({ncp * (ks.nbytes + vs.nbytes) >> 20} MiB)",
                            "us_warm": round(msw * 1e3, 2),
                            "GB/s_warm": round(sbytes / msw / 1e6, 1)}

    # ---- row B, other decode workloads: Q4_0-style centered K + int8 V (B=16,
    # T=16384; HBM-bound) and a Llama-3.2-3B-shaped KIVI int4 layer (B=1,
    # T=8192; latency-bound).  Device time per step from a replayed graph of
    # 10 steps, so host marshalling is not in the timed region.
    if "B" in args.rows:
        for wname, over in (("q4_0_centered", {}), ("llama3b_kivi_int4", {}),
                            ("llama3b_kivi_int4", {"batch": 16, "seq_len": 16384})):
            wb = synth.workload(wname, **over)
            eb = wb.extra
            Bb, Hb, Hqb, Db, Tb = wb.batch, wb.n_kv_heads, wb.n_q_heads, wb.head_dim, wb.seq_len
            kh, vh, qh = synth.full(wb, threads=max(1, min(16, os.cpu_count() or 1)))
            kdb, vdb, qb = (torch.from_numpy(x).to(dev) for x in (kh, vh, qh))
            del kh, vh
            bias, flags = None, 0
            if eb["k_kind"] == "tok_sym4":
                bias = torch.from_numpy(np.stack([synth.head_params(wb, h)[0] for h in range(Hb)]))
                flags = K.KVQ_CENTER_K
            Lb = K.Layout(batch=Bb, n_kv_heads=Hb, head_dim=Db, capacity=Tb, k_kind=eb["k_kind"],
                          k_bits=eb["k_bits"], k_group=eb["k_group"], v_kind="tok_affine",
                          v_bits=eb["v_bits"], v_group=eb["v_group"], in_dtype=wb.dtype, flags=flags)
            cb = K.Cache(Lb, k_bias=bias)
            K.kvq_quantize_append(Lb, cb, kdb, vdb)
            outb = torch.empty((Bb, Hqb, Db), dtype=torch.float32, device=dev)
            wsb = torch.empty(max(K.kvq_decode_workspace_bytes(Lb, Hqb), 16), dtype=torch.uint8, device=dev)
            stepb = lambda: K.kvq_decode_attention(Lb, cb, qb, out=outb, ws=wsb)
            # warm: the same cache 10 times per replayed graph
            usw = time_rotating([stepb] * 10, 10, torch) * 1e3
            # cold: identical caches (appended from the same inputs) in rotation
            cache_bytes = sum(x.numel() for x in (cb.k_codes, cb.k_meta, cb.v_codes, cb.v_meta) if x is not None)
            ncp = n_copies(cache_bytes)
            caches = [cb]
            for _ in range(ncp - 1):
                cx = K.Cache(Lb, k_bias=bias)
                K.kvq_quantize_append(Lb, cx, kdb, vdb)
                caches.append(cx)
            del kdb, vdb
            usb = time_rotating([(lambda cc=cc: K.kvq_decode_attention(Lb, cc, qb, out=outb, ws=wsb))
                                 for cc in caches], 10, torch) * 1e3
            trials_b = trials_note(1e3)
            del caches
            qo = Bb * Hqb * Db * (2 + 4)
            if eb["k_kind"] == "tok_sym4":     # codes + fp16 block scales; int8 V + (scale, zero)
                nb = Bb * Hb * Tb * (Db // 2 + (Db // 32) * 2 + Db * eb["v_bits"] // 8 + (Db // eb["v_group"]) * 4) + qo
            else:                              # KIVI: codes + one table row per 32 tokens; int4 V
                nb = Bb * Hb * (Tb * Db * eb["k_bits"] // 8 + (Tb // eb["k_group"]) * Db * 4 +
                                Tb * Db * eb["v_bits"] // 8 + Tb * (Db // eb["v_group"]) * 4) + qo
            rows[f"B_decode_{wname}" + (f"_B{Bb}_T{Tb}" if over else "")] = {
                "workload": f"{wname} B={Bb} Hq/Hkv={Hqb}/{Hb} D={Db} T={Tb} K {eb['k_kind']} "
                            f"{eb['k_bits']}-bit, V affine {eb['v_bits']}-bit",
                "us": round(usb, 2), "trials_us": trials_b, "algorithmic_bytes": nb,
                "GB/s": round(nb / usb / 1e3, 1),
                "frac_hbm": round(nb / usb / 1e3 / PEAK_HBM_GBS, 4),
                "timing": f"cold: graph replay over {ncp} identical caches ({ncp * cache_bytes >> 20} MiB)",
                "us_warm": round(usw, 2), "GB/s_warm": round(nb / usw / 1e3, 1)}
            del cb, outb, wsb

    # ---- row E: multi-query (prefill-chunk) attention over the cache, the
    # microbenchmark shape of 128 causal queries per head with 32/8 heads x 128
    # over a 4-bit affine g64 cache; matrix-core bound (algorithmic FLOPs:
    # 2 per multiply-add of QK^T and PV over the visible slots)
    if "E" in args.rows:
        we = synth.workload("affine4_g64")
        n_q = 128
        for Te in [int(x) for x in args.e_lengths.split(",")]:
            ke, ve, _ = synth.full(we, T=Te, batch=1, threads=max(1, min(16, os.cpu_count() or 1)))
            Le = K.Layout(**{**L.__dict__, "batch": 1, "capacity": Te})
            ce = K.Cache(Le)
            K.kvq_quantize_append(Le, ce, bf16(ke), bf16(ve))
            del ke, ve
            rng = np.random.default_rng(Te)
            qe = torch.from_numpy(rng.standard_normal((1, Hq, n_q, D), dtype=np.float32)).to(dev).to(torch.bfloat16)
            oe = torch.empty((1, Hq, n_q, D), dtype=torch.float32, device=dev)
            wse = torch.empty(max(K.kvq_prefill_workspace_bytes(Le, Hq, n_q), 16), dtype=torch.uint8, device=dev)
            mse = time_stream(lambda: K.kvq_prefill_attention(Le, ce, qe, causal=True, out=oe, ws=wse), 20, 3, torch)
            trials_e = trials_note(1e3)
            flops = 4 * D * Hq * (n_q * (Te - n_q) + n_q * (n_q + 1) // 2)
            tf = flops / mse / 1e9
            rows[f"E_prefill_attention_T{Te}"] = {
                "workload": f"{we.name} B=1 Hq/Hkv={Hq}/{Hkv} D={D} T={Te}, {n_q} causal queries per head",
                "us": round(mse * 1e3, 2), "trials_us": trials_e, "algorithmic_flops": flops,
                "TFLOP/s": round(tf, 1),
                "frac_mfma_fp16": round(tf / PEAK_MFMA_F16_TFLOPS, 4)}
            del ce, oe, wse

    # bandwidth probes on the same device: a 2 GiB device copy (read + write)
    # and a 2 GiB read (a sum reduction), both torch library kernels
    probes = None
    if args.mode == "full":
        n = 1 << 31
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        msc = time_stream(lambda: dst.copy_(src), 10, 3, torch)
        msr = time_stream(lambda: torch.sum(src), 10, 3, torch)
        del src, dst
        probes = {"copy_GB/s": round(2 * n / msc / 1e6, 1), "read_GB/s": round(n / msr / 1e6, 1),
                  "what": "torch copy_ of 2 GiB (read + write bytes) and torch.sum over 2 GiB (read bytes)"}
        probes["step_frac_of_copy_probe"] = round(gbs / probes["copy_GB/s"], 4)
        probes["step_frac_of_read_probe"] = round(gbs / probes["read_GB/s"], 4)
        log(f"probes: copy {probes['copy_GB/s']} GB/s, read {probes['read_GB/s']} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing CPU oracle baseline")
        cpu = cpu_baseline(w)

    result = {
        "metric": "quantized decode-attention GB/s and % HBM roofline at T=32K; SnapKV prefill scores/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "warmup_settling": {
            "what": "us per step over the untimed warm-up steps (run right after the prefill append), "
                    "by blocks of 50: the shader clock dips under the first tens of ms of sustained "
                    "decode and settles after about 100 steps",
            "us_first_20": round(1e3 * sum(warm[:20]) / max(1, len(warm[:20])), 1) if warm else None,
            "us_per_50": [round(1e3 * sum(warm[i:i + 50]) / len(warm[i:i + 50]), 1)
                          for i in range(0, len(warm), 50)]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 q / u4 codes, fp16 MFMA operands (exact), fp32 accumulate",
        "data": "synthetic (seeded N(0,1), synth.affine4_g64)",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "seq_len": T, "k_format": "tok_affine u4 g64 fp16 scale+zero",
                   "v_format": "tok_affine u4 g64 fp16 scale+zero",
                   "token_q_heads_per_s": round(B * Hq * T / (ms * 1e-3), 1),
                   "token_kv_heads_per_s": round(B * Hkv * T / (ms * 1e-3), 1),
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "decode_mfma_kernel<bf16, 64, 64> (one launch per step)"},
        "cpu_baseline": cpu,
        "bandwidth_probes": probes,
        "rows": rows,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

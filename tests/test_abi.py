"""Host-side tests of the libkvq C ABI (no GPU needed).

Validation runs before anything is enqueued, so invalid calls can be made
with fake (never dereferenced) device pointers on a machine without a GPU.
"""
import ctypes
import json
import os
import re

import pytest

import evicted_kv_cache_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # 16-byte aligned, never dereferenced by validation
MIS = 0x10004           # misaligned


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"kvq_quantize_append", "kvq_decode_attention", "kvq_evict_streaming",
            "kvq_snapkv_select"} <= set(names)
    lib = K.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(K.EXPORTS)
    assert lib.kvq_version() == 1


def test_status_strings():
    for code in (0, 1, -1, -2, -3, -4, -5, -6, -7):
        assert K.status_string(code) and K.status_string(code) != "unknown status"
    assert K.status_string(-99) == "unknown status"


def c5_layout(**kw):
    base = dict(batch=64, n_kv_heads=8, head_dim=128, capacity=32768, k_kind="tok_affine",
                k_bits=4, k_group=64, v_kind="tok_affine", v_bits=4, v_group=64, in_dtype="bf16")
    base.update(kw)
    return K.Layout(**base)


def test_cache_sizes_headline_layout():
    s = K.kvq_cache_sizes(c5_layout())
    # 4-bit codes: 64 B per token-head; g64 fp16 (scale, zero): 8 B per token-head
    assert s.k_codes == s.v_codes == 64 * 8 * 32768 * 64 == 2 ** 30
    assert s.k_meta == s.v_meta == 64 * 8 * 32768 * 8 == 2 ** 27
    elems = 64 * 8 * 32768 * 128
    assert (s.k_codes + s.k_meta) * 8 / elems == 4.5        # P4: 4.5 bits/elt at g64
    s32 = K.kvq_cache_sizes(c5_layout(k_group=32))
    assert (s32.k_codes + s32.k_meta) * 8 / elems == 5.0    # P4: 5.0 bits/elt at g32


def test_cache_sizes_match_tinygpt_int8_value_bytes():
    """P1 cache-bytes table at T=500 (12 layers x 8 heads x 32 dim): int8 values
    cost 1 B/element and per-token fp16 scale+zero 2 x 2 B per token-head;
    with layers laid out as batch, kvq's per-token int8 V has exactly those bytes."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "p1_streaming_kivi.json")))
    t, b = g["tinygpt"], g["int8_kivi_bytes"]
    L = K.Layout(batch=t["layers"], n_kv_heads=t["heads"], head_dim=t["head_dim"],
                 capacity=t["T"], k_kind="kivi_ch", k_bits=8, k_group=32,
                 v_kind="tok_affine", v_bits=8, v_group=t["head_dim"], in_dtype="f32")
    s = K.kvq_cache_sizes(L)
    assert s.v_codes == b["v_codes"]
    assert s.v_meta == 2 * b["v_scales_each"]
    assert s.k_codes == b["k_codes"]
    # P1's K keeps one (scale, zero) per channel over all of T; kvq freezes one
    # per 32-token group: table rows = capacity / 32 + 3 (two runs of slots)
    assert s.k_table_rows == 500 // 32 + 3
    # P1's printed total for its own layout (whole-T K scales) is consistent
    assert b["k_codes"] + b["v_codes"] + 2 * b["k_scales_each"] + 2 * b["v_scales_each"] == b["total"]


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), K.KVQ_ERR_UNSUPPORTED),
    (dict(head_dim=0), K.KVQ_ERR_INVALID_ARG),
    (dict(batch=0), K.KVQ_ERR_INVALID_ARG),
    (dict(k_bits=3), K.KVQ_ERR_UNSUPPORTED),
    (dict(v_bits=6), K.KVQ_ERR_UNSUPPORTED),
    (dict(k_kind="tok_sym4", k_bits=2, k_group=32), K.KVQ_ERR_UNSUPPORTED),
    (dict(k_group=48), K.KVQ_ERR_UNSUPPORTED),
    (dict(v_kind="tok_sym4"), K.KVQ_ERR_UNSUPPORTED),
    (dict(k_kind="kivi_ch", k_group=12), K.KVQ_ERR_UNSUPPORTED),
    (dict(k_kind="tok_sym4", k_group=64), K.KVQ_ERR_UNSUPPORTED),
    # P3 gate: centering only for the symmetric 4-bit K format
    (dict(flags=K.KVQ_CENTER_K), K.KVQ_ERR_UNSUPPORTED),
    (dict(k_kind="plain", flags=K.KVQ_CENTER_K), K.KVQ_ERR_UNSUPPORTED),
    (dict(k_kind="plain", flags=K.KVQ_CENTER_K | K.KVQ_TEST_CENTER_ANY), K.KVQ_ERR_UNSUPPORTED),
    (dict(flags=0x100), K.KVQ_ERR_INVALID_ARG),
])
def test_layout_validation(kw, code):
    with pytest.raises(K.KvqError) as e:
        K.kvq_cache_sizes(c5_layout(**kw))
    assert e.value.status == code


def test_two_bit_layouts_sizes():
    """KIVI-2bit: four codes per byte for per-channel and per-token kinds."""
    s = K.kvq_cache_sizes(c5_layout(k_kind="kivi_ch", k_bits=2, k_group=32, v_bits=2, v_group=32))
    assert s.k_codes == s.v_codes == 64 * 8 * 32768 * 128 // 4
    assert s.v_meta == 64 * 8 * 32768 * (128 // 32) * 4
    s2 = K.kvq_cache_sizes(c5_layout(k_bits=2, v_bits=2, head_dim=32, k_group=32, v_group=32))
    assert s2.k_codes == 64 * 8 * 32768 * 8


def test_centering_gate_accepts_sym4_and_test_seam():
    K.kvq_cache_sizes(c5_layout(k_kind="tok_sym4", k_group=32, flags=K.KVQ_CENTER_K))
    K.kvq_cache_sizes(c5_layout(k_kind="plain", in_dtype="f32",
                                flags=K.KVQ_CENTER_K | K.KVQ_TEST_CENTER_ANY))


def fake_cache(L, n_stored=0, n_quant=None, misalign=None, base=FAKE):
    s = K.kvq_cache_sizes(L)
    ptr = {n: (base + (1 << 32) * i if getattr(s, n) else None)
           for i, n in enumerate(("k_codes", "k_meta", "k_resid", "v_codes", "v_meta", "pos", "k_row"))}
    if misalign:
        ptr[misalign] = MIS
    c = K.c_cache(ptr["k_codes"], ptr["k_meta"], ptr["k_resid"], ptr["v_codes"], ptr["v_meta"],
                  ptr["pos"], ptr["k_row"], None, n_stored,
                  n_stored if n_quant is None else n_quant, n_stored, n_stored)
    return c


def call_append(L, c, n_new, k=FAKE, v=FAKE):
    cl = L.c()
    return K.lib().kvq_quantize_append(ctypes.byref(cl), ctypes.byref(c), k, v, n_new, None)


def test_append_validation_without_gpu():
    L = c5_layout(batch=1, capacity=100)
    c = fake_cache(L, n_stored=90)
    assert call_append(L, c, 11) == K.KVQ_ERR_CAPACITY          # nothing auto-evicts
    assert c.n_stored == 90                                      # cache unchanged on error
    assert call_append(L, c, 0) == K.KVQ_ERR_INVALID_ARG
    assert call_append(L, c, 1, k=MIS) == K.KVQ_ERR_ALIGNMENT
    assert call_append(L, c, 1, k=0) == K.KVQ_ERR_INVALID_ARG
    bad = fake_cache(L, n_stored=5, misalign="v_meta")
    assert call_append(L, bad, 1) == K.KVQ_ERR_ALIGNMENT
    missing = fake_cache(L, n_stored=5)
    missing.k_meta = None
    assert call_append(L, missing, 1) == K.KVQ_ERR_INVALID_ARG
    # counters must be consistent
    inc = fake_cache(L, n_stored=5, n_quant=3)
    assert call_append(L, inc, 1) == K.KVQ_ERR_INVALID_ARG
    # centering without a bias pointer
    Ls = c5_layout(batch=1, capacity=100, k_kind="tok_sym4", k_group=32, flags=K.KVQ_CENTER_K)
    assert call_append(Ls, fake_cache(Ls), 1) == K.KVQ_ERR_INVALID_ARG


def test_kivi_residual_counter_validation():
    L = c5_layout(batch=1, capacity=100, k_kind="kivi_ch", k_group=32)
    assert call_append(L, fake_cache(L, n_stored=40, n_quant=0), 1) == K.KVQ_ERR_INVALID_ARG


def call_decode(L, c, hq, ws=FAKE, ws_bytes=1 << 30, q=FAKE, out=FAKE, qdt=K.KVQ_BF16, scale=0.0):
    cl = L.c()
    return K.lib().kvq_decode_attention(ctypes.byref(cl), ctypes.byref(c), q, qdt, hq,
                                        ctypes.c_float(scale), out, ws, ws_bytes, None)


def test_decode_validation_without_gpu():
    L = c5_layout(batch=2, capacity=1000)
    c = fake_cache(L, n_stored=500)
    assert call_decode(L, c, 12) == K.KVQ_ERR_INVALID_ARG        # not a multiple of Hkv
    assert call_decode(L, c, 8 * 9) == K.KVQ_ERR_UNSUPPORTED     # > 8 q-heads per kv-head
    assert call_decode(L, c, 32, ws=0) == K.KVQ_ERR_WORKSPACE
    need = K.kvq_decode_workspace_bytes(L, 32)
    assert need > 0
    assert call_decode(L, c, 32, ws_bytes=need - 1) == K.KVQ_ERR_WORKSPACE
    assert call_decode(L, c, 32, q=MIS) == K.KVQ_ERR_ALIGNMENT
    assert call_decode(L, c, 32, qdt=7) == K.KVQ_ERR_INVALID_ARG
    assert call_decode(L, c, 32, scale=float("nan")) == K.KVQ_ERR_INVALID_ARG


def call_decode_noalloc(L, c, hq, q=FAKE, out=FAKE, qdt=K.KVQ_BF16, scale=0.0):
    cl = L.c()
    return K.lib().kvq_decode_attention_noalloc(ctypes.byref(cl), ctypes.byref(c), q, qdt, hq,
                                                ctypes.c_float(scale), out, None)


def test_decode_noalloc_validation_without_gpu():
    """The no-allocation decode validates like kvq_decode_attention and
    rejects, before touching the device, a call whose split partials exceed
    the fixed scratch (8 MiB): the LDS-tiled kernel writes B * Hq * splits *
    (D + 2) fp32, here 4096 * 64 * 130 * 4 B at one split."""
    L = c5_layout(batch=2, capacity=1000)
    c = fake_cache(L, n_stored=500)
    assert call_decode_noalloc(L, c, 12) == K.KVQ_ERR_INVALID_ARG
    assert call_decode_noalloc(L, c, 8 * 9) == K.KVQ_ERR_UNSUPPORTED
    assert call_decode_noalloc(L, c, 32, q=MIS) == K.KVQ_ERR_ALIGNMENT
    assert call_decode_noalloc(L, c, 32, qdt=7) == K.KVQ_ERR_INVALID_ARG
    assert call_decode_noalloc(L, c, 32, scale=float("nan")) == K.KVQ_ERR_INVALID_ARG
    big = c5_layout(batch=4096, capacity=64, k_kind="kivi_ch", k_bits=8, k_group=32, v_bits=8,
                    v_group=128)
    assert call_decode_noalloc(big, fake_cache(big, n_stored=40, n_quant=32), 64) == K.KVQ_ERR_SCRATCH


def call_evict(L, src, dst, sink, window):
    cl = L.c()
    return K.lib().kvq_evict_streaming(ctypes.byref(cl), ctypes.byref(src), ctypes.byref(dst),
                                       sink, window, None)


def test_evict_validation_without_gpu():
    L = c5_layout(batch=1, capacity=300, k_kind="kivi_ch", k_group=32)
    src = fake_cache(L, n_stored=280, n_quant=256)
    dst = fake_cache(L, base=FAKE + (1 << 40))
    # below the cap: NOOP, nothing enqueued (no GPU call happens)
    assert call_evict(L, src, dst, 4, 276) == K.KVQ_NOOP
    assert dst.n_stored == 0
    # out-of-place: dst must not alias src
    assert call_evict(L, src, src, 4, 256) == K.KVQ_ERR_INVALID_ARG
    # the open K group must stay: window >= k_group
    assert call_evict(L, src, dst, 4, 16) == K.KVQ_ERR_INVALID_ARG
    assert call_evict(L, src, dst, -1, 256) == K.KVQ_ERR_INVALID_ARG
    # kept positions may not form a third run: after a first eviction the
    # sink prefix can only shrink and the window must stay past it
    src.n_head = 4
    assert call_evict(L, src, dst, 8, 200) == K.KVQ_ERR_UNSUPPORTED
    assert call_evict(L, src, dst, 2, 277) == K.KVQ_ERR_UNSUPPORTED   # window reaches slot 3 < n_head


def test_snapkv_validation_without_gpu():
    lib = K.lib()
    ws = K.kvq_snapkv_workspace_bytes(1, 8, 8192, 128, 32)
    assert ws > 8 * 8192 * 4

    def call(B=1, H=8, S=8192, D=128, w=32, sink=4, budget=512, ws_bytes=ws, k=FAKE):
        return lib.kvq_snapkv_select(k, FAKE, B, H, S, D, w, sink, budget, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, ws_bytes, None)
    assert call(D=96) == K.KVQ_ERR_UNSUPPORTED
    assert call(w=0) == K.KVQ_ERR_INVALID_ARG
    assert call(budget=0) == K.KVQ_ERR_INVALID_ARG
    assert call(sink=-1) == K.KVQ_ERR_INVALID_ARG
    assert call(w=200) == K.KVQ_ERR_UNSUPPORTED
    assert call(S=100, w=200, ws_bytes=0) == K.KVQ_ERR_WORKSPACE  # w clamps to S: allowed, ws checked
    assert call(ws_bytes=ws - 1) == K.KVQ_ERR_WORKSPACE
    assert call(k=MIS) == K.KVQ_ERR_ALIGNMENT
    assert lib.kvq_snapkv_select_from_scores(MIS, 1, 8, 100, 4, 10, FAKE, None) == K.KVQ_ERR_ALIGNMENT
    assert lib.kvq_snapkv_select_from_scores(FAKE, 1, 8, 0, 4, 10, FAKE, None) == K.KVQ_ERR_INVALID_ARG


def test_snapkv_options_validation_without_gpu():
    lib = K.lib()

    def opts(q=None, hq=0, pool=1):
        return ctypes.byref(K.c_snapkv_opts(q, hq, pool))

    def wsb(o, B=1, H=8, S=8192, D=128, w=32):
        return lib.kvq_snapkv_workspace_bytes_ex(o, B, H, S, D, w)

    base = K.kvq_snapkv_workspace_bytes(1, 8, 8192, 128, 32)
    assert wsb(None) == base == wsb(opts())
    # pooling adds one score buffer; query windows of G*w rows grow the statistics
    assert wsb(opts(pool=7)) == base + 8 * 8192 * 4
    assert wsb(opts(q=FAKE, hq=32)) > base
    assert wsb(opts(pool=4)) == 0 and wsb(opts(q=FAKE, hq=12)) == 0
    assert wsb(opts(q=FAKE, hq=64)) == 0                            # 8 * 32 rows > 128
    big = wsb(opts(q=FAKE, hq=32, pool=5))

    def call(o, S=8192, w=32, ws_bytes=big, k=FAKE):
        return lib.kvq_snapkv_select_ex(o, k, FAKE, 1, 8, S, 128, w, 4, 512, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, ws_bytes, None)
    assert call(opts(pool=0)) == K.KVQ_ERR_INVALID_ARG
    assert call(opts(pool=6)) == K.KVQ_ERR_INVALID_ARG
    assert call(opts(pool=33)) == K.KVQ_ERR_UNSUPPORTED
    assert call(opts(q=FAKE, hq=12)) == K.KVQ_ERR_INVALID_ARG      # not a multiple of Hkv
    assert call(opts(q=FAKE, hq=4)) == K.KVQ_ERR_INVALID_ARG       # fewer query than kv heads
    assert call(opts(q=FAKE, hq=64)) == K.KVQ_ERR_UNSUPPORTED      # 256 rows per kv-head
    assert call(opts(q=FAKE, hq=32), S=16) == K.KVQ_ERR_INVALID_ARG  # window longer than prompt
    assert call(opts(q=MIS, hq=32)) == K.KVQ_ERR_ALIGNMENT
    assert call(opts(q=FAKE, hq=32, pool=5), ws_bytes=big - 1) == K.KVQ_ERR_WORKSPACE
    assert call(opts(pool=5), ws_bytes=base) == K.KVQ_ERR_WORKSPACE   # pooled buffer missing
    assert call(opts(q=FAKE, hq=32, pool=5), k=MIS) == K.KVQ_ERR_ALIGNMENT
    pool = lib.kvq_snapkv_pool_scores
    assert pool(FAKE, FAKE + 16 * 4, 1, 1, 100, 3, None) == K.KVQ_ERR_INVALID_ARG   # overlap
    assert pool(FAKE, 0x100000, 1, 1, 100, 2, None) == K.KVQ_ERR_INVALID_ARG
    assert pool(FAKE, 0x100000, 1, 1, 100, 35, None) == K.KVQ_ERR_UNSUPPORTED
    assert pool(None, 0x100000, 1, 1, 100, 3, None) == K.KVQ_ERR_INVALID_ARG


def test_append_at_validation_without_gpu():
    L = c5_layout(batch=2, capacity=100, in_dtype="f16", flags=K.KVQ_POS_PER_HEAD)
    assert K.kvq_cache_sizes(L).pos == 2 * 8 * 100 * 4           # one position row per (b, h)
    assert K.kvq_cache_sizes(c5_layout(batch=2, capacity=100)).pos == 100 * 4
    lib = K.lib()

    def call(c, n_new=10, src_rows=0, positions=FAKE, pos_rows=0, next_pos=50):
        cl = L.c()
        return lib.kvq_quantize_append_at(ctypes.byref(cl), ctypes.byref(c), FAKE, FAKE, n_new, src_rows,
                                          positions, pos_rows, next_pos, None)
    c = fake_cache(L, n_stored=0)
    assert call(c, positions=None) == K.KVQ_ERR_INVALID_ARG
    assert call(c, src_rows=5) == K.KVQ_ERR_INVALID_ARG          # fewer source rows than n_new
    assert call(c, pos_rows=9) == K.KVQ_ERR_INVALID_ARG
    assert call(c, next_pos=9) == K.KVQ_ERR_INVALID_ARG          # counter below the stored count
    assert call(c, positions=MIS) == K.KVQ_ERR_ALIGNMENT
    assert call(c, n_new=101, next_pos=200) == K.KVQ_ERR_CAPACITY
    c2 = fake_cache(L, n_stored=20)                              # its counter is 20
    assert call(c2, next_pos=19) == K.KVQ_ERR_INVALID_ARG
    assert c2.n_stored == 20 and c.n_stored == 0


def test_snapkv_prefill_chunk_validation_without_gpu():
    lib = K.lib()
    B, H, D, cap = 1, 8, 128, 600
    ws = K.kvq_snapkv_chunk_workspace_bytes(B, H, D, cap, 32)
    assert ws > B * H * cap * 8                                  # scores + kept indices at least
    assert K.kvq_snapkv_chunk_workspace_bytes(B, H, 96, cap, 32) == 0

    def state(base, capacity=cap, n_kept=0, next_pos=0):
        return K.c_snapkv_state(base, base + (1 << 30), base + (2 << 30), capacity, n_kept, next_pos)

    def call(si, so, n=100, budget=512, ws_bytes=ws, kc=FAKE, opts=None):
        return lib.kvq_snapkv_prefill_chunk(opts, ctypes.byref(si), ctypes.byref(so), kc, FAKE, n, B, H, D,
                                            32, 4, budget, None, FAKE, ws_bytes, None)
    A, Bs = 1 << 36, 1 << 37
    assert call(state(A, n_kept=550, next_pos=550), state(Bs), n=51) == K.KVQ_ERR_CAPACITY   # past in capacity
    assert call(state(A), state(Bs, capacity=50), n=100) == K.KVQ_ERR_CAPACITY             # out too small
    assert call(state(A), state(A + 16)) == K.KVQ_ERR_INVALID_ARG                          # overlapping states
    assert call(state(A), state(Bs), n=0) == K.KVQ_ERR_INVALID_ARG
    assert call(state(A, n_kept=10, next_pos=5), state(Bs)) == K.KVQ_ERR_INVALID_ARG       # counters
    assert call(state(A), state(Bs), ws_bytes=ws - 1) == K.KVQ_ERR_WORKSPACE
    assert call(state(A), state(Bs), kc=MIS) == K.KVQ_ERR_ALIGNMENT
    assert call(state(A), state(Bs), budget=0) == K.KVQ_ERR_INVALID_ARG
    o = K.c_snapkv_opts(FAKE, 32, 4)
    assert call(state(A), state(Bs), opts=ctypes.byref(o)) == K.KVQ_ERR_INVALID_ARG        # even pool width
    si = state(A, n_kept=7, next_pos=9)
    assert call(si, state(Bs), n=cap) == K.KVQ_ERR_CAPACITY
    assert (si.n_kept, si.next_pos) == (7, 9)                                              # untouched on error


def test_rope_validation_without_gpu():
    lib = K.lib()
    assert lib.kvq_rope_table(None, 10, 128, 10000.0, None) == K.KVQ_ERR_INVALID_ARG
    assert lib.kvq_rope_table(FAKE, 0, 128, 10000.0, None) == K.KVQ_ERR_INVALID_ARG
    assert lib.kvq_rope_table(FAKE, 10, 96, 10000.0, None) == K.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_rope_table(FAKE, 10, 128, 1.0, None) == K.KVQ_ERR_INVALID_ARG
    assert lib.kvq_rope_table(MIS, 10, 128, 10000.0, None) == K.KVQ_ERR_ALIGNMENT
    L = c5_layout(batch=1, capacity=100)
    c = fake_cache(L, n_stored=50)

    def call(table=FAKE, rows=64, q_pos=49, q=FAKE):
        cl = L.c()
        return lib.kvq_decode_attention_rope(ctypes.byref(cl), ctypes.byref(c), q, K.KVQ_BF16, 32, 0.0, table,
                                             rows, q_pos, FAKE, FAKE, 1 << 30, None)
    assert call(table=None) == K.KVQ_ERR_INVALID_ARG
    assert call(q_pos=64) == K.KVQ_ERR_INVALID_ARG           # query position outside the table
    assert call(q_pos=-1) == K.KVQ_ERR_INVALID_ARG
    assert call(rows=49, q_pos=10) == K.KVQ_ERR_INVALID_ARG  # fewer table rows than stored slots
    assert call(table=MIS) == K.KVQ_ERR_ALIGNMENT
    assert call(q=MIS) == K.KVQ_ERR_ALIGNMENT


def test_prefill_attention_validation_without_gpu():
    lib = K.lib()
    L = c5_layout(batch=1, capacity=32768)
    ws = K.kvq_prefill_workspace_bytes(L, 32, 128)
    assert ws >= 32 * 128 * (128 + 2) * 4                 # at least one split's partials
    assert K.kvq_prefill_workspace_bytes(L, 30, 128) == 0  # Hq not a multiple of Hkv
    c = fake_cache(L, n_stored=100)

    def call(n_q=128, causal=0, ws_bytes=ws, q=FAKE, Hq=32):
        cl = L.c()
        return lib.kvq_prefill_attention(ctypes.byref(cl), ctypes.byref(c), q, K.KVQ_BF16, Hq, n_q, 0.0, causal,
                                         FAKE, FAKE, ws_bytes, None)
    assert call(n_q=0) == K.KVQ_ERR_INVALID_ARG
    assert call(causal=2) == K.KVQ_ERR_INVALID_ARG
    assert call(n_q=101, causal=1) == K.KVQ_ERR_INVALID_ARG     # the chunk is longer than the cache
    assert call(ws_bytes=ws - 1) == K.KVQ_ERR_WORKSPACE
    assert call(q=MIS) == K.KVQ_ERR_ALIGNMENT
    assert call(Hq=30) == K.KVQ_ERR_INVALID_ARG
    assert call(Hq=80) == K.KVQ_ERR_UNSUPPORTED                 # more than 8 query heads per kv-head
    # 8 kv-heads x ceil(4 * 262144 / 128) = 65536 row blocks of 128 rows
    assert call(n_q=262144) == K.KVQ_ERR_UNSUPPORTED
    assert call(n_q=262112, ws_bytes=0) == K.KVQ_ERR_WORKSPACE   # 65528 row blocks: past the limit check


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(K, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(K, "_lib", None)
    with pytest.raises(ImportError):
        K.lib()

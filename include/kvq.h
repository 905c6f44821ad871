/*
 * kvq.h -- C ABI of libkvq: decode-time attention over a compressed KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * Four operations make up the path:
 *   kvq_quantize_append   quantize-on-write of new K/V rows
 *   kvq_decode_attention  fused dequantize + QK^T + softmax + PV for one query
 *                         token per sequence, reading the packed cache
 *   kvq_evict_streaming   StreamingLLM sink + window compaction
 *   kvq_snapkv_select     SnapKV prefill scoring, selection and gather
 *
 * Sources the operations follow (cited by page title and section):
 *   [P1] "StreamingLLM + KIVI -- long-context decode without growing the KV
 *        cache" (posttrainllm.com).
 *   [P2] "SnapKV -- Prefill Observation-Window Token Eviction" (veloxquant-mlx).
 *   [P3] "kv-cache: optional per-channel K-cache mean-centering for Q4_0"
 *        (llama.cpp pull request #51).
 *   [P4] "Low-bit KV caches on MLX: what exists and what is missing".
 *
 * Conventions for every call:
 *   - Pointers named in a layout comment as device memory are device pointers
 *     on the current HIP device; the layout/cache/size structs themselves are
 *     host memory.  The caller owns all memory; the library allocates nothing
 *     and keeps no state besides cached device properties and the fixed
 *     scratch of kvq_decode_attention_noalloc.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and never synchronized; outputs are valid once the stream reaches them.
 *   - Arguments are validated on the host before anything is enqueued.  On an
 *     error nothing is launched and caches are left unchanged.  Launch
 *     failures are reported as KVQ_ERR_HIP.
 *   - Every device pointer must be 16-byte aligned (KVQ_ERR_ALIGNMENT).
 *   - Lengths are uniform over the batch and follow from the calls, so no
 *     device-to-host read-back is ever needed: the cache struct's counters
 *     are host-side and updated when work is enqueued.
 *   - Calls on one cache must be ordered (same stream or explicit events).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_VERSION 1

typedef enum {
    KVQ_OK = 0,
    KVQ_NOOP = 1,               /* nothing to do (eviction below the cap) */
    KVQ_ERR_INVALID_ARG = -1,
    KVQ_ERR_UNSUPPORTED = -2,   /* valid request outside what the kernels implement */
    KVQ_ERR_CAPACITY = -3,      /* append past the cache capacity */
    KVQ_ERR_ALIGNMENT = -4,
    KVQ_ERR_WORKSPACE = -5,     /* workspace missing or too small */
    KVQ_ERR_HIP = -6,           /* a HIP launch or runtime call failed */
    KVQ_ERR_SCRATCH = -7        /* needs more than the fixed scratch of a no-allocation call */
} kvq_status;

/* Element types of K/V inputs, queries and PLAIN storage. */
typedef enum { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 } kvq_dtype;

/* Storage kinds.
 *
 * KVQ_PLAIN      values stored as given, in the layout's in_dtype.
 * KVQ_KIVI_CH    (K only) KIVI per-channel keys ([P1] "KIVI"; [P4] s.3):
 *                one (scale, zero) per (batch, kv-head, channel) for each
 *                closed group of k_group consecutive tokens (group = append
 *                index / k_group).  Keys of the open group wait in a
 *                full-precision residual buffer and are attended from it.
 * KVQ_TOK_AFFINE per-token asymmetric groups of `group` channels along
 *                head_dim ([P1] "Affine quantisation formula" per token for V;
 *                [P4] s.1 mx.quantize group layout for K and V).
 * KVQ_TOK_SYM4   (K only) symmetric 4-bit blocks of 32 channels with one fp16
 *                scale (the Q4_0 shape, [P3] "The idea"), optionally after
 *                subtracting a fixed per-(kv-head, channel) mean.
 */
typedef enum { KVQ_PLAIN = 0, KVQ_KIVI_CH = 1, KVQ_TOK_AFFINE = 2, KVQ_TOK_SYM4 = 3 } kvq_kind;

/* layout.flags */
#define KVQ_CENTER_K         0x1  /* subtract cache.k_bias before quantizing K (TOK_SYM4 only) */
#define KVQ_TEST_CENTER_ANY  0x2  /* test seam: also allow KVQ_CENTER_K with PLAIN keys */
#define KVQ_POS_PER_HEAD     0x4  /* one position row per (batch, kv-head): caches that hold
                                     SnapKV-kept rows, whose positions differ between heads */

/* Quantization arithmetic (bit-exact specification, fp32, IEEE round to
 * nearest even, no fused multiply-add):
 *   affine slice x[0..n):  range = max - min;  s = max(1e-5, range / (2^bits - 1));
 *       scale = fp16(s), zero = fp16(min);  code u = clamp(rint((x - zero) / scale), 0, 2^bits-1)
 *       where zero and scale are the stored fp16 values widened to fp32.
 *       Dequantized value: u * scale + zero.            ([P1] formula, eps 1e-5)
 *   symmetric block of 32: x' = x - bias; d = fp16(max(1e-5, max|x'| / 7));
 *       code u = clamp(rint(x' / d), -8, 7) + 8;  value (u - 8) * d.
 * Inputs must be finite.  K/V rows holding NaN or +-Inf, or a k_bias that
 * makes x - bias overflow, are outside this specification: the call still
 * completes and writes only the slots and table rows it appends, but the
 * codes and metadata of the groups that hold such values are unspecified,
 * and so is attention over them.
 * Codes are stored packed: 8-bit codes one per byte; 4-bit codes two per
 * byte with element 2i in the low nibble of byte i; 2-bit codes (KIVI-2bit,
 * [P2] "SnapKV-adapted" table; [P4] s.1 mx.quantize widths) four per byte,
 * element 4i + r in bits [2r, 2r + 2) of byte i.
 */
typedef struct kvq_layout {
    int32_t batch;        /* B >= 1 */
    int32_t n_kv_heads;   /* Hkv >= 1 */
    int32_t head_dim;     /* D in {32, 64, 128} */
    int32_t capacity;     /* slots per (batch, kv-head), >= 1 */
    int32_t k_kind;       /* kvq_kind */
    int32_t k_bits;       /* 2, 4 or 8 (KIVI_CH, TOK_AFFINE); 4 (TOK_SYM4); ignored for PLAIN */
    int32_t k_group;      /* KIVI_CH: tokens per group (8..128, power of two);
                             TOK_AFFINE: channels per group (32, 64 or 128, dividing D);
                             TOK_SYM4: must be 32; PLAIN: ignored */
    int32_t v_kind;       /* KVQ_PLAIN or KVQ_TOK_AFFINE */
    int32_t v_bits;       /* 2, 4 or 8 (TOK_AFFINE) */
    int32_t v_group;      /* channels per group (32, 64 or 128, dividing D) */
    int32_t in_dtype;     /* kvq_dtype of appended K/V, PLAIN storage and the KIVI residual */
    int32_t flags;        /* KVQ_CENTER_K | KVQ_TEST_CENTER_ANY | KVQ_POS_PER_HEAD */
} kvq_layout;

/* One layer's cache.  Device buffers (sizes from kvq_cache_sizes):
 *   k_codes  coded K:  [B][Hkv][capacity][D*k_bits/8] bytes
 *            PLAIN K:  [B][Hkv][capacity][D] in_dtype
 *   k_meta   TOK_AFFINE: [B][Hkv][capacity][D/k_group][2] fp16 (scale, zero)
 *            TOK_SYM4:   [B][Hkv][capacity][D/32] fp16 scales
 *            KIVI_CH:    [B][Hkv][k_table_rows][D][2] fp16 (scale, zero) table,
 *                        one row per live token group, rows in group order
 *            PLAIN: unused (may be NULL)
 *   k_resid  KIVI_CH only: [B][Hkv][k_group][D] in_dtype; residual row i holds
 *            the key of slot n_quant + i
 *   v_codes, v_meta  as for K with v_kind / v_bits / v_group
 *   pos      [capacity] int32 absolute position of each slot (shared over
 *            batch and heads; [P2]: positions stay the true positions), or
 *            [B][Hkv][capacity] with KVQ_POS_PER_HEAD
 *   k_row    KIVI_CH only: [capacity] int32 table row of each coded slot
 *   k_bias   [Hkv][D] fp32 mean subtracted from K before TOK_SYM4
 *            quantization when layout.flags has KVQ_CENTER_K ([P3]); else NULL
 * Host counters (maintained by the library; zero them for an empty cache):
 *   n_stored  slots in use, n_quant  slots whose K is coded (KIVI_CH: the
 *   rest are in the residual; other kinds: == n_stored), next_pos  position
 *   of the next appended token (generation counter, [P1] "stored count" vs
 *   current length), n_head  length of the slot prefix whose positions equal
 *   their slot index.
 */
typedef struct kvq_cache {
    void* k_codes;
    void* k_meta;
    void* k_resid;
    void* v_codes;
    void* v_meta;
    int32_t* pos;
    int32_t* k_row;
    const float* k_bias;
    int32_t n_stored;
    int32_t n_quant;
    int32_t next_pos;
    int32_t n_head;
} kvq_cache;

typedef struct kvq_sizes {
    size_t k_codes, k_meta, k_resid, v_codes, v_meta, pos, k_row;  /* bytes */
    int32_t k_table_rows;   /* KIVI_CH table rows (capacity / k_group + 3), else 0 */
    int32_t reserved;
} kvq_sizes;

/* Validate a layout and report the byte size of every cache buffer (host only). */
kvq_status kvq_cache_sizes(const kvq_layout* layout, kvq_sizes* out);

/* Zero the host counters of a cache (host only). */
kvq_status kvq_cache_reset(kvq_cache* cache);

/* Quantize-on-write ([P1] "KIVI": K per channel, V per token; [P4] s.1 and
 * s.3).  Appends n_new tokens per (batch, kv-head) at slots n_stored ..
 * n_stored+n_new-1 with positions next_pos ...  V rows (and TOK_AFFINE /
 * TOK_SYM4 / PLAIN K rows) are quantized immediately and never change.
 * KIVI_CH keys enter the residual; every time the residual reaches k_group
 * keys the group closes: per channel its min/max over exactly those keys
 * gives (scale, zero), its codes are written to k_codes and one table row is
 * appended.  Appending in chunks gives the same bytes as appending one token
 * at a time.
 *   k_new, v_new: device [B][Hkv][n_new][D] in_dtype.  n_new >= 1.
 * Errors: KVQ_ERR_CAPACITY if n_stored + n_new > capacity (nothing evicts
 * automatically; [P1] "Implementation": append, then evict);
 * KVQ_ERR_UNSUPPORTED for KVQ_CENTER_K on a kind other than TOK_SYM4 (or
 * PLAIN with KVQ_TEST_CENTER_ANY) -- the Q4_0-only gate of [P3].           */
kvq_status kvq_quantize_append(const kvq_layout* layout, kvq_cache* cache,
                               const void* k_new, const void* v_new,
                               int32_t n_new, void* stream);

/* kvq_quantize_append for rows that carry their own positions: SnapKV-kept
 * rows stacked into a quantized cache ([P2] "SnapKV-adapted": any quantizer
 * can be stacked on the kept tokens; "RoPE position semantics": kept rows
 * keep their true absolute positions).  Rows [0, n_new) of each (batch,
 * kv-head) slice are appended exactly as kvq_quantize_append would.
 *   k_new, v_new  device [B][Hkv][src_rows][D] in_dtype; src_rows >= n_new,
 *                 0 means n_new (e.g. a kvq_snapkv_state: src_rows = its
 *                 capacity).
 *   positions     device int32: [B][Hkv][pos_rows] with KVQ_POS_PER_HEAD
 *                 (pos_rows >= n_new, 0 means n_new), else [n_new].  Copied
 *                 into the new slots' positions as given.
 *   next_pos      the cache's generation counter afterwards (the prompt
 *                 length for kept prefill rows); later kvq_quantize_append
 *                 calls continue from it.  Must be >= the current counter
 *                 and >= n_stored + n_new; positions themselves are not
 *                 inspected on the host.
 * Errors as kvq_quantize_append, plus KVQ_ERR_INVALID_ARG for a missing
 * positions array, src_rows or pos_rows below n_new, or next_pos below the
 * current counter or the stored count.                                    */
kvq_status kvq_quantize_append_at(const kvq_layout* layout, kvq_cache* cache,
                                  const void* k_new, const void* v_new, int32_t n_new,
                                  int32_t src_rows, const int32_t* positions,
                                  int32_t pos_rows, int32_t next_pos, void* stream);

/* Workspace bytes kvq_decode_attention needs for this layout (any fill). */
size_t kvq_decode_workspace_bytes(const kvq_layout* layout, int32_t n_q_heads);

/* Decode attention for one query token per sequence ([P4] s.1: scores
 * against the packed keys, softmax, weighted sum of the packed values; no
 * dequantized buffer of K or V is ever written; [P4] s.5: split over the token
 * axis for long caches).
 *   out[b][hq][:] = sum_t softmax_t(sm_scale * q[b][hq] . k_t) v_t
 * over the n_stored slots of kv-head hk = hq / (n_q_heads / Hkv), where k_t,
 * v_t are the dequantized entries (KIVI_CH residual keys as stored).
 * Centered keys are attended as stored: the per-row constant q.k_bar does not
 * change the softmax ([P3] "Why this is safe").
 *   q: device [B][n_q_heads][D] of q_dtype; out: device [B][n_q_heads][D] fp32.
 *   sm_scale <= 0 selects 1/sqrt(D).  n_q_heads must be a multiple of Hkv with
 *   at most 8 query heads per kv-head.
 *   ws: device workspace of at least kvq_decode_workspace_bytes bytes.
 * An empty cache (n_stored == 0) writes zeros.                              */
kvq_status kvq_decode_attention(const kvq_layout* layout, const kvq_cache* cache,
                                const void* q, int32_t q_dtype, int32_t n_q_heads,
                                float sm_scale, float* out,
                                void* ws, size_t ws_bytes, void* stream);

/* kvq_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  The split partials live in a fixed
 * scratch array of KVQ_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends; its address is looked up once
 * per device, on the first call with that device current.  Nothing is
 * allocated or freed by the call itself.
 *   Arguments, layout and results as kvq_decode_attention.
 *   The scratch is shared by every call on one GPU and keeps the last call's
 *   partials: calls that overlap on one GPU (different streams, or several
 *   host threads) race and must be ordered by the caller.
 * Errors as kvq_decode_attention (never KVQ_ERR_WORKSPACE), plus
 * KVQ_ERR_SCRATCH when the split partials of this call (B * n_q_heads *
 * splits * (head_dim + 2) fp32) exceed the scratch: every layout of the
 * per-token 4-bit-key or KIVI 4-bit-key kernels fits, the LDS-tiled kernel
 * of the other layouts fits while B * n_q_heads <= 16129 at head_dim 128.  */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_layout* layout, const kvq_cache* cache,
                                        const void* q, int32_t q_dtype, int32_t n_q_heads,
                                        float sm_scale, float* out, void* stream);

/* Multi-query attention over the cache: a prefill chunk of n_q queries per
 * head ([P4] s.5: the fused-attention microbenchmark shape, 128 queries with
 * GQA 4:1 over a long cache, where attention is a dense contraction).  Row
 * (b, hq, i) is the decode of query i of head hq over the cache's slots
 * [0, T) (T = n_stored), or with causal = 1 -- the chunk's own rows being
 * the cache's last n_q slots -- over slots [0, T - n_q + i].
 *   q    device [B][Hq][n_q][D] (q_dtype), before any position rotation
 *   out  device [B][Hq][n_q][D] fp32
 *   ws   at least kvq_prefill_workspace_bytes(layout, Hq, n_q) bytes
 * The products run on the matrix cores per 64-token tile: 4-bit per-token
 * affine keys in groups of 64 or 128 channels (fp16 or bf16 queries) enter
 * as their codes with the group scales and zero points applied to the sums;
 * other keys are unpacked to an fp16 pair (rounded value and residual);
 * values and probabilities enter as fp16; scores, softmax and accumulation
 * are fp32.  Errors as kvq_decode_attention, plus KVQ_ERR_INVALID_ARG for
 * n_q < 1, causal not 0/1 or a causal chunk longer than the cache;
 * KVQ_ERR_UNSUPPORTED for B > 65535, Hkv * ceil(Hq / Hkv * n_q / 128) >
 * 65535, or more than 2^30 workgroups in one launch.                        */
size_t kvq_prefill_workspace_bytes(const kvq_layout* layout, int32_t n_q_heads, int32_t n_q);
kvq_status kvq_prefill_attention(const kvq_layout* layout, const kvq_cache* cache, const void* q,
                                 int32_t q_dtype, int32_t n_q_heads, int32_t n_q, float sm_scale,
                                 int32_t causal, float* out, void* ws, size_t ws_bytes, void* stream);

/* RoPE on read for StreamingLLM re-positioning ([P1] "RoPE caveat": keys
 * are stored before the rotary embedding and rotated when read, at their
 * slot index in the compressed cache, so sink and window keys sit at
 * consecutive positions).  The rotation is the half-split form: for j < D/2
 * the pair (x_j, x_{j+D/2}) turns by pos * base^(-2j/D).
 *
 * kvq_rope_table fills table (device [n_pos][D/2][2] fp32: cos, sin of each
 * angle, computed in fp64).  base > 1 (10000 is the usual value).          */
kvq_status kvq_rope_table(float* table, int32_t n_pos, int32_t head_dim, float base,
                          void* stream);

/* kvq_decode_attention with RoPE applied on read: the key of slot t is
 * rotated at position t (its index in the compressed cache), the query
 * (also given before the rotation) at q_pos -- for the newest token usually
 * its own slot, n_stored - 1.  rope_table from kvq_rope_table with
 * table_rows >= max(n_stored, q_pos + 1) rows.  Runs the LDS-tiled kernel
 * for every layout.  Errors as kvq_decode_attention, plus
 * KVQ_ERR_INVALID_ARG for a missing table, q_pos outside [0, table_rows) or
 * n_stored > table_rows.                                                   */
kvq_status kvq_decode_attention_rope(const kvq_layout* layout, const kvq_cache* cache,
                                     const void* q, int32_t q_dtype, int32_t n_q_heads,
                                     float sm_scale, const float* rope_table,
                                     int32_t table_rows, int32_t q_pos, float* out, void* ws,
                                     size_t ws_bytes, void* stream);

/* StreamingLLM compaction ([P1] "Implementation", "StreamingLLM"): when
 * n_stored > sink + window, copy slots [0, sink) and the last `window` slots,
 * in order, from src into dst (out-of-place; dst has the same layout and its
 * own buffers, which must not overlap src's).  Codes, metadata, positions and
 * residual keys are copied bit-for-bit; nothing is re-quantized.  KIVI_CH
 * table rows no kept slot refers to are dropped and k_row is renumbered
 * ([P1]: per-channel K scales are not sliced by eviction).
 * Returns KVQ_NOOP (nothing enqueued, dst untouched) when n_stored <= sink +
 * window.  KIVI_CH requires window >= k_group (the open group is never
 * evicted) and that the kept positions form at most two runs (the sink
 * prefix and one run of consecutive positions): KVQ_ERR_UNSUPPORTED otherwise.
 * On success dst's counters are set (n_stored = sink + window).            */
kvq_status kvq_evict_streaming(const kvq_layout* layout, const kvq_cache* src,
                               kvq_cache* dst, int32_t sink, int32_t window,
                               void* stream);

/* Workspace bytes for kvq_snapkv_select (0 for invalid or unsupported sizes). */
size_t kvq_snapkv_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t seq_len,
                                  int32_t head_dim, int32_t obs_window);

/* SnapKV prefill selection ([P2] "How it works"):
 *   1. scores[j] = mean over the last w' = min(obs_window, S) key rows i of
 *      softmax_j(K[i] . K[j] / sqrt(D))  (keys stand in for queries; no mask)
 *   2. the first n_s = min(n_sink, n_keep) positions are always kept
 *   3. the top n_keep - n_s of the other positions by score are added
 *      (equal scores: lower position first), n_keep = min(budget, S)
 *   4. kept positions in ascending order; K/V rows gathered in that order.
 *   k, v:        device [B][Hkv][S][D] fp16
 *   scores:      device [B][Hkv][S] fp32 output, or NULL (kept in workspace)
 *   kept:        device [B][Hkv][n_keep] int32 output
 *   k_out,v_out: device [B][Hkv][n_keep][D] fp16 outputs
 * obs_window and budget >= 1, n_sink >= 0; D in {32, 64, 128}; obs_window <= 128.
 * Clamps (obs_window > S, budget >= S, n_sink > budget) are not errors.     */
kvq_status kvq_snapkv_select(const void* k, const void* v, int32_t batch,
                             int32_t n_kv_heads, int32_t seq_len, int32_t head_dim,
                             int32_t obs_window, int32_t n_sink, int32_t budget,
                             float* scores, int32_t* kept, void* k_out, void* v_out,
                             void* ws, size_t ws_bytes, void* stream);

/* How kvq_snapkv_select computes step 1.  Where every (b, h, key chunk)
 * workgroup fits on the device at once (S <= 32768, n_keep <= 4096), the keys
 * are read once: each workgroup keeps its chunk's logits in registers while
 * the chunks of a head exchange their per-row softmax statistics through the
 * workspace, and the select launch that follows clears the exchange flags
 * (two launches per call).  Otherwise the logits are computed twice, in a
 * statistics pass and a scores pass (three launches).  A workgroup waits for
 * the rest of its head for at most the time set here (default 200 us; it
 * then recomputes the head's statistics itself, which gives the same
 * result); 0 makes every late workgroup take that path at once.  Calls that
 * share one workspace must not overlap.  Returns the previous limit;
 * negative values are ignored.                                              */
int32_t kvq_snapkv_set_wait_us(int32_t microseconds);

/* Steps 2-4 of kvq_snapkv_select without the gather, from given scores
 * [B][Hkv][S] fp32 (finite; -0 ranks as +0).  kept: [B][Hkv][n_keep].     */
kvq_status kvq_snapkv_select_from_scores(const float* scores, int32_t batch,
                                         int32_t n_kv_heads, int32_t seq_len,
                                         int32_t n_sink, int32_t budget,
                                         int32_t* kept, void* stream);

/* SnapKV variants of the paper that the page leaves out ([P2] "Proxy
 * limitation"): the prompt's final query vectors as the observation window,
 * and max-pool smoothing of the scores before ranking.
 *   q_window     device [B][n_q_heads][obs_window][D] fp16 queries, or NULL:
 *                the last obs_window key rows stand in for them (the page's
 *                proxy).  With queries, a kv-head's score is the mean over
 *                all n_q_heads/Hkv * obs_window rows of its query-head group
 *                (query head hq belongs to kv-head hq / (n_q_heads / Hkv)).
 *   n_q_heads    query heads when q_window is set: a multiple of Hkv, with
 *                (n_q_heads / Hkv) * obs_window <= 128 and obs_window <= S
 *                (the window is the prompt's own last queries).
 *   pool_kernel  odd width 1..31: positions are ranked by the maximum score
 *                over [j - (w-1)/2, j + (w-1)/2] (clipped at the ends); 1 = none.
 *                The scores output stays unpooled.                           */
typedef struct kvq_snapkv_opts {
    const void* q_window;
    int32_t n_q_heads;
    int32_t pool_kernel;
} kvq_snapkv_opts;

/* Workspace bytes for kvq_snapkv_select_ex (opts NULL: as kvq_snapkv_select;
 * 0 for invalid or unsupported options or sizes).                           */
size_t kvq_snapkv_workspace_bytes_ex(const kvq_snapkv_opts* opts, int32_t batch, int32_t n_kv_heads,
                                     int32_t seq_len, int32_t head_dim, int32_t obs_window);

/* kvq_snapkv_select with the options above (opts NULL gives the same result
 * as kvq_snapkv_select).  Errors as kvq_snapkv_select, plus
 * KVQ_ERR_INVALID_ARG for an even or non-positive pool_kernel, n_q_heads
 * not a positive multiple of Hkv or obs_window > S with q_window set;
 * KVQ_ERR_ALIGNMENT for a q_window not 16-byte aligned; KVQ_ERR_UNSUPPORTED for pool_kernel > 31
 * or more than 128 observation rows per kv-head.                            */
kvq_status kvq_snapkv_select_ex(const kvq_snapkv_opts* opts, const void* k, const void* v,
                                int32_t batch, int32_t n_kv_heads, int32_t seq_len, int32_t head_dim,
                                int32_t obs_window, int32_t n_sink, int32_t budget, float* scores,
                                int32_t* kept, void* k_out, void* v_out, void* ws, size_t ws_bytes,
                                void* stream);

/* Max-pool smoothing alone: pooled[b][h][j] = max of scores[b][h][j'] over
 * |j' - j| <= (pool_kernel - 1) / 2, 0 <= j' < S.  Device [B][Hkv][S] fp32;
 * pooled must not overlap scores.  pool_kernel odd, 1..31.                  */
kvq_status kvq_snapkv_pool_scores(const float* scores, float* pooled, int32_t batch,
                                  int32_t n_kv_heads, int32_t seq_len, int32_t pool_kernel,
                                  void* stream);

/* Chunked SnapKV prefill ([P2] "How it works": every prefill call scores
 * and selects again, so the budget holds across chunks; "RoPE position
 * semantics": kept rows keep their absolute positions, and decode appends
 * never pass through the selection).  A state holds the rows kept so far:
 *   k, v      device [B][Hkv][capacity][D] fp16, rows [0, n_kept) in
 *             ascending position order
 *   pos       device [B][Hkv][capacity] int32 absolute positions of the rows
 *   n_kept    host counter; next_pos  host: position of the next prompt token
 * Zero the counters for an empty state.                                     */
typedef struct kvq_snapkv_state {
    void* k;
    void* v;
    int32_t* pos;
    int32_t capacity;
    int32_t n_kept;
    int32_t next_pos;
} kvq_snapkv_state;

/* Workspace bytes for kvq_snapkv_prefill_chunk with an `in` state of the
 * given capacity (0 for invalid or unsupported sizes or options). */
size_t kvq_snapkv_chunk_workspace_bytes(const kvq_snapkv_opts* opts, int32_t batch,
                                        int32_t n_kv_heads, int32_t head_dim,
                                        int32_t capacity, int32_t obs_window);

/* One prefill chunk.  The chunk's rows (device [B][Hkv][chunk_len][D] fp16,
 * positions in->next_pos + i) are first written after the kept rows of `in`
 * (in->n_kept grows by chunk_len, in->next_pos by chunk_len).  Then SnapKV
 * (kvq_snapkv_select_ex, with opts) runs over those n = n_kept + chunk_len
 * candidate rows: the observation window is the last min(obs_window, n)
 * candidate key rows, or opts->q_window (the queries of the chunk's last
 * obs_window tokens, obs_window <= n).  The sinks are the first n_sink
 * candidates, which are the prompt's first positions once they were kept.
 * The min(budget, n) selected rows and their positions go to rows [0,
 * n_keep) of `out` in ascending order; out->n_kept = n_keep and
 * out->next_pos = in->next_pos.  Pass `out` as `in` for the next chunk.
 *   scores  optional device [B][Hkv][n] fp32 (unpooled scores of the
 *           candidates), or NULL.
 * Errors: KVQ_ERR_CAPACITY when n > in->capacity or n_keep > out->capacity;
 * KVQ_ERR_INVALID_ARG for overlapping states, missing buffers and the
 * argument errors of kvq_snapkv_select_ex; KVQ_ERR_WORKSPACE, ALIGNMENT and
 * UNSUPPORTED as there.                                                     */
kvq_status kvq_snapkv_prefill_chunk(const kvq_snapkv_opts* opts, kvq_snapkv_state* in,
                                    kvq_snapkv_state* out, const void* k_chunk,
                                    const void* v_chunk, int32_t chunk_len, int32_t batch,
                                    int32_t n_kv_heads, int32_t head_dim, int32_t obs_window,
                                    int32_t n_sink, int32_t budget, float* scores, void* ws,
                                    size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* kvq_status_string(kvq_status status);

/* KVQ_VERSION of the built library. */
int32_t kvq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */

// api.hip -- host side of the libkvq C ABI: validation, buffer sizing,
// host counters and kernel dispatch.  No call allocates, frees or
// synchronizes; every argument is checked before anything is enqueued.
#include <math.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

int esize(int dt) { return dt == KVQ_F32 ? 4 : 2; }
bool valid_dtype(int dt) { return dt == KVQ_F32 || dt == KVQ_F16 || dt == KVQ_BF16; }

// Layout checks shared by every call.  Returns KVQ_OK or an error.
kvq_status check_layout(const kvq_layout* L) {
    if (!L) return KVQ_ERR_INVALID_ARG;
    if (L->batch < 1 || L->n_kv_heads < 1 || L->capacity < 1) return KVQ_ERR_INVALID_ARG;
    if (!valid_dtype(L->in_dtype)) return KVQ_ERR_INVALID_ARG;
    if (L->flags & ~(KVQ_CENTER_K | KVQ_TEST_CENTER_ANY | KVQ_POS_PER_HEAD)) return KVQ_ERR_INVALID_ARG;
    const int D = L->head_dim;
    if (D != 32 && D != 64 && D != 128) return D > 0 ? KVQ_ERR_UNSUPPORTED : KVQ_ERR_INVALID_ARG;
    switch (L->k_kind) {
        case KVQ_PLAIN: break;
        case KVQ_KIVI_CH:
            if (L->k_bits != 2 && L->k_bits != 4 && L->k_bits != 8) return KVQ_ERR_UNSUPPORTED;
            if (!is_pow2(L->k_group) || L->k_group < 8 || L->k_group > 128) return KVQ_ERR_UNSUPPORTED;
            break;
        case KVQ_TOK_AFFINE:
            if (L->k_bits != 2 && L->k_bits != 4 && L->k_bits != 8) return KVQ_ERR_UNSUPPORTED;
            if ((L->k_group != 32 && L->k_group != 64 && L->k_group != 128) || L->k_group > D)
                return KVQ_ERR_UNSUPPORTED;
            break;
        case KVQ_TOK_SYM4:
            if (L->k_bits != 4 || L->k_group != 32) return KVQ_ERR_UNSUPPORTED;
            break;
        default: return KVQ_ERR_INVALID_ARG;
    }
    switch (L->v_kind) {
        case KVQ_PLAIN: break;
        case KVQ_TOK_AFFINE:
            if (L->v_bits != 2 && L->v_bits != 4 && L->v_bits != 8) return KVQ_ERR_UNSUPPORTED;
            if ((L->v_group != 32 && L->v_group != 64 && L->v_group != 128) || L->v_group > D)
                return KVQ_ERR_UNSUPPORTED;
            break;
        case KVQ_KIVI_CH: case KVQ_TOK_SYM4: return KVQ_ERR_UNSUPPORTED;   // K-only kinds
        default: return KVQ_ERR_INVALID_ARG;
    }
    if (L->flags & KVQ_CENTER_K) {
        // Mean-centering is gated to the symmetric 4-bit K format (the
        // zero-point formats already absorb a static mean); PLAIN keys are
        // allowed only through the test seam.
        const bool ok = L->k_kind == KVQ_TOK_SYM4 ||
                        (L->k_kind == KVQ_PLAIN && (L->flags & KVQ_TEST_CENTER_ANY));
        if (!ok) return KVQ_ERR_UNSUPPORTED;
        // the seam stores centered keys at full precision: fp32 only
        if (L->k_kind == KVQ_PLAIN && L->in_dtype != KVQ_F32) return KVQ_ERR_UNSUPPORTED;
    }
    return KVQ_OK;
}

int table_rows(const kvq_layout* L) {
    return L->k_kind == KVQ_KIVI_CH ? L->capacity / L->k_group + 3 : 0;
}

void sizes_of(const kvq_layout* L, kvq_sizes* s) {
    memset(s, 0, sizeof *s);
    const size_t BH = (size_t)L->batch * L->n_kv_heads;
    const size_t C = (size_t)L->capacity, D = (size_t)L->head_dim;
    switch (L->k_kind) {
        case KVQ_PLAIN: s->k_codes = BH * C * D * esize(L->in_dtype); break;
        case KVQ_KIVI_CH:
            s->k_codes = BH * C * D * L->k_bits / 8;
            s->k_table_rows = table_rows(L);
            s->k_meta = BH * (size_t)s->k_table_rows * D * 2 * 2;
            s->k_resid = BH * (size_t)L->k_group * D * esize(L->in_dtype);
            s->k_row = C * 4;
            break;
        case KVQ_TOK_AFFINE:
            s->k_codes = BH * C * D * L->k_bits / 8;
            s->k_meta = BH * C * (D / L->k_group) * 2 * 2;
            break;
        case KVQ_TOK_SYM4:
            s->k_codes = BH * C * D / 2;
            s->k_meta = BH * C * (D / 32) * 2;
            break;
    }
    if (L->v_kind == KVQ_PLAIN) {
        s->v_codes = BH * C * D * esize(L->in_dtype);
    } else {
        s->v_codes = BH * C * D * L->v_bits / 8;
        s->v_meta = BH * C * (D / L->v_group) * 2 * 2;
    }
    s->pos = ((L->flags & KVQ_POS_PER_HEAD) ? BH : 1) * C * 4;
}

// Device buffers a layout needs must be present and aligned.
kvq_status check_cache(const kvq_layout* L, const kvq_cache* c) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (c->n_stored < 0 || c->n_stored > L->capacity || c->n_quant < 0 || c->n_quant > c->n_stored ||
        c->next_pos < c->n_stored || c->n_head < 0 || c->n_head > c->n_stored)
        return KVQ_ERR_INVALID_ARG;
    if (L->k_kind != KVQ_KIVI_CH && c->n_quant != c->n_stored) return KVQ_ERR_INVALID_ARG;
    if (L->k_kind == KVQ_KIVI_CH && c->n_stored - c->n_quant >= L->k_group)
        return KVQ_ERR_INVALID_ARG;
    const void* need[8] = {c->k_codes, c->v_codes, c->pos, nullptr, nullptr, nullptr, nullptr, nullptr};
    int n = 3;
    if (L->k_kind != KVQ_PLAIN) need[n++] = c->k_meta;
    if (L->k_kind == KVQ_KIVI_CH) { need[n++] = c->k_resid; need[n++] = c->k_row; }
    if (L->v_kind != KVQ_PLAIN) need[n++] = c->v_meta;
    for (int i = 0; i < n; ++i) if (!need[i]) return KVQ_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i) if (!aligned16(need[i])) return KVQ_ERR_ALIGNMENT;
    if (L->flags & KVQ_CENTER_K) {
        if (!c->k_bias) return KVQ_ERR_INVALID_ARG;
        if (!aligned16(c->k_bias)) return KVQ_ERR_ALIGNMENT;
    }
    return KVQ_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

int32_t kvq_version(void) { return KVQ_VERSION; }

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_NOOP: return "nothing to do";
        case KVQ_ERR_INVALID_ARG: return "invalid argument";
        case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case KVQ_ERR_CAPACITY: return "cache capacity exceeded";
        case KVQ_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
        case KVQ_ERR_HIP: return "HIP runtime or launch error";
        case KVQ_ERR_SCRATCH: return "request exceeds the fixed scratch of the no-allocation call";
    }
    return "unknown status";
}

kvq_status kvq_cache_sizes(const kvq_layout* L, kvq_sizes* out) {
    if (!out) return KVQ_ERR_INVALID_ARG;
    const kvq_status st = check_layout(L);
    if (st != KVQ_OK) return st;
    sizes_of(L, out);
    return KVQ_OK;
}

kvq_status kvq_cache_reset(kvq_cache* c) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    c->n_stored = c->n_quant = c->next_pos = c->n_head = 0;
    return KVQ_OK;
}

// Append n_new rows of each (b, h) slice (slices src_rows rows apart) at
// positions pos_src (null: c->next_pos + i), then set the generation
// counter to next_after.
static kvq_status append_impl(const kvq_layout* L, kvq_cache* c, const void* k_new, const void* v_new,
                              int32_t n_new, int32_t src_rows, const int32_t* pos_src, int32_t pos_rows,
                              int64_t next_after, hipStream_t s) {
    const int B = L->batch, H = L->n_kv_heads, D = L->head_dim;

    // V rows, per-token K rows and positions: one launch; values are
    // quantized once, at write time.
    RowAppendArgs ra{};
    ra.rows.B = B; ra.rows.H = H; ra.rows.n = n_new; ra.rows.D = D; ra.rows.cap = L->capacity;
    ra.rows.slot0 = c->n_stored; ra.rows.in_dtype = L->in_dtype; ra.rows.src_rows = src_rows;
    ra.k_src = k_new; ra.k_codes = c->k_codes; ra.k_meta = c->k_meta;
    ra.k_bias = (L->flags & KVQ_CENTER_K) ? c->k_bias : nullptr;
    ra.k_kind = L->k_kind; ra.k_bits = L->k_bits; ra.k_group = L->k_group;
    ra.v_src = v_new; ra.v_codes = c->v_codes; ra.v_meta = c->v_meta;
    ra.v_kind = L->v_kind; ra.v_bits = L->v_bits; ra.v_group = L->v_group;
    ra.pos = c->pos; ra.first_pos = c->next_pos;
    ra.pos_src = pos_src; ra.pos_src_rows = pos_rows; ra.pos_per_head = (L->flags & KVQ_POS_PER_HEAD) ? 1 : 0;
    hipError_t e = launch_row_append(ra, s);
    if (e != hipSuccess) return KVQ_ERR_HIP;

    int new_quant = c->n_stored + n_new;
    if (L->k_kind == KVQ_KIVI_CH) {
        // per-channel keys: the residual group fills and closes separately
        ChannelQuantArgs k{};
        k.k_new = k_new; k.resid = c->k_resid; k.codes = c->k_codes; k.table = c->k_meta;
        k.k_row = c->k_row;
        k.B = B; k.H = H; k.D = D; k.cap = L->capacity; k.rows = table_rows(L);
        k.Gt = L->k_group; k.bits = L->k_bits; k.in_dtype = L->in_dtype;
        k.r0 = c->n_stored - c->n_quant;
        k.n_new = n_new;
        k.src_rows = src_rows;
        k.n_quant = c->n_quant;
        k.n_groups = (k.r0 + n_new) / L->k_group;
        e = launch_channel_quant(k, s);
        if (e != hipSuccess) return KVQ_ERR_HIP;
        new_quant = c->n_quant + k.n_groups * L->k_group;
    }

    if (c->n_head == c->n_stored) c->n_head += n_new;   // never evicted: slots in append order
    c->n_stored += n_new;
    c->next_pos = (int32_t)next_after;
    c->n_quant = new_quant;
    return KVQ_OK;
}

kvq_status kvq_quantize_append(const kvq_layout* L, kvq_cache* c, const void* k_new,
                               const void* v_new, int32_t n_new, void* stream) {
    kvq_status st = check_layout(L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, c)) != KVQ_OK) return st;
    if (n_new < 1 || !k_new || !v_new) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGNMENT;
    if ((int64_t)c->n_stored + n_new > L->capacity) return KVQ_ERR_CAPACITY;
    if ((int64_t)c->next_pos + n_new > INT32_MAX) return KVQ_ERR_CAPACITY;
    return append_impl(L, c, k_new, v_new, n_new, n_new, nullptr, 0, (int64_t)c->next_pos + n_new,
                       static_cast<hipStream_t>(stream));
}

kvq_status kvq_quantize_append_at(const kvq_layout* L, kvq_cache* c, const void* k_new, const void* v_new,
                                  int32_t n_new, int32_t src_rows, const int32_t* positions,
                                  int32_t pos_rows, int32_t next_pos, void* stream) {
    kvq_status st = check_layout(L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, c)) != KVQ_OK) return st;
    if (n_new < 1 || !k_new || !v_new || !positions) return KVQ_ERR_INVALID_ARG;
    if (src_rows == 0) src_rows = n_new;
    if (pos_rows == 0) pos_rows = n_new;
    if (src_rows < n_new || pos_rows < n_new) return KVQ_ERR_INVALID_ARG;
    if (next_pos < c->next_pos || next_pos < c->n_stored + n_new) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(positions)) return KVQ_ERR_ALIGNMENT;
    // row starts of every slice must stay 16-byte aligned
    if (((int64_t)src_rows * L->head_dim * esize(L->in_dtype)) % 16 != 0) return KVQ_ERR_ALIGNMENT;
    if ((int64_t)c->n_stored + n_new > L->capacity) return KVQ_ERR_CAPACITY;
    return append_impl(L, c, k_new, v_new, n_new, src_rows, positions,
                       (L->flags & KVQ_POS_PER_HEAD) ? pos_rows : 0, next_pos,
                       static_cast<hipStream_t>(stream));
}

size_t kvq_decode_workspace_bytes(const kvq_layout* L, int32_t n_q_heads) {
    if (check_layout(L) != KVQ_OK || n_q_heads < 1) return 0;
    return decode_workspace_bytes(L->batch, n_q_heads, L->head_dim, L->capacity);
}

// Kernel arguments and split plan of one decode (workspace pointers unset).
static DecodeArgs decode_args(const kvq_layout* L, const kvq_cache* c, const void* q, int32_t q_dtype,
                              int32_t n_q_heads, float sm_scale, const float* rope, int32_t q_pos, float* out) {
    const int D = L->head_dim;
    DecodeArgs a{};
    a.k_codes = c->k_codes; a.k_meta = c->k_meta; a.k_resid = c->k_resid;
    a.v_codes = c->v_codes; a.v_meta = c->v_meta; a.k_row = c->k_row;
    a.q = q; a.out = out;
    a.B = L->batch; a.Hkv = L->n_kv_heads; a.Hq = n_q_heads; a.D = D; a.cap = L->capacity;
    a.T = c->n_stored; a.n_quant = c->n_quant; a.Gt = L->k_group;
    a.k_kind = L->k_kind; a.k_bits = L->k_bits; a.k_group = L->k_group;
    a.v_kind = L->v_kind; a.v_bits = L->v_bits; a.v_group = L->v_group;
    a.in_dtype = L->in_dtype; a.q_dtype = q_dtype;
    a.rope = rope; a.q_pos = q_pos;
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)D);
    a.scale_log2 = scale * 1.4426950408889634f;
    if (decode_fast_applies(a)) decode_fast_plan(a.B, a.Hkv, a.T, a.v_bits, &a.n_splits, &a.split_len);
    else decode_plan(a.B, a.Hkv, a.T, &a.n_splits, &a.split_len);
    return a;
}

// Split partials the launch writes: B Hq n_splits (D + 2) fp32, none when the
// fast kernels run unsplit (they then write the output directly).
static size_t decode_partial_bytes(const DecodeArgs& a) {
    if (a.n_splits == 1 && decode_fast_applies(a)) return 0;
    return (size_t)a.B * a.Hq * a.n_splits * (a.D + 2) * sizeof(float);
}

static kvq_status decode_launch(DecodeArgs& a, void* ws, hipStream_t s) {
    a.ws_o = static_cast<float*>(ws);
    a.ws_ml = a.ws_o + (size_t)a.B * a.Hq * a.n_splits * a.D;
    return hip_status(launch_decode(a, s));
}

static kvq_status decode_impl(const kvq_layout* L, const kvq_cache* c, const void* q, int32_t q_dtype,
                              int32_t n_q_heads, float sm_scale, const float* rope, int32_t q_pos, float* out,
                              void* ws, size_t ws_bytes, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = L->head_dim;
    if (c->n_stored == 0)
        return hip_status(launch_zero_f32(out, (size_t)L->batch * n_q_heads * D, s));
    const size_t need = decode_workspace_bytes(L->batch, n_q_heads, D, L->capacity);
    if (!ws || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    if (!aligned16(ws)) return KVQ_ERR_ALIGNMENT;
    DecodeArgs a = decode_args(L, c, q, q_dtype, n_q_heads, sm_scale, rope, q_pos, out);
    return decode_launch(a, ws, s);
}

static kvq_status decode_check(const kvq_layout* L, const kvq_cache* c, const void* q, int32_t q_dtype,
                               int32_t n_q_heads, float sm_scale, float* out) {
    kvq_status st = check_layout(L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, c)) != KVQ_OK) return st;
    if (!q || !out || !valid_dtype(q_dtype)) return KVQ_ERR_INVALID_ARG;
    if (n_q_heads < 1 || n_q_heads % L->n_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
    if (n_q_heads / L->n_kv_heads > 8) return KVQ_ERR_UNSUPPORTED;
    if (!(sm_scale == sm_scale) || isinf(sm_scale)) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_ALIGNMENT;
    return KVQ_OK;
}

kvq_status kvq_decode_attention(const kvq_layout* L, const kvq_cache* c, const void* q,
                                int32_t q_dtype, int32_t n_q_heads, float sm_scale, float* out,
                                void* ws, size_t ws_bytes, void* stream) {
    kvq_status st = decode_check(L, c, q, q_dtype, n_q_heads, sm_scale, out);
    if (st != KVQ_OK) return st;
    return decode_impl(L, c, q, q_dtype, n_q_heads, sm_scale, nullptr, 0, out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- no-allocation decode
// The split partials of kvq_decode_attention_noalloc live in this fixed
// array (KVQ_NOALLOC_SCRATCH_BYTES), one copy per GPU the library runs on.
// Host code never uses the array's name as an address: the device address
// of each GPU's copy comes from hipGetSymbolAddress, looked up once per
// device on the first call with that device current.  Partials are written
// before they are read, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

static kvq_status noalloc_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return KVQ_ERR_HIP;
    *ptr = g_scratch_ptr[dev];
    return KVQ_OK;
}

kvq_status kvq_decode_attention_noalloc(const kvq_layout* L, const kvq_cache* c, const void* q,
                                        int32_t q_dtype, int32_t n_q_heads, float sm_scale, float* out,
                                        void* stream) {
    kvq_status st = decode_check(L, c, q, q_dtype, n_q_heads, sm_scale, out);
    if (st != KVQ_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c->n_stored == 0)
        return hip_status(launch_zero_f32(out, (size_t)L->batch * n_q_heads * L->head_dim, s));
    DecodeArgs a = decode_args(L, c, q, q_dtype, n_q_heads, sm_scale, nullptr, 0, out);
    if (decode_partial_bytes(a) > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_SCRATCH;
    void* ws = nullptr;
    if ((st = noalloc_scratch(&ws)) != KVQ_OK) return st;
    return decode_launch(a, ws, s);
}

kvq_status kvq_decode_attention_rope(const kvq_layout* L, const kvq_cache* c, const void* q, int32_t q_dtype,
                                     int32_t n_q_heads, float sm_scale, const float* rope_table,
                                     int32_t table_rows, int32_t q_pos, float* out, void* ws, size_t ws_bytes,
                                     void* stream) {
    kvq_status st = decode_check(L, c, q, q_dtype, n_q_heads, sm_scale, out);
    if (st != KVQ_OK) return st;
    if (!rope_table || table_rows < 1 || q_pos < 0 || q_pos >= table_rows) return KVQ_ERR_INVALID_ARG;
    if (c->n_stored > table_rows) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(rope_table)) return KVQ_ERR_ALIGNMENT;
    return decode_impl(L, c, q, q_dtype, n_q_heads, sm_scale, rope_table, q_pos, out, ws, ws_bytes, stream);
}

// Workspace of kvq_prefill_attention: partials of the largest split plan a
// cache of this capacity can need (the plan's split count grows with T).
static size_t prefill_ws_bytes(const kvq_layout* L, int Hq, int n_q) {
    const int ns = prefill_max_splits(L->batch, L->n_kv_heads, Hq, n_q, L->capacity);
    return (size_t)L->batch * Hq * n_q * ns * (L->head_dim + 2) * sizeof(float);
}

size_t kvq_prefill_workspace_bytes(const kvq_layout* L, int32_t n_q_heads, int32_t n_q) {
    if (check_layout(L) != KVQ_OK || n_q_heads < 1 || n_q < 1 || n_q_heads % L->n_kv_heads != 0) return 0;
    return prefill_ws_bytes(L, n_q_heads, n_q);
}

kvq_status kvq_prefill_attention(const kvq_layout* L, const kvq_cache* c, const void* q, int32_t q_dtype,
                                 int32_t n_q_heads, int32_t n_q, float sm_scale, int32_t causal, float* out,
                                 void* ws, size_t ws_bytes, void* stream) {
    kvq_status st = decode_check(L, c, q, q_dtype, n_q_heads, sm_scale, out);
    if (st != KVQ_OK) return st;
    if (n_q < 1 || (causal != 0 && causal != 1)) return KVQ_ERR_INVALID_ARG;
    if (causal && c->n_stored < n_q) return KVQ_ERR_INVALID_ARG;     // the chunk must be in the cache
    const int64_t rows = (int64_t)L->batch * n_q_heads * n_q;
    if (rows > INT32_MAX || L->batch > 65535) return KVQ_ERR_UNSUPPORTED;
    const int64_t R = (int64_t)(n_q_heads / L->n_kv_heads) * n_q;
    if ((int64_t)L->n_kv_heads * ((R + 127) / 128) > 65535) return KVQ_ERR_UNSUPPORTED;   // grid rows, 128-row blocks
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = L->head_dim;
    if (c->n_stored == 0) return hip_status(launch_zero_f32(out, (size_t)rows * D, s));
    if (!ws || ws_bytes < prefill_ws_bytes(L, n_q_heads, n_q)) return KVQ_ERR_WORKSPACE;
    if (!aligned16(ws)) return KVQ_ERR_ALIGNMENT;

    DecodeArgs a{};
    a.k_codes = c->k_codes; a.k_meta = c->k_meta; a.k_resid = c->k_resid;
    a.v_codes = c->v_codes; a.v_meta = c->v_meta; a.k_row = c->k_row;
    a.q = q; a.out = out;
    a.B = L->batch; a.Hkv = L->n_kv_heads; a.Hq = n_q_heads; a.D = D; a.cap = L->capacity;
    a.T = c->n_stored; a.n_quant = c->n_quant; a.Gt = L->k_group;
    a.k_kind = L->k_kind; a.k_bits = L->k_bits; a.k_group = L->k_group;
    a.v_kind = L->v_kind; a.v_bits = L->v_bits; a.v_group = L->v_group;
    a.in_dtype = L->in_dtype; a.q_dtype = q_dtype;
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)D);
    a.scale_log2 = scale * 1.4426950408889634f;
    int n_rb = 1;
    prefill_plan(a.B, a.Hkv, a.Hq, n_q, a.T, prefill_factored(a), &n_rb, &a.n_splits, &a.split_len);
    if (a.n_splits > prefill_max_splits(a.B, a.Hkv, a.Hq, n_q, L->capacity)) return KVQ_ERR_WORKSPACE;
    if ((int64_t)a.n_splits * a.Hkv * n_rb * a.B > (1 << 30)) return KVQ_ERR_UNSUPPORTED;   // workgroups of one launch
    a.ws_o = static_cast<float*>(ws);
    a.ws_ml = a.ws_o + (size_t)rows * a.n_splits * D;
    return hip_status(launch_prefill_attention(a, n_q, n_rb, causal, s));
}

kvq_status kvq_rope_table(float* table, int32_t n_pos, int32_t head_dim, float base, void* stream) {
    if (!table || n_pos < 1) return KVQ_ERR_INVALID_ARG;
    if (head_dim != 32 && head_dim != 64 && head_dim != 128)
        return head_dim > 0 ? KVQ_ERR_UNSUPPORTED : KVQ_ERR_INVALID_ARG;
    if (!(base > 1.0f) || isinf(base)) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(table)) return KVQ_ERR_ALIGNMENT;
    return hip_status(launch_rope_table(table, n_pos, head_dim, (double)base, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_evict_streaming(const kvq_layout* L, const kvq_cache* src, kvq_cache* dst,
                               int32_t sink, int32_t window, void* stream) {
    kvq_status st = check_layout(L);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(L, src)) != KVQ_OK) return st;
    if (!dst) return KVQ_ERR_INVALID_ARG;
    if (sink < 0 || window < 1) return KVQ_ERR_INVALID_ARG;
    const int n = src->n_stored;
    if ((int64_t)sink + window >= n) return KVQ_NOOP;
    // dst buffers: present, aligned, disjoint from src
    kvq_cache probe = *dst;
    probe.n_stored = probe.n_quant = probe.next_pos = probe.n_head = 0;
    if ((st = check_cache(L, &probe)) != KVQ_OK) return st;
    kvq_sizes sz;
    sizes_of(L, &sz);
    const void* sp[7] = {src->k_codes, src->k_meta, src->k_resid, src->v_codes, src->v_meta, src->pos, src->k_row};
    const void* dp[7] = {dst->k_codes, dst->k_meta, dst->k_resid, dst->v_codes, dst->v_meta, dst->pos, dst->k_row};
    const size_t nb[7] = {sz.k_codes, sz.k_meta, sz.k_resid, sz.v_codes, sz.v_meta, sz.pos, sz.k_row};
    for (int i = 0; i < 7; ++i)
        for (int j = 0; j < 7; ++j)
            if (overlaps(sp[i], nb[i], dp[j], nb[j])) return KVQ_ERR_INVALID_ARG;
    const int r = n - src->n_quant;                    // open K group (KIVI_CH)
    if (L->k_kind == KVQ_KIVI_CH) {
        if (window < L->k_group) return KVQ_ERR_INVALID_ARG;
        // kept positions must stay two runs: the sink prefix (positions ==
        // slots) and one run of consecutive positions
        const int h = src->n_head;
        const bool fresh = (h == n);
        if (!fresh && (sink > h || n - window < h)) return KVQ_ERR_UNSUPPORTED;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = L->head_dim;
    EvictArgs a{};
    int nbuf = 0;
    auto add = [&](const void* sptr, void* dptr, size_t row_bytes) {
        a.src[nbuf] = sptr; a.dst[nbuf] = dptr; a.row_bytes[nbuf] = (int)row_bytes; ++nbuf;
    };
    if (L->k_kind == KVQ_PLAIN) add(src->k_codes, dst->k_codes, (size_t)D * esize(L->in_dtype));
    else add(src->k_codes, dst->k_codes, (size_t)D * L->k_bits / 8);
    if (L->k_kind == KVQ_TOK_AFFINE) add(src->k_meta, dst->k_meta, (size_t)(D / L->k_group) * 4);
    if (L->k_kind == KVQ_TOK_SYM4) add(src->k_meta, dst->k_meta, (size_t)(D / 32) * 2);
    if (L->v_kind == KVQ_PLAIN) add(src->v_codes, dst->v_codes, (size_t)D * esize(L->in_dtype));
    else {
        add(src->v_codes, dst->v_codes, (size_t)D * L->v_bits / 8);
        add(src->v_meta, dst->v_meta, (size_t)(D / L->v_group) * 4);
    }
    a.n_buf = nbuf;
    a.src_pos = src->pos; a.dst_pos = dst->pos;
    a.BH = L->batch * L->n_kv_heads; a.cap = L->capacity; a.n = n; a.sink = sink; a.window = window;
    a.pos_per_head = (L->flags & KVQ_POS_PER_HEAD) ? 1 : 0;
    a.n_quant_new = sink + window - (L->k_kind == KVQ_KIVI_CH ? r : 0);
    if (L->k_kind == KVQ_KIVI_CH) {
        a.src_row = src->k_row; a.dst_row = dst->k_row;
        a.src_table = src->k_meta; a.dst_table = dst->k_meta;
        a.table_row_bytes = D * 4; a.rows = table_rows(L);
        a.src_resid = src->k_resid; a.dst_resid = dst->k_resid; a.resid_bytes = sz.k_resid;
    }
    if (launch_evict(a, s) != hipSuccess) return KVQ_ERR_HIP;
    dst->n_stored = sink + window;
    dst->n_quant = a.n_quant_new;
    dst->next_pos = src->next_pos;
    dst->n_head = sink < src->n_head ? sink : src->n_head;
    return KVQ_OK;
}

// Observation rows per kv-head for a SnapKV call: the last min(w, S) key
// rows, or G * w query rows with query windows; -1 when the options are
// invalid, -2 when they are valid but unsupported.
static int snap_rows(const kvq_snapkv_opts* o, int32_t H, int32_t S, int32_t w) {
    int64_t rows = w < S ? w : S;
    if (o && o->q_window) {
        if (o->n_q_heads < H || o->n_q_heads % H != 0 || w > S) return -1;
        rows = (int64_t)(o->n_q_heads / H) * w;
    }
    return rows > 128 ? -2 : (int)rows;
}

static int snap_pool(const kvq_snapkv_opts* o) { return o ? o->pool_kernel : 1; }

size_t kvq_snapkv_workspace_bytes_ex(const kvq_snapkv_opts* opts, int32_t B, int32_t H, int32_t S, int32_t D,
                                     int32_t w) {
    if (B < 1 || H < 1 || S < 1 || w < 1 || (D != 32 && D != 64 && D != 128)) return 0;
    const int rows = snap_rows(opts, H, S, w);
    const int pool = snap_pool(opts);
    if (rows < 1 || pool < 1 || pool % 2 == 0) return 0;
    return snapkv_ws_bytes(B, H, S, D, rows, pool > 1);
}

size_t kvq_snapkv_workspace_bytes(int32_t B, int32_t H, int32_t S, int32_t D, int32_t w) {
    return kvq_snapkv_workspace_bytes_ex(nullptr, B, H, S, D, w);
}

int32_t kvq_snapkv_set_wait_us(int32_t microseconds) {
    const int32_t prev = g_snap_wait_us;
    if (microseconds >= 0) g_snap_wait_us = microseconds;
    return prev;
}

// Tags of the one-read scores' ready flags: distinct for every call of the
// process (a flag left by an earlier call, or stale workspace contents, never
// reads as this call's), never 0 (the cleared value).
static uint64_t snap_next_tag() {
    static std::atomic<uint64_t> next{0x9E3779B97F4A7C15ull ^
                                      (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count()};
    uint64_t t = next.fetch_add(0x9E3779B97F4A7C15ull) * 0xBF58476D1CE4E5B9ull;
    return t ? t : 1u;
}

// The device wall clock's rate (kHz), per device.
static int64_t wall_clock_khz() {
    static int64_t cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100000;
    if (cached[dev] == 0) {
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
            khz = 100000;
        cached[dev] = khz;
    }
    return cached[dev];
}

// One SnapKV pass over S candidate rows per (b, h) (slices kv_stride elements
// apart): scores, optional pooling, selection into kept, gather into
// k_out / v_out (slices out_stride apart) with optional positions.  The
// caller has validated everything; ws holds at least snapkv_ws_bytes.
struct SnapRun {
    const kvq_snapkv_opts* opts;
    const void* k; const void* v; int64_t kv_stride;
    int B, H, S, D, w, n_sink, budget, rows, pool;
    float* scores; int32_t* kept;
    void* k_out; void* v_out; int64_t out_stride;
    const int32_t* pos_in; int pos_in_rows; int32_t* pos_out; int pos_out_rows;
    char* ws;
};

static kvq_status snap_run(const SnapRun& r, hipStream_t s) {
    SnapArgs a{};
    a.k = static_cast<const uint16_t*>(r.k); a.v = static_cast<const uint16_t*>(r.v);
    a.kept = r.kept; a.k_out = static_cast<uint16_t*>(r.k_out); a.v_out = static_cast<uint16_t*>(r.v_out);
    a.B = r.B; a.H = r.H; a.S = r.S; a.D = r.D; a.w = r.w; a.n_sink = r.n_sink; a.budget = r.budget;
    a.n_chunks = (r.S + 127) / 128;
    a.n_rows = r.rows;
    a.kv_stride = r.kv_stride; a.out_stride = r.out_stride;
    a.pos_in = r.pos_in; a.pos_in_rows = r.pos_in_rows; a.pos_out = r.pos_out; a.pos_out_rows = r.pos_out_rows;
    const void* qw = r.opts ? r.opts->q_window : nullptr;
    if (qw) {
        a.obs = static_cast<const uint16_t*>(qw);
        a.obs_stride = (int64_t)r.rows * r.D;
    } else {
        a.obs = a.k + (int64_t)(r.S - r.rows) * r.D;
        a.obs_stride = r.kv_stride;
    }
    size_t stats = (size_t)r.B * r.H * a.n_chunks * r.rows * 2 * sizeof(float);
    stats = (stats + 255) & ~(size_t)255;
    const size_t sc = ((size_t)r.B * r.H * r.S * sizeof(float) + 255) & ~(size_t)255;
    a.stats = reinterpret_cast<float*>(r.ws);
    a.scores = r.scores ? r.scores : reinterpret_cast<float*>(r.ws + stats);
    a.flags = reinterpret_cast<uint64_t*>(r.ws + stats + sc + (r.pool > 1 ? sc : 0));
    if (snapkv_one_read_applies(a)) {
        a.tag = snap_next_tag();
        a.wait_ticks = (int64_t)g_snap_wait_us * wall_clock_khz() / 1000;
        if (launch_snapkv_scores_one_read(a, s) != hipSuccess) return KVQ_ERR_HIP;
    } else {
        a.flags = nullptr;
        if (launch_snapkv_scores(a, s) != hipSuccess) return KVQ_ERR_HIP;
    }
    const float* rank = a.scores;
    if (r.pool > 1) {
        float* pooled = reinterpret_cast<float*>(r.ws + stats + sc);
        if (launch_snapkv_pool(a.scores, pooled, (int64_t)r.B * r.H, r.S, r.pool, s) != hipSuccess)
            return KVQ_ERR_HIP;
        rank = pooled;
    }
    if (launch_snapkv_select_gather(a, rank, s) != hipSuccess) return KVQ_ERR_HIP;
    return KVQ_OK;
}

// Validation common to the SnapKV calls: returns KVQ_OK and the observation
// rows and pool width, or an error.
static kvq_status snap_check(const kvq_snapkv_opts* opts, int32_t B, int32_t H, int32_t S, int32_t D,
                             int32_t w, int32_t n_sink, int32_t budget, int* rows, int* pool) {
    if (B < 1 || H < 1 || S < 1 || w < 1 || budget < 1 || n_sink < 0) return KVQ_ERR_INVALID_ARG;
    if (D != 32 && D != 64 && D != 128) return D > 0 ? KVQ_ERR_UNSUPPORTED : KVQ_ERR_INVALID_ARG;
    *pool = snap_pool(opts);
    if (*pool < 1 || *pool % 2 == 0) return KVQ_ERR_INVALID_ARG;
    if (*pool > 31) return KVQ_ERR_UNSUPPORTED;
    *rows = snap_rows(opts, H, S, w);
    if (*rows == -1) return KVQ_ERR_INVALID_ARG;
    if (*rows == -2) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)B * H * S > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    if (opts && opts->q_window && !aligned16(opts->q_window)) return KVQ_ERR_ALIGNMENT;
    return KVQ_OK;
}

kvq_status kvq_snapkv_select_ex(const kvq_snapkv_opts* opts, const void* k, const void* v, int32_t B, int32_t H,
                                int32_t S, int32_t D, int32_t w, int32_t n_sink, int32_t budget, float* scores,
                                int32_t* kept, void* k_out, void* v_out, void* ws, size_t ws_bytes,
                                void* stream) {
    if (!k || !v || !kept || !k_out || !v_out) return KVQ_ERR_INVALID_ARG;
    int rows = 0, pool = 1;
    kvq_status st = snap_check(opts, B, H, S, D, w, n_sink, budget, &rows, &pool);
    if (st != KVQ_OK) return st;
    const void* ptrs[7] = {k, v, scores, kept, k_out, v_out, ws};
    for (const void* p : ptrs) if (p && !aligned16(p)) return KVQ_ERR_ALIGNMENT;
    const size_t need = snapkv_ws_bytes(B, H, S, D, rows, pool > 1);
    if (!ws || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    const int n_keep = budget < S ? budget : S;
    SnapRun r{opts, k, v, (int64_t)S * D, B, H, S, D, w, n_sink, budget, rows, pool, scores, kept,
              k_out, v_out, (int64_t)n_keep * D, nullptr, 0, nullptr, 0, static_cast<char*>(ws)};
    return snap_run(r, static_cast<hipStream_t>(stream));
}

// Workspace of a prefill chunk: a SnapKV pass over up to `capacity` rows plus
// the kept indices.
static size_t chunk_ws_bytes(int B, int H, int cap, int D, int rows, bool pooled) {
    const size_t kept = ((size_t)B * H * cap * sizeof(int32_t) + 255) & ~(size_t)255;
    return snapkv_ws_bytes(B, H, cap, D, rows, pooled) + kept;
}

size_t kvq_snapkv_chunk_workspace_bytes(const kvq_snapkv_opts* opts, int32_t B, int32_t H, int32_t D,
                                        int32_t capacity, int32_t w) {
    if (B < 1 || H < 1 || capacity < 1 || w < 1 || (D != 32 && D != 64 && D != 128)) return 0;
    // observation rows: at most min(w, capacity) key rows, or G * w query rows
    const int rows = snap_rows(opts, H, capacity, w < capacity ? w : capacity);
    const int pool = snap_pool(opts);
    if (rows < 1 || pool < 1 || pool % 2 == 0) return 0;
    return chunk_ws_bytes(B, H, capacity, D, rows, pool > 1);
}

kvq_status kvq_snapkv_prefill_chunk(const kvq_snapkv_opts* opts, kvq_snapkv_state* in, kvq_snapkv_state* out,
                                    const void* k_chunk, const void* v_chunk, int32_t chunk_len, int32_t B,
                                    int32_t H, int32_t D, int32_t w, int32_t n_sink, int32_t budget,
                                    float* scores, void* ws, size_t ws_bytes, void* stream) {
    if (!in || !out || !k_chunk || !v_chunk || chunk_len < 1) return KVQ_ERR_INVALID_ARG;
    if (!in->k || !in->v || !in->pos || !out->k || !out->v || !out->pos) return KVQ_ERR_INVALID_ARG;
    if (in->capacity < 1 || out->capacity < 1 || in->n_kept < 0 || in->next_pos < in->n_kept)
        return KVQ_ERR_INVALID_ARG;
    const int64_t n64 = (int64_t)in->n_kept + chunk_len;
    if (n64 > in->capacity || (int64_t)in->next_pos + chunk_len > INT32_MAX) return KVQ_ERR_CAPACITY;
    const int S = (int)n64;
    int rows = 0, pool = 1;
    kvq_status st = snap_check(opts, B, H, S, D, w, n_sink, budget, &rows, &pool);
    if (st != KVQ_OK) return st;
    const int n_keep = budget < S ? budget : S;
    if (n_keep > out->capacity) return KVQ_ERR_CAPACITY;
    const void* ptrs[9] = {k_chunk, v_chunk, in->k, in->v, in->pos, out->k, out->v, out->pos, ws};
    for (const void* p : ptrs) if (!aligned16(p)) return KVQ_ERR_ALIGNMENT;
    if (scores && !aligned16(scores)) return KVQ_ERR_ALIGNMENT;
    // the two states must not share memory
    const size_t rb_in = (size_t)B * H * in->capacity * D * 2, rb_out = (size_t)B * H * out->capacity * D * 2;
    const size_t pb_in = (size_t)B * H * in->capacity * 4, pb_out = (size_t)B * H * out->capacity * 4;
    const void* ip[3] = {in->k, in->v, in->pos};
    const void* op[3] = {out->k, out->v, out->pos};
    const size_t inb[3] = {rb_in, rb_in, pb_in}, outb[3] = {rb_out, rb_out, pb_out};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            if (overlaps(ip[i], inb[i], op[j], outb[j])) return KVQ_ERR_INVALID_ARG;
    const size_t need = chunk_ws_bytes(B, H, in->capacity, D, rows, pool > 1);
    if (!ws || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_snapkv_chunk_copy(k_chunk, v_chunk, in->k, in->v, in->pos, B, H, D, chunk_len, in->capacity,
                                 in->n_kept, in->next_pos, s) != hipSuccess)
        return KVQ_ERR_HIP;
    char* wsb = static_cast<char*>(ws);
    int32_t* kept = reinterpret_cast<int32_t*>(wsb + snapkv_ws_bytes(B, H, in->capacity, D, rows, pool > 1));
    SnapRun r{opts, in->k, in->v, (int64_t)in->capacity * D, B, H, S, D, w, n_sink, budget, rows, pool,
              scores, kept, out->k, out->v, (int64_t)out->capacity * D, in->pos, in->capacity, out->pos,
              out->capacity, wsb};
    if ((st = snap_run(r, s)) != KVQ_OK) return st;
    in->n_kept = S;
    in->next_pos += chunk_len;
    out->n_kept = n_keep;
    out->next_pos = in->next_pos;
    return KVQ_OK;
}

kvq_status kvq_snapkv_select(const void* k, const void* v, int32_t B, int32_t H, int32_t S,
                             int32_t D, int32_t w, int32_t n_sink, int32_t budget, float* scores,
                             int32_t* kept, void* k_out, void* v_out, void* ws, size_t ws_bytes,
                             void* stream) {
    return kvq_snapkv_select_ex(nullptr, k, v, B, H, S, D, w, n_sink, budget, scores, kept, k_out, v_out, ws,
                                ws_bytes, stream);
}

kvq_status kvq_snapkv_pool_scores(const float* scores, float* pooled, int32_t B, int32_t H, int32_t S,
                                  int32_t pool_kernel, void* stream) {
    if (!scores || !pooled) return KVQ_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || S < 1 || pool_kernel < 1 || pool_kernel % 2 == 0) return KVQ_ERR_INVALID_ARG;
    if (pool_kernel > 31) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)B * H * S > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    const char* a0 = reinterpret_cast<const char*>(scores);
    const char* b0 = reinterpret_cast<const char*>(pooled);
    const size_t n = (size_t)B * H * S * sizeof(float);
    if (a0 < b0 + n && b0 < a0 + n) return KVQ_ERR_INVALID_ARG;
    return hip_status(launch_snapkv_pool(scores, pooled, (int64_t)B * H, S, pool_kernel,
                                         static_cast<hipStream_t>(stream)));
}

kvq_status kvq_snapkv_select_from_scores(const float* scores, int32_t B, int32_t H, int32_t S,
                                         int32_t n_sink, int32_t budget, int32_t* kept, void* stream) {
    if (!scores || !kept) return KVQ_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || S < 1 || budget < 1 || n_sink < 0) return KVQ_ERR_INVALID_ARG;
    if ((int64_t)B * H * S > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    if (!aligned16(scores) || !aligned16(kept)) return KVQ_ERR_ALIGNMENT;
    return hip_status(launch_snapkv_select(scores, B, H, S, n_sink, budget, kept,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"

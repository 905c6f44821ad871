// kvq_internal.h -- shared device helpers and kernel launch interfaces of
// libkvq (gfx950).  Not part of the public ABI (include/kvq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// ---------------------------------------------------------------- dtypes
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// fp32 -> fp16, round to nearest even, subnormals kept (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Load element i of an array of dtype DT as fp32 (exact widening).
template <int DT>
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i) {
    if constexpr (DT == KVQ_F32) {
        return static_cast<const float*>(p)[i];
    } else if constexpr (DT == KVQ_F16) {
        return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    } else {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
}

// Load 4 consecutive elements (index i is a multiple of 4).
template <int DT>
__device__ __forceinline__ void load4_as_f32(const void* p, int64_t i, float v[4]) {
    if constexpr (DT == KVQ_F32) {
        float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        if constexpr (DT == KVQ_F16) {
            v[0] = f16_bits_to_f32(x.x & 0xFFFFu); v[1] = f16_bits_to_f32(x.x >> 16);
            v[2] = f16_bits_to_f32(x.y & 0xFFFFu); v[3] = f16_bits_to_f32(x.y >> 16);
        } else {
            v[0] = bf16_bits_to_f32(x.x & 0xFFFFu); v[1] = bf16_bits_to_f32(x.x >> 16);
            v[2] = bf16_bits_to_f32(x.y & 0xFFFFu); v[3] = bf16_bits_to_f32(x.y >> 16);
        }
    }
}

__host__ __device__ constexpr int dtype_bytes(int dt) { return dt == KVQ_F32 ? 4 : 2; }

// Exchange through LDS between the lanes of one wave: the stores before the
// call are visible to the loads after it.  The fences order the LDS accesses
// for the compiler (the wave barrier alone does not touch memory); at
// wavefront scope they emit no wait, since one wave's LDS operations complete
// in order.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- cross-lane
// Exchanges and reductions within a wave without going through LDS: DPP row
// operations for lane distances up to 8 (inside 16-lane rows) and the gfx950
// lane swaps across rows (v_permlane16_swap: odd rows of the first operand
// with even rows of the second; v_permlane32_swap: upper half of the first
// with the lower half of the second).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
// The 32-bit value of lane l ^ M, M in {1, 2, 4, 8, 16, 32}.
template <int M>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x) {
    const int lane = threadIdx.x & 63;
    if constexpr (M == 1) {
        return dpp_u32<0xB1>(x);                 // quad_perm [1, 0, 3, 2]
    } else if constexpr (M == 2) {
        return dpp_u32<0x4E>(x);                 // quad_perm [2, 3, 0, 1]
    } else if constexpr (M == 4) {
        const uint32_t dn = dpp_u32<0x124>(x);   // row_ror:4  -> lane l - 4 (mod 16)
        const uint32_t up = dpp_u32<0x12C>(x);   // row_ror:12 -> lane l + 4 (mod 16)
        return (lane & 4) ? dn : up;
    } else if constexpr (M == 8) {
        return dpp_u32<0x128>(x);                // row_ror:8
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(M == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}
template <int M>
__device__ __forceinline__ float lane_xor(float v) { return __uint_as_float(lane_xor_u32<M>(__float_as_uint(v))); }

// op over each 16-lane row (Wide = false) or the whole wave (Wide = true),
// left in every lane.  Each step combines the same two partial values in
// every lane of a pair, so all lanes hold the identical result.
template <bool Wide, typename T, typename Op>
__device__ __forceinline__ T lane_reduce(T v, Op op) {
    auto u = [](T x) { return __builtin_bit_cast(uint32_t, x); };
    auto f = [](uint32_t x) { return __builtin_bit_cast(T, x); };
    v = op(v, f(dpp_u32<0xB1>(u(v))));
    v = op(v, f(dpp_u32<0x4E>(u(v))));
    v = op(v, f(dpp_u32<0x141>(u(v))));          // row_half_mirror
    v = op(v, f(dpp_u32<0x140>(u(v))));          // row_mirror
    if constexpr (Wide) {
        const auto r16 = __builtin_amdgcn_permlane16_swap(u(v), u(v), false, false);
        v = op(f(r16[0]), f(r16[1]));
        const auto r32 = __builtin_amdgcn_permlane32_swap(u(v), u(v), false, false);
        v = op(f(r32[0]), f(r32[1]));
    }
    return v;
}
__device__ __forceinline__ float row16_max(float v) { return lane_reduce<false>(v, [](float a, float b) { return fmaxf(a, b); }); }
__device__ __forceinline__ float row16_sum(float v) { return lane_reduce<false>(v, [](float a, float b) { return a + b; }); }
__device__ __forceinline__ float wave64_max(float v) { return lane_reduce<true>(v, [](float a, float b) { return fmaxf(a, b); }); }
__device__ __forceinline__ float wave64_sum(float v) { return lane_reduce<true>(v, [](float a, float b) { return a + b; }); }
// x + (x of lane l ^ 32), and the same for 16 with a pair of operands:
// swap32_sum(a, b): lanes 0..31 get a[l] + a[l + 32], lanes 32..63 b[l - 32] + b[l];
// swap16_sum(a, b): lanes of even rows get a[l] + a[l + 16], of odd rows b[l - 16] + b[l].
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Quantization constants of the specification (kvq.h): eps = 1e-5.
constexpr float kEps = 1e-5f;

// ---------------------------------------------------------------- launch args

// Per-token group quantization (TOK_AFFINE / TOK_SYM4) or plain copy of rows
// src [B][H][n][D] into slots [slot0, slot0 + n) of dst [B][H][cap][...].
struct RowQuantArgs {
    const void* src;
    void* codes;
    void* meta;
    const float* bias;     // TOK_SYM4 centering [H][D] or nullptr
    int B, H, n, D, cap, slot0;
    int kind, bits, group, in_dtype;
    int src_rows;          // rows between consecutive (b, h) slices of src (>= n)
};
// One fused launch: K rows (per-token kinds), V rows and positions.
struct RowAppendArgs {
    RowQuantArgs rows;      // shape: B, H, n, D, cap, slot0, in_dtype
    const void* k_src; void* k_codes; void* k_meta; const float* k_bias;
    int k_kind, k_bits, k_group;
    const void* v_src; void* v_codes; void* v_meta;
    int v_kind, v_bits, v_group;
    int32_t* pos; int first_pos;
    // positions of the new rows: pos_src (per-head rows of pos_src_rows when
    // pos_per_head, else [n]) or, when null, first_pos + i
    const int32_t* pos_src; int pos_src_rows; int pos_per_head;
};
hipError_t launch_row_append(const RowAppendArgs& a, hipStream_t s);

// KIVI per-channel: close `n_groups` groups made of the current residual
// (r0 keys) followed by new keys, then store the remaining new keys in the
// residual.
struct ChannelQuantArgs {
    const void* k_new;     // [B][H][src_rows][D], rows [0, n_new) appended
    void* resid;           // [B][H][Gt][D]
    void* codes;           // [B][H][cap][D*bits/8]
    void* table;           // [B][H][rows][D][2] fp16
    int32_t* k_row;        // [cap]
    int B, H, D, cap, rows, Gt, bits, in_dtype;
    int r0;                // residual fill before the append
    int n_new;
    int n_quant;           // coded slots before the append
    int n_groups;          // groups closed by this append
    int src_rows;
};
hipError_t launch_channel_quant(const ChannelQuantArgs& a, hipStream_t s);


// Decode attention.
struct DecodeArgs {
    const void* k_codes; const void* k_meta; const void* k_resid;
    const void* v_codes; const void* v_meta;
    const int32_t* k_row;
    const void* q; float* out;
    float* ws_o;           // [B][Hq][ns][D]
    float* ws_ml;          // [B][Hq][ns][2]
    int B, Hkv, Hq, D, cap, T, n_quant, Gt;
    int k_kind, k_bits, k_group, v_kind, v_bits, v_group;
    int in_dtype, q_dtype;
    float scale_log2;      // sm_scale * log2(e)
    int n_splits, split_len;
    // RoPE on read (null: none): table [positions][D/2] of (cos, sin); the key
    // of slot t is rotated at position t, the query at q_pos
    const float* rope; int q_pos;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_rope_table(float* table, int n_pos, int D, double base, hipStream_t s);
// log-sum-exp merge of per-split partials ws_o [rows][ns][D], ws_ml [rows][ns][2]
hipError_t launch_decode_combine(const float* ws_o, const float* ws_ml, float* out, int64_t rows, int D, int ns,
                                 hipStream_t s);
// The same merge over fp16 partials o / l (the multi-query attention's).
hipError_t launch_decode_combine_f16(const uint16_t* ws_o, const float* ws_ml, float* out, int64_t rows, int D,
                                     int ns, hipStream_t s);
// Multi-query attention over the cache (DecodeArgs with T, splits and q as
// [B][Hq][n_q][D]; out [B][Hq][n_q][D]).
bool prefill_factored(const DecodeArgs& a);
void prefill_plan(int B, int Hkv, int Hq, int n_q, int T, bool factored, int* n_rb, int* n_splits, int* split_len);
int prefill_max_splits(int B, int Hkv, int Hq, int n_q, int T);
hipError_t launch_prefill_attention(const DecodeArgs& a, int n_q, int n_rb, int causal, hipStream_t s);
// The fast decode: matrix-core kernels for 4-bit K (per-token affine,
// symmetric blocks or KIVI per-channel) and affine 4/8-bit V at head_dim
// 128 with 1-4 query heads per kv-head (decode_mfma.hip).
bool decode_fast_applies(const DecodeArgs& a);
void decode_fast_plan(int B, int Hkv, int T, int v_bits, int* n_splits, int* split_len);
hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s);
bool decode_mfma_applies(const DecodeArgs& a);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s);
size_t decode_workspace_bytes(int B, int Hq, int D, int cap);
void decode_plan(int B, int Hkv, int T, int* n_splits, int* split_len);

// StreamingLLM compaction.
struct EvictArgs {
    // row buffers: src/dst base, bytes per slot row
    const void* src[4]; void* dst[4]; int row_bytes[4]; int n_buf;
    const int32_t* src_pos; int32_t* dst_pos;
    const int32_t* src_row; int32_t* dst_row;      // KIVI_CH only (else nullptr)
    const void* src_table; void* dst_table; int table_row_bytes; int rows;
    const void* src_resid; void* dst_resid; size_t resid_bytes;
    int BH, cap, n, sink, window, n_quant_new;
    int pos_per_head;      // pos is [BH][cap] (else [cap], shared)
};
hipError_t launch_evict(const EvictArgs& a, hipStream_t s);

// SnapKV.
struct SnapArgs {
    const uint16_t* k; const uint16_t* v;
    // observation rows of (b, h): obs + (b * H + h) * obs_stride + r * D, r < n_rows
    const uint16_t* obs; int64_t obs_stride; int n_rows;
    float* scores; int32_t* kept; uint16_t* k_out; uint16_t* v_out;
    float* stats;          // [B][H][n_stat][n_rows][2]
    int B, H, S, D, w, n_sink, budget;
    int n_chunks;          // 128-key chunks (scores grid)
    int n_stat, stat_f, stat_reps;   // stats partials per row; set by the launcher
    int64_t kv_stride;     // elements between (b, h) slices of k and v
    int64_t out_stride;    // elements between (b, h) slices of k_out and v_out
    // optional: positions gathered with the rows (pos_in null: the row index)
    const int32_t* pos_in; int32_t* pos_out; int pos_in_rows, pos_out_rows;
    // one-read scores: per-(b, h, chunk) ready flags (null: the two-pass
    // scores), the call's tag, keys per chunk and the bounded wait
    uint64_t* flags; uint64_t tag; int one_chunk, n_one; int64_t wait_ticks;
};
size_t snapkv_ws_bytes(int B, int H, int S, int D, int n_rows, bool pooled);
hipError_t launch_snapkv_pool(const float* in, float* out, int64_t rows, int S, int kernel, hipStream_t s);
hipError_t launch_snapkv_scores(const SnapArgs& a, hipStream_t s);
// One-read scores (logits kept in registers across a per-head exchange of the
// row statistics): true and the launch made when the shape allows it (a.flags
// set), false to use launch_snapkv_scores.
bool snapkv_one_read_applies(const SnapArgs& a);
hipError_t launch_snapkv_scores_one_read(SnapArgs& a, hipStream_t s);
// Bytes of ready flags the one-read scores need in the workspace (0 when the
// shape does not allow it).
size_t snapkv_flag_bytes(int B, int H, int S, int n_rows);
// Process-wide bound on the one-read wait, in microseconds (tests set 0 to
// force the recomputing path).
extern int g_snap_wait_us;
// Copy chunk rows [B][H][n][D] fp16 into rows [row0, row0 + n) of a state
// [B][H][cap][D] and set their positions first_pos + i ([B][H][cap] int32).
hipError_t launch_snapkv_chunk_copy(const void* k_chunk, const void* v_chunk, void* k_state, void* v_state,
                                    int32_t* pos_state, int B, int H, int D, int n, int cap, int row0,
                                    int first_pos, hipStream_t s);
hipError_t launch_snapkv_select(const float* scores, int B, int H, int S, int n_sink, int budget,
                                int32_t* kept, hipStream_t s);
hipError_t launch_snapkv_gather(const SnapArgs& a, hipStream_t s);
// Top-k of `rank` and the gather of the kept rows (one launch where the keys fit
// in registers and at most 4096 rows are kept, else select then gather).
hipError_t launch_snapkv_select_gather(const SnapArgs& a, const float* rank, hipStream_t s);

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s);

}  // namespace kvq

// dequant8.h -- reading the packed cache eight channels at a time (gfx950).
//
// Shared by the LDS-tiled decode and the multi-query attention: keys and
// values of one slot, channels 8c .. 8c+7, dequantized to fp32 straight from
// the packed codes (value = u * scale + zero; symmetric keys (u - 8) * d;
// KIVI per-channel keys through the slot's table row, or from the
// full-precision residual while their group is open).
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace dq {

// 8 consecutive elements of a row of dtype `dt` as fp32 (exact widening).
__device__ __forceinline__ void load8(const void* base, int64_t elem, int dt, float x[8]) {
    if (dt == KVQ_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
        const float4 u = p[0], v = p[1];
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (dt == KVQ_F16) {
                x[2 * i] = f16_bits_to_f32(ww[i] & 0xFFFFu);
                x[2 * i + 1] = f16_bits_to_f32(ww[i] >> 16);
            } else {
                x[2 * i] = bf16_bits_to_f32(ww[i] & 0xFFFFu);
                x[2 * i + 1] = bf16_bits_to_f32(ww[i] >> 16);
            }
        }
    }
}

// The 8 codes of channels 8c .. 8c+7 of a code row (2, 4 or 8 bits per code).
__device__ __forceinline__ void codes8(const uint8_t* row, int c, int bits, float u[8]) {
    if (bits == 2) {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(row + 2 * c);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = (float)((w >> (2 * i)) & 0x3u);
    } else if (bits == 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(row + 4 * c);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = (float)((w >> (4 * i)) & 0xFu);
    } else {
        const uint2 w = *reinterpret_cast<const uint2*>(row + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u[i] = (float)((w.x >> (8 * i)) & 0xFFu);
            u[4 + i] = (float)((w.y >> (8 * i)) & 0xFFu);
        }
    }
}

// Dequantized keys of token t, channels 8c .. 8c+7 (k = u s + z, or as stored).
template <int KK>
__device__ __forceinline__ void k_values8(const DecodeArgs& a, int64_t bh, int t, int c, float x[8]) {
    const int D = a.D;
    const int64_t slot = bh * a.cap + t;
    if constexpr (KK == KVQ_PLAIN) {
        load8(a.k_codes, slot * D + 8 * c, a.in_dtype, x);
    } else if constexpr (KK == KVQ_KIVI_CH) {
        if (t >= a.n_quant) {                  // open group: full-precision residual
            load8(a.k_resid, (bh * a.Gt + (t - a.n_quant)) * D + 8 * c, a.in_dtype, x);
            return;
        }
        float u[8];
        codes8(static_cast<const uint8_t*>(a.k_codes) + slot * (D * a.k_bits / 8), c, a.k_bits, u);
        const int rows = a.cap / a.Gt + 3;
        const uint4* m = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(a.k_meta) +
                                                        ((bh * rows + a.k_row[t]) * D + 8 * c));
        const uint4 m0 = m[0], m1 = m[1];
        const uint32_t mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(u[i], f16_bits_to_f32(mm[i] & 0xFFFFu), f16_bits_to_f32(mm[i] >> 16));
    } else if constexpr (KK == KVQ_TOK_SYM4) {
        float u[8];
        codes8(static_cast<const uint8_t*>(a.k_codes) + slot * (D / 2), c, 4, u);
        const float d = f16_bits_to_f32(static_cast<const uint16_t*>(a.k_meta)[slot * (D / 32) + (8 * c) / 32]);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (u[i] - 8.0f) * d;
    } else {  // TOK_AFFINE
        float u[8];
        codes8(static_cast<const uint8_t*>(a.k_codes) + slot * (D * a.k_bits / 8), c, a.k_bits, u);
        const uint32_t m = static_cast<const uint32_t*>(a.k_meta)[slot * (D / a.k_group) + (8 * c) / a.k_group];
        const float sc = f16_bits_to_f32(m & 0xFFFFu), z = f16_bits_to_f32(m >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(u[i], sc, z);
    }
}

template <int VK>
__device__ __forceinline__ void v_values8(const DecodeArgs& a, int64_t bh, int t, int c, float x[8]) {
    const int D = a.D;
    const int64_t slot = bh * a.cap + t;
    if constexpr (VK == KVQ_PLAIN) {
        load8(a.v_codes, slot * D + 8 * c, a.in_dtype, x);
    } else {
        float u[8];
        codes8(static_cast<const uint8_t*>(a.v_codes) + slot * (D * a.v_bits / 8), c, a.v_bits, u);
        const uint32_t m = static_cast<const uint32_t*>(a.v_meta)[slot * (D / a.v_group) + (8 * c) / a.v_group];
        const float sc = f16_bits_to_f32(m & 0xFFFFu), z = f16_bits_to_f32(m >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(u[i], sc, z);
    }
}

// Two-stage form for loops that fetch a tile ahead of its use: the fetch
// issues the global loads of the codes and the metadata word (for KIVI keys
// the table row index), the finish unpacks and scales.  Kinds without codes
// (PLAIN, KIVI keys still in the residual) load in the finish stage.
struct Pre8 { uint32_t c0, c1, meta; int32_t row; };

__device__ __forceinline__ void fetch_codes8(const uint8_t* row, int c, int bits, Pre8& p) {
    if (bits == 2) {
        p.c0 = *reinterpret_cast<const uint16_t*>(row + 2 * c);
    } else if (bits == 4) {
        p.c0 = *reinterpret_cast<const uint32_t*>(row + 4 * c);
    } else {
        const uint2 w = *reinterpret_cast<const uint2*>(row + 8 * c);
        p.c0 = w.x; p.c1 = w.y;
    }
}

__device__ __forceinline__ void unpack_codes8(const Pre8& p, int bits, float u[8]) {
    if (bits == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = (float)((p.c0 >> (2 * i)) & 0x3u);
    } else if (bits == 4) {
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = (float)((p.c0 >> (4 * i)) & 0xFu);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u[i] = (float)((p.c0 >> (8 * i)) & 0xFFu);
            u[4 + i] = (float)((p.c1 >> (8 * i)) & 0xFFu);
        }
    }
}

template <int KK>
__device__ __forceinline__ void k_fetch8(const DecodeArgs& a, int64_t bh, int t, int c, Pre8& p) {
    const int D = a.D;
    const int64_t slot = bh * a.cap + t;
    if constexpr (KK == KVQ_KIVI_CH) {
        if (t < a.n_quant) {
            fetch_codes8(static_cast<const uint8_t*>(a.k_codes) + slot * (D * a.k_bits / 8), c, a.k_bits, p);
            p.row = a.k_row[t];
        }
    } else if constexpr (KK == KVQ_TOK_SYM4) {
        fetch_codes8(static_cast<const uint8_t*>(a.k_codes) + slot * (D / 2), c, 4, p);
        p.meta = static_cast<const uint16_t*>(a.k_meta)[slot * (D / 32) + (8 * c) / 32];
    } else if constexpr (KK == KVQ_TOK_AFFINE) {
        fetch_codes8(static_cast<const uint8_t*>(a.k_codes) + slot * (D * a.k_bits / 8), c, a.k_bits, p);
        p.meta = static_cast<const uint32_t*>(a.k_meta)[slot * (D / a.k_group) + (8 * c) / a.k_group];
    }
}

template <int KK>
__device__ __forceinline__ void k_finish8(const DecodeArgs& a, int64_t bh, int t, int c, const Pre8& p, float x[8]) {
    const int D = a.D;
    const int64_t slot = bh * a.cap + t;
    if constexpr (KK == KVQ_PLAIN) {
        load8(a.k_codes, slot * D + 8 * c, a.in_dtype, x);
    } else if constexpr (KK == KVQ_KIVI_CH) {
        if (t >= a.n_quant) {
            load8(a.k_resid, (bh * a.Gt + (t - a.n_quant)) * D + 8 * c, a.in_dtype, x);
            return;
        }
        float u[8];
        unpack_codes8(p, a.k_bits, u);
        const int rows = a.cap / a.Gt + 3;
        const uint4* m = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(a.k_meta) +
                                                        ((bh * rows + p.row) * D + 8 * c));
        const uint4 m0 = m[0], m1 = m[1];
        const uint32_t mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(u[i], f16_bits_to_f32(mm[i] & 0xFFFFu), f16_bits_to_f32(mm[i] >> 16));
    } else if constexpr (KK == KVQ_TOK_SYM4) {
        float u[8];
        unpack_codes8(p, 4, u);
        const float d = f16_bits_to_f32(p.meta & 0xFFFFu);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (u[i] - 8.0f) * d;
    } else {
        float u[8];
        unpack_codes8(p, a.k_bits, u);
        const float sc = f16_bits_to_f32(p.meta & 0xFFFFu), z = f16_bits_to_f32(p.meta >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(u[i], sc, z);
    }
}

template <int VK>
__device__ __forceinline__ void v_fetch8(const DecodeArgs& a, int64_t bh, int t, int c, Pre8& p) {
    if constexpr (VK == KVQ_TOK_AFFINE) {
        const int D = a.D;
        const int64_t slot = bh * a.cap + t;
        fetch_codes8(static_cast<const uint8_t*>(a.v_codes) + slot * (D * a.v_bits / 8), c, a.v_bits, p);
        p.meta = static_cast<const uint32_t*>(a.v_meta)[slot * (D / a.v_group) + (8 * c) / a.v_group];
    }
}

template <int VK>
__device__ __forceinline__ void v_finish8(const DecodeArgs& a, int64_t bh, int t, int c, const Pre8& p, float x[8]) {
    if constexpr (VK == KVQ_PLAIN) {
        load8(a.v_codes, (bh * a.cap + t) * a.D + 8 * c, a.in_dtype, x);
    } else {
        float u[8];
        unpack_codes8(p, a.v_bits, u);
        const float sc = f16_bits_to_f32(p.meta & 0xFFFFu), z = f16_bits_to_f32(p.meta >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(u[i], sc, z);
    }
}

}  // namespace dq
}  // namespace kvq

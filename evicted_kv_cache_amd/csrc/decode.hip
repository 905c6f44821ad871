// decode.hip -- fused decode attention over the compressed cache (gfx950).
//
// Split-T flash decoding: block (split, kv-head, batch) streams its slice of
// slots tile by tile, dequantizing keys and values in registers straight from
// the packed codes ("Low-bit KV caches on MLX", s.1: the packed layout is read
// directly, no full-precision copy; s.5: two-pass split over the token axis
// for long caches), keeps a running max / sum per query head (online softmax
// in base 2) and writes unnormalized partials; a combine kernel merges the
// splits by log-sum-exp.  Keys centered before quantization are used as
// stored: a constant per-row logit shift leaves the softmax unchanged
// ("kv-cache: optional per-channel K-cache mean-centering", "Why this is safe").
//
// This file holds the generic kernel that serves every layout.  The
// bandwidth-tuned kernels for per-token 4-bit layouts live in decode_fast.hip.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTile = 256;
constexpr int kMaxGroup = 8;   // query heads per kv-head

__device__ __forceinline__ uint32_t code_at(const uint8_t* row, int d, int bits) {
    if (bits == 4) return (row[d >> 1] >> ((d & 1) * 4)) & 0xFu;
    return row[d];
}

template <int KK, int DT>
__device__ __forceinline__ float k_value(const DecodeArgs& a, int64_t bh, int t, int d) {
    const int D = a.D;
    if constexpr (KK == KVQ_PLAIN) {
        return load_as_f32<DT>(a.k_codes, (bh * a.cap + t) * D + d);
    } else if constexpr (KK == KVQ_TOK_AFFINE) {
        const int64_t slot = bh * a.cap + t;
        const uint8_t* row = static_cast<const uint8_t*>(a.k_codes) + slot * (D * a.k_bits / 8);
        const uint32_t m = static_cast<const uint32_t*>(a.k_meta)[slot * (D / a.k_group) + d / a.k_group];
        return (float)code_at(row, d, a.k_bits) * f16_bits_to_f32(m & 0xFFFFu) + f16_bits_to_f32(m >> 16);
    } else if constexpr (KK == KVQ_TOK_SYM4) {
        const int64_t slot = bh * a.cap + t;
        const uint8_t* row = static_cast<const uint8_t*>(a.k_codes) + slot * (D / 2);
        const uint16_t sc = static_cast<const uint16_t*>(a.k_meta)[slot * (D / 32) + d / 32];
        return ((float)code_at(row, d, 4) - 8.0f) * f16_bits_to_f32(sc);
    } else {  // KIVI_CH
        if (t >= a.n_quant)
            return load_as_f32<DT>(a.k_resid, (bh * a.Gt + (t - a.n_quant)) * D + d);
        const int64_t slot = bh * a.cap + t;
        const uint8_t* row = static_cast<const uint8_t*>(a.k_codes) + slot * (D * a.k_bits / 8);
        const int rows = a.cap / a.Gt + 3;
        const int r = a.k_row[t];
        const uint32_t m = static_cast<const uint32_t*>(a.k_meta)[(bh * rows + r) * D + d];
        return (float)code_at(row, d, a.k_bits) * f16_bits_to_f32(m & 0xFFFFu) + f16_bits_to_f32(m >> 16);
    }
}

template <int VK, int DT>
__device__ __forceinline__ float v_value(const DecodeArgs& a, int64_t bh, int t, int d) {
    const int D = a.D;
    const int64_t slot = bh * a.cap + t;
    if constexpr (VK == KVQ_PLAIN) {
        return load_as_f32<DT>(a.v_codes, slot * D + d);
    } else {
        const uint8_t* row = static_cast<const uint8_t*>(a.v_codes) + slot * (D * a.v_bits / 8);
        const uint32_t m = static_cast<const uint32_t*>(a.v_meta)[slot * (D / a.v_group) + d / a.v_group];
        return (float)code_at(row, d, a.v_bits) * f16_bits_to_f32(m & 0xFFFFu) + f16_bits_to_f32(m >> 16);
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

template <int KK, int VK, int DT, int QDT>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a) {
    const int split = blockIdx.x;
    const int hk = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int D = a.D;
    const int gq = a.Hq / a.Hkv;
    const int64_t bh = (int64_t)b * a.Hkv + hk;

    __shared__ float q_s[kMaxGroup][128];
    __shared__ float p_s[kMaxGroup][kTile];
    __shared__ float m_s[kMaxGroup], l_s[kMaxGroup], alpha_s[kMaxGroup];

    for (int idx = tid; idx < gq * D; idx += 256) {
        const int h = idx / D, d = idx % D;
        q_s[h][d] = load_as_f32<QDT>(a.q, ((int64_t)b * a.Hq + hk * gq + h) * D + d) * a.scale_log2;
    }
    if (tid < kMaxGroup) { m_s[tid] = -INFINITY; l_s[tid] = 0.0f; }
    __syncthreads();

    const int t_begin = split * a.split_len;
    const int t_end = min(a.T, t_begin + a.split_len);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};   // outputs o_idx = tid + 256 k  (gq * D <= 1024)

    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        const int t = t0 + tid;
        float lg[kMaxGroup];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) lg[h] = 0.0f;
        if (t < t_end) {
            for (int d = 0; d < D; ++d) {
                const float kv = k_value<KK, DT>(a, bh, t, d);
#pragma unroll
                for (int h = 0; h < kMaxGroup; ++h)
                    if (h < gq) lg[h] = fmaf(q_s[h][d], kv, lg[h]);
            }
        } else {
#pragma unroll
            for (int h = 0; h < kMaxGroup; ++h) lg[h] = -INFINITY;
        }
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
            if (h < gq) p_s[h][tid] = lg[h];
        __syncthreads();
        const int wave = tid >> 6, lane = tid & 63;
        for (int h = wave; h < gq; h += 4) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, p_s[h][lane + 64 * i]);
            mx = wave_max(mx);
            const float m_old = m_s[h];
            const float m_new = fmaxf(m_old, mx);
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = exp2f(p_s[h][lane + 64 * i] - m_new);
                p_s[h][lane + 64 * i] = e;
                sum += e;
            }
            sum = wave_sum(sum);
            if (lane == 0) {
                const float alpha = exp2f(m_old - m_new);
                l_s[h] = l_s[h] * alpha + sum;
                m_s[h] = m_new;
                alpha_s[h] = alpha;
            }
        }
        __syncthreads();
        const int nt = min(kTile, t_end - t0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int o_idx = tid + 256 * k;
            if (o_idx < gq * D) {
                const int h = o_idx / D, d = o_idx % D;
                float s = acc[k] * alpha_s[h];
                for (int tt = 0; tt < nt; ++tt)
                    s = fmaf(p_s[h][tt], v_value<VK, DT>(a, bh, t0 + tt, d), s);
                acc[k] = s;
            }
        }
        __syncthreads();
    }
    const int ns = a.n_splits;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int o_idx = tid + 256 * k;
        if (o_idx < gq * D) {
            const int h = o_idx / D, d = o_idx % D;
            a.ws_o[(((int64_t)b * a.Hq + hk * gq + h) * ns + split) * D + d] = acc[k];
        }
    }
    if (tid < gq) {
        float* ml = a.ws_ml + (((int64_t)b * a.Hq + hk * gq + tid) * ns + split) * 2;
        ml[0] = m_s[tid];
        ml[1] = l_s[tid];
    }
}

// out[row][d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* ws_o, const float* ws_ml,
                                                             float* out, int D, int ns) {
    const int64_t row = blockIdx.x;
    const int d = threadIdx.x;
    if (d >= D) return;
    const float* ml = ws_ml + row * ns * 2;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < ns; ++s) {
        const float w = exp2f(ml[2 * s] - M);
        den = fmaf(w, ml[2 * s + 1], den);
        num = fmaf(w, ws_o[(row * ns + s) * D + d], num);
    }
    out[row * D + d] = num / den;
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

template <int KK, int VK, int DT>
hipError_t launch_generic_q(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.n_splits, (unsigned)a.Hkv, (unsigned)a.B);
    switch (a.q_dtype) {
        case KVQ_F32: hipLaunchKernelGGL((decode_generic_kernel<KK, VK, DT, KVQ_F32>), grid, dim3(256), 0, s, a); break;
        case KVQ_F16: hipLaunchKernelGGL((decode_generic_kernel<KK, VK, DT, KVQ_F16>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((decode_generic_kernel<KK, VK, DT, KVQ_BF16>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int KK, int VK>
hipError_t launch_generic_dt(const DecodeArgs& a, hipStream_t s) {
    switch (a.in_dtype) {
        case KVQ_F32: return launch_generic_q<KK, VK, KVQ_F32>(a, s);
        case KVQ_F16: return launch_generic_q<KK, VK, KVQ_F16>(a, s);
        default: return launch_generic_q<KK, VK, KVQ_BF16>(a, s);
    }
}

template <int KK>
hipError_t launch_generic_v(const DecodeArgs& a, hipStream_t s) {
    if (a.v_kind == KVQ_PLAIN) return launch_generic_dt<KK, KVQ_PLAIN>(a, s);
    return launch_generic_dt<KK, KVQ_TOK_AFFINE>(a, s);
}

}  // namespace

// Split plan: enough (split, kv-head, batch) blocks to cover the chip twice,
// splits at least one tile long.
void decode_plan(int B, int Hkv, int T, int* n_splits, int* split_len) {
    const int units = B * Hkv;
    int want = (512 + units - 1) / units;
    const int max_tiles = (T + kTile - 1) / kTile;
    int ns = want < max_tiles ? want : max_tiles;
    if (ns < 1) ns = 1;
    int len = (T + ns - 1) / ns;
    len = ((len + kTile - 1) / kTile) * kTile;
    if (len < kTile) len = kTile;
    *split_len = len;
    *n_splits = (T + len - 1) / len;
    if (*n_splits < 1) *n_splits = 1;
}

size_t decode_workspace_bytes(int B, int Hq, int D, int cap) {
    // decode_plan never uses more splits than min(ceil(512 / (B * Hkv)), tiles(T)),
    // which is at most min(ceil(512 / B), tiles(capacity)) for any Hkv >= 1, T <= capacity
    const int want = (512 + B - 1) / B;
    const int tiles = (cap + kTile - 1) / kTile;
    int ns = want < tiles ? want : tiles;
    if (ns < 1) ns = 1;
    return (size_t)B * Hq * ns * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    hipError_t e;
    if (decode_fast_applies(a)) {
        e = launch_decode_fast(a, s);
        if (e != hipSuccess || a.n_splits == 1) return e;
        hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(128), 0, s,
                           a.ws_o, a.ws_ml, a.out, a.D, a.n_splits);
        return hipGetLastError();
    }
    switch (a.k_kind) {
        case KVQ_PLAIN: e = launch_generic_v<KVQ_PLAIN>(a, s); break;
        case KVQ_KIVI_CH: e = launch_generic_v<KVQ_KIVI_CH>(a, s); break;
        case KVQ_TOK_AFFINE: e = launch_generic_v<KVQ_TOK_AFFINE>(a, s); break;
        default: e = launch_generic_v<KVQ_TOK_SYM4>(a, s); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(128), 0, s,
                       a.ws_o, a.ws_ml, a.out, a.D, a.n_splits);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace kvq

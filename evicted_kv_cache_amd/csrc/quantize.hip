// quantize.hip -- quantize-on-write kernels of libkvq (gfx950).
//
// Per-token groups along head_dim (TOK_AFFINE, for V and for mlx-style K) and
// symmetric 4-bit blocks with optional mean-centering (TOK_SYM4) run one row
// per group of head_dim/4 lanes, 4 consecutive channels per lane; group
// min/max (or max|x|) is a butterfly over the lanes of one group.
// KIVI per-channel keys close whole token groups: one lane per channel pair
// walks the group's tokens.
//
// The arithmetic follows the bit-exact specification in include/kvq.h
// ("StreamingLLM + KIVI", section "Affine quantisation formula", with eps
// 1e-5 and fp16 scale/zero; "kv-cache: optional per-channel K-cache
// mean-centering for Q4_0", section "The idea", for the symmetric blocks):
// every subtract / divide is one correctly rounded fp32 operation (the file
// is compiled with -ffp-contract=off), rint rounds half to even, fp32->fp16
// conversion rounds to nearest even and keeps subnormals.
#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

template <int DT>
__device__ __forceinline__ void copy4_raw(const void* src, int64_t si, void* dst, int64_t di) {
    if constexpr (DT == KVQ_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(dst) + di) =
            *reinterpret_cast<const float4*>(static_cast<const float*>(src) + si);
    } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + di) =
            *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + si);
    }
}

// Affine code against stored (fp16-rounded) scale and zero.
__device__ __forceinline__ uint32_t affine_code(float x, float s, float z, float top) {
    float diff = x - z;
    float ratio = diff / s;
    float y = rintf(ratio);
    y = fmaxf(y, 0.0f);      // also maps NaN to 0
    y = fminf(y, top);
    return (uint32_t)y;
}

template <int DT, int KIND, int BITS>
__global__ __launch_bounds__(256) void row_quant_kernel(RowQuantArgs a) {
    const int tpr = a.D >> 2;                    // lanes per row (8, 16 or 32)
    const int rows_per_block = 256 / tpr;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / tpr;
    const int lane = threadIdx.x % tpr;
    const int64_t total = (int64_t)a.B * a.H * a.n;
    if (row >= total) return;                    // whole rows (hence whole groups) exit together
    const int64_t bh = row / a.n;
    const int i = (int)(row - bh * a.n);
    const int d0 = lane * 4;
    const int64_t drow = bh * a.cap + a.slot0 + i;

    if constexpr (KIND == KVQ_PLAIN) {
        if (DT == KVQ_F32 && a.bias) {
            // test seam: centered keys kept at full precision (fp32 subtract)
            const float* x = static_cast<const float*>(a.src) + row * a.D + d0;
            const float* bb = a.bias + (int64_t)(bh % a.H) * a.D + d0;
            float4 y;
            y.x = x[0] - bb[0]; y.y = x[1] - bb[1]; y.z = x[2] - bb[2]; y.w = x[3] - bb[3];
            *reinterpret_cast<float4*>(static_cast<float*>(a.codes) + drow * a.D + d0) = y;
        } else {
            copy4_raw<DT>(a.src, row * a.D + d0, a.codes, drow * a.D + d0);
        }
        return;
    } else {
        float x[4];
        load4_as_f32<DT>(a.src, row * a.D + d0, x);
        uint32_t u[4];
        if constexpr (KIND == KVQ_TOK_SYM4) {
            if (a.bias) {
                const int h = (int)(bh % a.H);
                const float* bb = a.bias + (int64_t)h * a.D + d0;
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] = x[k] - bb[k];
            }
            float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
            for (int off = 1; off < 8; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
            float dd = amax / 7.0f;
            dd = fmaxf(dd, kEps);
            const uint16_t d16 = f32_to_f16_bits(dd);
            const float df = f16_bits_to_f32(d16);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float y = rintf(x[k] / df);
                y = fmaxf(y, -8.0f);
                y = fminf(y, 7.0f);
                u[k] = (uint32_t)(int)(y + 8.0f);
            }
            if ((lane & 7) == 0)
                static_cast<uint16_t*>(a.meta)[drow * (a.D >> 5) + (d0 >> 5)] = d16;
        } else {  // KVQ_TOK_AFFINE
            const int lpg = a.group >> 2;        // lanes per group (8, 16 or 32)
            float mn = fminf(fminf(x[0], x[1]), fminf(x[2], x[3]));
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            for (int off = 1; off < lpg; off <<= 1) {
                mn = fminf(mn, __shfl_xor(mn, off));
                mx = fmaxf(mx, __shfl_xor(mx, off));
            }
            constexpr float top = (float)((1 << BITS) - 1);
            float range = mx - mn;
            float s = range / top;
            s = fmaxf(s, kEps);
            const uint16_t s16 = f32_to_f16_bits(s);
            const uint16_t z16 = f32_to_f16_bits(mn);
            const float sf = f16_bits_to_f32(s16);
            const float zf = f16_bits_to_f32(z16);
#pragma unroll
            for (int k = 0; k < 4; ++k) u[k] = affine_code(x[k], sf, zf, top);
            if ((lane & (lpg - 1)) == 0) {
                const int ng = a.D / a.group;
                static_cast<uint32_t*>(a.meta)[drow * ng + d0 / a.group] =
                    (uint32_t)s16 | ((uint32_t)z16 << 16);
            }
        }
        if constexpr (BITS == 4) {
            const uint16_t packed = (uint16_t)(u[0] | (u[1] << 4) | (u[2] << 8) | (u[3] << 12));
            static_cast<uint16_t*>(a.codes)[drow * (a.D >> 2) + lane] = packed;
        } else {
            const uint32_t packed = u[0] | (u[1] << 8) | (u[2] << 16) | (u[3] << 24);
            static_cast<uint32_t*>(a.codes)[drow * (a.D >> 2) + lane] = packed;
        }
    }
}

// KIVI per-channel: block (group j, bh), lane = channel pair.  Token tau of
// the combined sequence [residual (r0 keys), new keys] lives in the residual
// for tau < r0 and in k_new otherwise.
template <int DT, int BITS>
__global__ __launch_bounds__(64) void channel_close_kernel(ChannelQuantArgs a) {
    const int j = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int dp = threadIdx.x;
    const int D = a.D;
    const int Gt = a.Gt;
    if (dp >= (D >> 1)) return;
    const int c0 = dp * 2;
    const int row = (a.n_quant > 0 ? a.k_row[a.n_quant - 1] + 1 : 0) + j;
    if (row < 0 || row >= a.rows) return;   // cannot happen while at most two position runs are kept
    auto val = [&](int tau, int c) -> float {
        if (tau < a.r0) return load_as_f32<DT>(a.resid, (bh * Gt + tau) * D + c);
        return load_as_f32<DT>(a.k_new, (bh * a.n_new + (tau - a.r0)) * D + c);
    };
    const int tau0 = j * Gt;
    float mn0 = val(tau0, c0), mx0 = mn0, mn1 = val(tau0, c0 + 1), mx1 = mn1;
    for (int t = 1; t < Gt; ++t) {
        const float x0 = val(tau0 + t, c0), x1 = val(tau0 + t, c0 + 1);
        mn0 = fminf(mn0, x0); mx0 = fmaxf(mx0, x0);
        mn1 = fminf(mn1, x1); mx1 = fmaxf(mx1, x1);
    }
    constexpr float top = (float)((1 << BITS) - 1);
    float r0 = mx0 - mn0, r1 = mx1 - mn1;
    float s0 = r0 / top, s1 = r1 / top;
    s0 = fmaxf(s0, kEps); s1 = fmaxf(s1, kEps);
    const uint16_t s0h = f32_to_f16_bits(s0), z0h = f32_to_f16_bits(mn0);
    const uint16_t s1h = f32_to_f16_bits(s1), z1h = f32_to_f16_bits(mn1);
    const float s0f = f16_bits_to_f32(s0h), z0f = f16_bits_to_f32(z0h);
    const float s1f = f16_bits_to_f32(s1h), z1f = f16_bits_to_f32(z1h);
    uint2 meta;
    meta.x = (uint32_t)s0h | ((uint32_t)z0h << 16);
    meta.y = (uint32_t)s1h | ((uint32_t)z1h << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.table) + ((bh * a.rows + row) * D + c0) * 2) = meta;
    const int slot0 = a.n_quant + tau0;
    for (int t = 0; t < Gt; ++t) {
        const uint32_t u0 = affine_code(val(tau0 + t, c0), s0f, z0f, top);
        const uint32_t u1 = affine_code(val(tau0 + t, c0 + 1), s1f, z1f, top);
        const int64_t slot = bh * a.cap + slot0 + t;
        if constexpr (BITS == 4) {
            static_cast<uint8_t*>(a.codes)[slot * (D >> 1) + dp] = (uint8_t)(u0 | (u1 << 4));
        } else {
            static_cast<uint16_t*>(a.codes)[slot * (D >> 1) + dp] = (uint16_t)(u0 | (u1 << 8));
        }
    }
    if (bh == 0) {
        for (int t = dp; t < Gt; t += (D >> 1)) a.k_row[slot0 + t] = row;
    }
}

// New keys that stay open go to the residual: new key i (i >= i0) is stored
// at residual row r0 + i - n_groups * Gt.
template <int ES>
__global__ __launch_bounds__(256) void resid_store_kernel(ChannelQuantArgs a, int i0) {
    const int n_keep = a.n_new - i0;
    const int64_t per_bh = (int64_t)n_keep * a.D;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per_bh * a.B * a.H) return;
    const int64_t bh = idx / per_bh;
    const int64_t rem = idx - bh * per_bh;
    const int i = i0 + (int)(rem / a.D);
    const int d = (int)(rem % a.D);
    const int rr = a.r0 + i - a.n_groups * a.Gt;
    using T = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
    static_cast<T*>(a.resid)[(bh * a.Gt + rr) * a.D + d] =
        static_cast<const T*>(a.k_new)[(bh * a.n_new + i) * a.D + d];
}

__global__ __launch_bounds__(256) void fill_pos_kernel(int32_t* pos, int slot0, int first, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) pos[slot0 + i] = first + i;
}

template <int DT, int KIND, int BITS>
hipError_t launch_row(const RowQuantArgs& a, hipStream_t s) {
    const int tpr = a.D / 4;
    const int rpb = 256 / tpr;
    const int64_t rows = (int64_t)a.B * a.H * a.n;
    const int64_t blocks = (rows + rpb - 1) / rpb;
    hipLaunchKernelGGL((row_quant_kernel<DT, KIND, BITS>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_row_dt(const RowQuantArgs& a, hipStream_t s) {
    if (a.kind == KVQ_PLAIN) return launch_row<DT, KVQ_PLAIN, 8>(a, s);
    if (a.kind == KVQ_TOK_SYM4) return launch_row<DT, KVQ_TOK_SYM4, 4>(a, s);
    if (a.bits == 4) return launch_row<DT, KVQ_TOK_AFFINE, 4>(a, s);
    return launch_row<DT, KVQ_TOK_AFFINE, 8>(a, s);
}

template <int DT>
hipError_t launch_channel_dt(const ChannelQuantArgs& a, hipStream_t s) {
    if (a.n_groups > 0) {
        dim3 grid((unsigned)a.n_groups, (unsigned)(a.B * a.H));
        if (a.bits == 4)
            hipLaunchKernelGGL((channel_close_kernel<DT, 4>), grid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL((channel_close_kernel<DT, 8>), grid, dim3(64), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int i0 = a.n_groups > 0 ? a.n_groups * a.Gt - a.r0 : 0;
    const int64_t n = (int64_t)(a.n_new - i0) * a.D * a.B * a.H;
    if (n > 0) {
        const unsigned blocks = (unsigned)((n + 255) / 256);
        if (dtype_bytes(DT) == 4)
            hipLaunchKernelGGL((resid_store_kernel<4>), dim3(blocks), dim3(256), 0, s, a, i0);
        else
            hipLaunchKernelGGL((resid_store_kernel<2>), dim3(blocks), dim3(256), 0, s, a, i0);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_row_quant(const RowQuantArgs& a, hipStream_t s) {
    switch (a.in_dtype) {
        case KVQ_F32: return launch_row_dt<KVQ_F32>(a, s);
        case KVQ_F16: return launch_row_dt<KVQ_F16>(a, s);
        default: return launch_row_dt<KVQ_BF16>(a, s);
    }
}

hipError_t launch_channel_quant(const ChannelQuantArgs& a, hipStream_t s) {
    switch (a.in_dtype) {
        case KVQ_F32: return launch_channel_dt<KVQ_F32>(a, s);
        case KVQ_F16: return launch_channel_dt<KVQ_F16>(a, s);
        default: return launch_channel_dt<KVQ_BF16>(a, s);
    }
}

hipError_t launch_fill_pos(int32_t* pos, int slot0, int first_pos, int n, hipStream_t s) {
    hipLaunchKernelGGL(fill_pos_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       pos, slot0, first_pos, n);
    return hipGetLastError();
}

}  // namespace kvq

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

// rint(num / den) with the IEEE-rounded quotient, via a reciprocal.  With
// r = fl(1/den), y = fl(num * r) is within |num/den| * 2^-23 of the exact
// quotient, i.e. within 2^-15 for |num/den| <= 256 (beyond that the code is
// clamped anyway), and the IEEE quotient is within 2^-24 |num/den| of it.  So
// rint(y) is the rint of the IEEE quotient unless y lies within 2^-14 of a
// half-integer; only then is the division done exactly.
__device__ __forceinline__ float rint_div(float num, float den, float r) {
    const float y = num * r;
    const float fr = __builtin_amdgcn_fractf(y);   // y - floor(y)
    if (fabsf(fr - 0.5f) < 6.103515625e-05f) return rintf(num / den);
    return rintf(y);
}

// Affine code against stored (fp16-rounded) scale and zero:
// clamp(rint((x - z) / s), 0, top), with one fp32 subtract and the IEEE quotient.
__device__ __forceinline__ uint32_t affine_code(float x, float s, float z, float r, float top) {
    float diff = x - z;
    float y = rint_div(diff, s, r);
    y = fmaxf(y, 0.0f);      // also maps NaN to 0
    y = fminf(y, top);
    return (uint32_t)y;
}

// Row formats of the fused row kernel.
enum RowFmt { kFmtNone = 0, kFmtPlain = 1, kFmtAff4 = 2, kFmtAff8 = 3, kFmtSym4 = 4 };

template <int DT>
__device__ __forceinline__ void load8_as_f32(const void* p, int64_t i, float v[8]) {
    if constexpr (DT == KVQ_F32) {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (DT == KVQ_F16) {
                v[2 * k] = f16_bits_to_f32(w[k] & 0xFFFFu);
                v[2 * k + 1] = f16_bits_to_f32(w[k] >> 16);
            } else {
                v[2 * k] = bf16_bits_to_f32(w[k] & 0xFFFFu);
                v[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
            }
        }
    }
}

// One row part of the fused kernel: lanes of a row hold 8 consecutive channels each.
struct RowPart {
    const void* src; void* codes; void* meta; const float* bias; int group;
};

template <int DT, int FMT>
__device__ __forceinline__ void quant_vals8(const RowPart& r, float x[8], int64_t drow, int64_t bh,
                                            int lane, int D, int H);

// Plain rows are copied (or, for the centering test seam, centered in fp32);
// the other formats quantize 8 preloaded values per lane.
template <int DT, int FMT>
__device__ __forceinline__ void quant_row8(const RowPart& r, int64_t row, int64_t drow, int64_t bh,
                                           int lane, int D, int H) {
    const int d0 = lane * 8;
    if constexpr (FMT == kFmtPlain) {
        if (DT == KVQ_F32 && r.bias) {
            // test seam: centered keys kept at full precision (fp32 subtract)
            const float* x = static_cast<const float*>(r.src) + row * D + d0;
            const float* bb = r.bias + (int64_t)(bh % H) * D + d0;
            float* y = static_cast<float*>(r.codes) + drow * D + d0;
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = x[k] - bb[k];
        } else if constexpr (DT == KVQ_F32) {
            const float4* x = reinterpret_cast<const float4*>(static_cast<const float*>(r.src) + row * D + d0);
            float4* y = reinterpret_cast<float4*>(static_cast<float*>(r.codes) + drow * D + d0);
            y[0] = x[0]; y[1] = x[1];
        } else {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(r.codes) + drow * D + d0) =
                *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(r.src) + row * D + d0);
        }
        return;
    } else {
        float x[8];
        load8_as_f32<DT>(r.src, row * D + d0, x);
        quant_vals8<DT, FMT>(r, x, drow, bh, lane, D, H);
    }
}

template <int DT, int FMT>
__device__ __forceinline__ void quant_vals8(const RowPart& r, float x[8], int64_t drow, int64_t bh,
                                            int lane, int D, int H) {
    const int d0 = lane * 8;
    {
        uint32_t u[8];
        if constexpr (FMT == kFmtSym4) {
            if (r.bias) {
                const float* bb = r.bias + (int64_t)(bh % H) * D + d0;
#pragma unroll
                for (int k = 0; k < 8; ++k) x[k] = x[k] - bb[k];
            }
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
            amax = fmaxf(amax, __shfl_xor(amax, 1));     // 4 lanes per block of 32
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            float dd = amax / 7.0f;
            dd = fmaxf(dd, kEps);
            const uint16_t d16 = f32_to_f16_bits(dd);
            const float df = f16_bits_to_f32(d16);
            const float rdf = 1.0f / df;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float y = rint_div(x[k], df, rdf);
                y = fmaxf(y, -8.0f);
                y = fminf(y, 7.0f);
                u[k] = (uint32_t)(int)(y + 8.0f);
            }
            if ((lane & 3) == 0) static_cast<uint16_t*>(r.meta)[drow * (D >> 5) + (d0 >> 5)] = d16;
        } else {
            constexpr int BITS = FMT == kFmtAff4 ? 4 : 8;
            const int lpg = r.group >> 3;                 // lanes per group (4, 8 or 16)
            float mn = x[0], mx = x[0];
#pragma unroll
            for (int k = 1; k < 8; ++k) { mn = fminf(mn, x[k]); mx = fmaxf(mx, x[k]); }
            for (int off = 1; off < lpg; off <<= 1) {
                mn = fminf(mn, __shfl_xor(mn, off));
                mx = fmaxf(mx, __shfl_xor(mx, off));
            }
            constexpr float top = (float)((1 << BITS) - 1);
            float range = mx - mn;
            float sc = range / top;
            sc = fmaxf(sc, kEps);
            const uint16_t s16 = f32_to_f16_bits(sc);
            const uint16_t z16 = f32_to_f16_bits(mn);
            const float sf = f16_bits_to_f32(s16);
            const float zf = f16_bits_to_f32(z16);
            const float rs = 1.0f / sf;
#pragma unroll
            for (int k = 0; k < 8; ++k) u[k] = affine_code(x[k], sf, zf, rs, top);
            if ((lane & (lpg - 1)) == 0)
                static_cast<uint32_t*>(r.meta)[drow * (D / r.group) + d0 / r.group] =
                    (uint32_t)s16 | ((uint32_t)z16 << 16);
        }
        if constexpr (FMT == kFmtAff8) {
            uint2 pk;
            pk.x = u[0] | (u[1] << 8) | (u[2] << 16) | (u[3] << 24);
            pk.y = u[4] | (u[5] << 8) | (u[6] << 16) | (u[7] << 24);
            reinterpret_cast<uint2*>(r.codes)[drow * (D >> 3) + lane] = pk;
        } else {
            uint32_t pk = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) pk |= u[k] << (4 * k);
            static_cast<uint32_t*>(r.codes)[drow * (D >> 3) + lane] = pk;
        }
    }
}

// Fused append of K rows (unless KIVI per-channel, FK == kFmtNone), V rows
// and positions.  Blocks [0, nbk) quantize K rows, the rest V rows; block 0
// also writes the positions of the new slots.
template <int DT, int FK, int FV>
__global__ __launch_bounds__(256) void row_append_kernel(RowQuantArgs a, RowPart kp, RowPart vp,
                                                         int nbk, int nb_total, int32_t* pos, int first_pos) {
    const int tpr = a.D >> 3;                         // lanes per row (4, 8 or 16)
    const int rows_per_block = 256 / tpr;
    if (blockIdx.x == 0 && pos) {
        for (int i = threadIdx.x; i < a.n; i += 256) pos[a.slot0 + i] = first_pos + i;
    }
    const int64_t total = (int64_t)a.B * a.H * a.n;
    const int lane = threadIdx.x % tpr;
    // grid-stride over row blocks: [0, nbk) are K row blocks, the rest V.
    // Two row blocks per iteration, both loads issued before either is
    // quantized, so each lane keeps two 16-byte loads in flight.
    auto row_of = [&](int blk_all, bool& is_k, int64_t& row) {
        is_k = blk_all < nbk;
        const int blk = is_k ? blk_all : blk_all - nbk;
        row = (int64_t)blk * rows_per_block + threadIdx.x / tpr;
        return blk_all < nb_total && row < total;
    };
    for (int b0 = blockIdx.x; b0 < nb_total; b0 += 2 * gridDim.x) {
        bool ka, kb;
        int64_t ra, rb;
        const bool va = row_of(b0, ka, ra);
        const bool vb = row_of(b0 + gridDim.x, kb, rb);
        constexpr bool plain_k = FK == kFmtPlain || FK == kFmtNone, plain_v = FV == kFmtPlain;
        float xa[8], xb[8];
        if (va && !(ka ? plain_k : plain_v)) load8_as_f32<DT>(ka ? kp.src : vp.src, ra * a.D + lane * 8, xa);
        if (vb && !(kb ? plain_k : plain_v)) load8_as_f32<DT>(kb ? kp.src : vp.src, rb * a.D + lane * 8, xb);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bool v = t == 0 ? va : vb;
            if (!v) continue;                             // whole rows (hence groups) skip together
            const bool is_k = t == 0 ? ka : kb;
            const int64_t row = t == 0 ? ra : rb;
            float* x = t == 0 ? xa : xb;
            const int64_t bh = row / a.n;
            const int i = (int)(row - bh * a.n);
            const int64_t drow = bh * a.cap + a.slot0 + i;
            if (is_k) {
                if constexpr (FK == kFmtPlain) quant_row8<DT, FK>(kp, row, drow, bh, lane, a.D, a.H);
                else if constexpr (FK != kFmtNone) quant_vals8<DT, FK>(kp, x, drow, bh, lane, a.D, a.H);
            } else {
                if constexpr (FV == kFmtPlain) quant_row8<DT, FV>(vp, row, drow, bh, lane, a.D, a.H);
                else quant_vals8<DT, FV>(vp, x, drow, bh, lane, a.D, a.H);
            }
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
    const float r0f = 1.0f / s0f, r1f = 1.0f / s1f;
    uint2 meta;
    meta.x = (uint32_t)s0h | ((uint32_t)z0h << 16);
    meta.y = (uint32_t)s1h | ((uint32_t)z1h << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.table) + ((bh * a.rows + row) * D + c0) * 2) = meta;
    const int slot0 = a.n_quant + tau0;
    for (int t = 0; t < Gt; ++t) {
        const uint32_t u0 = affine_code(val(tau0 + t, c0), s0f, z0f, r0f, top);
        const uint32_t u1 = affine_code(val(tau0 + t, c0 + 1), s1f, z1f, r1f, top);
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

int row_fmt(int kind, int bits) {
    if (kind == KVQ_PLAIN) return kFmtPlain;
    if (kind == KVQ_TOK_SYM4) return kFmtSym4;
    if (kind == KVQ_TOK_AFFINE) return bits == 4 ? kFmtAff4 : kFmtAff8;
    return kFmtNone;   // KIVI per-channel keys take the channel path
}

template <int DT, int FK, int FV>
hipError_t launch_append_fv(const RowAppendArgs& a, hipStream_t s) {
    const int tpr = a.rows.D / 8;
    const int rpb = 256 / tpr;
    const int64_t rows = (int64_t)a.rows.B * a.rows.H * a.rows.n;
    const int nb = (int)((rows + rpb - 1) / rpb);
    const int nbk = FK == kFmtNone ? 0 : nb;
    const int nb_total = nbk + nb;
    const int grid = nb_total < 4096 ? nb_total : 4096;   // 16 blocks per CU, grid-stride beyond
    hipLaunchKernelGGL((row_append_kernel<DT, FK, FV>), dim3((unsigned)grid), dim3(256), 0, s,
                       a.rows, RowPart{a.k_src, a.k_codes, a.k_meta, a.k_bias, a.k_group},
                       RowPart{a.v_src, a.v_codes, a.v_meta, nullptr, a.v_group}, nbk, nb_total, a.pos,
                       a.first_pos);
    return hipGetLastError();
}

template <int DT, int FK>
hipError_t launch_append_fk(const RowAppendArgs& a, int fv, hipStream_t s) {
    switch (fv) {
        case kFmtPlain: return launch_append_fv<DT, FK, kFmtPlain>(a, s);
        case kFmtAff4: return launch_append_fv<DT, FK, kFmtAff4>(a, s);
        default: return launch_append_fv<DT, FK, kFmtAff8>(a, s);
    }
}

template <int DT>
hipError_t launch_append_dt(const RowAppendArgs& a, hipStream_t s) {
    const int fk = row_fmt(a.k_kind, a.k_bits), fv = row_fmt(a.v_kind, a.v_bits);
    switch (fk) {
        case kFmtNone: return launch_append_fk<DT, kFmtNone>(a, fv, s);
        case kFmtPlain: return launch_append_fk<DT, kFmtPlain>(a, fv, s);
        case kFmtAff4: return launch_append_fk<DT, kFmtAff4>(a, fv, s);
        case kFmtAff8: return launch_append_fk<DT, kFmtAff8>(a, fv, s);
        default: return launch_append_fk<DT, kFmtSym4>(a, fv, s);
    }
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

hipError_t launch_row_append(const RowAppendArgs& a, hipStream_t s) {
    switch (a.rows.in_dtype) {
        case KVQ_F32: return launch_append_dt<KVQ_F32>(a, s);
        case KVQ_F16: return launch_append_dt<KVQ_F16>(a, s);
        default: return launch_append_dt<KVQ_BF16>(a, s);
    }
}

hipError_t launch_channel_quant(const ChannelQuantArgs& a, hipStream_t s) {
    switch (a.in_dtype) {
        case KVQ_F32: return launch_channel_dt<KVQ_F32>(a, s);
        case KVQ_F16: return launch_channel_dt<KVQ_F16>(a, s);
        default: return launch_channel_dt<KVQ_BF16>(a, s);
    }
}

}  // namespace kvq

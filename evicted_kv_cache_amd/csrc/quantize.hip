// quantize.hip -- quantize-on-write kernels of libkvq (gfx950).
//
// Per-token groups along head_dim (TOK_AFFINE, for V and for mlx-style K) and
// symmetric 4-bit blocks with optional mean-centering (TOK_SYM4) run one row
// per head_dim/16 lanes, 16 consecutive channels per lane; group min/max (or
// max|x|) is a butterfly over the lanes of one group.
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
enum RowFmt { kFmtNone = 0, kFmtPlain = 1, kFmtAff4 = 2, kFmtAff8 = 3, kFmtSym4 = 4, kFmtAff2 = 5 };

constexpr int kEpl = 16;        // elements (channels) per lane in the row kernel
constexpr int kRowIter = 2;     // row passes per block

// The 16 consecutive input elements of one lane in one row, as loaded
// (widened only when used, so that every row's loads are in flight first).
template <int DT>
struct Raw16 { uint4 w[DT == KVQ_F32 ? 4 : 2]; };

template <int DT>
__device__ __forceinline__ void load_raw16(const char* p, Raw16<DT>& r) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int k = 0; k < (DT == KVQ_F32 ? 4 : 2); ++k) r.w[k] = q[k];
}

// Exact widening to fp32.
template <int DT>
__device__ __forceinline__ void widen16(const Raw16<DT>& r, float v[kEpl]) {
#pragma unroll
    for (int h = 0; h < (DT == KVQ_F32 ? 4 : 2); ++h) {
        const uint32_t w[4] = {r.w[h].x, r.w[h].y, r.w[h].z, r.w[h].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (DT == KVQ_F32) {
                v[4 * h + k] = __uint_as_float(w[k]);
            } else if constexpr (DT == KVQ_F16) {
                v[8 * h + 2 * k] = f16_bits_to_f32(w[k] & 0xFFFFu);
                v[8 * h + 2 * k + 1] = f16_bits_to_f32(w[k] >> 16);
            } else {
                v[8 * h + 2 * k] = bf16_bits_to_f32(w[k] & 0xFFFFu);
                v[8 * h + 2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
            }
        }
    }
}

// One row part of the fused kernel (K or V).
struct RowPart {
    const void* src; void* codes; void* meta; const float* bias; int group;
};

// DPP lane exchanges inside a row of 16 lanes: partner l^1, l^2 (quad
// permutes) and the mirror within 8 lanes (l -> 7 - l), which after the two
// quad steps pairs the two quads of an 8-lane group.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141;

// max / min over the `lanes` lanes (2, 4 or 8, aligned) holding one group;
// `lanes` is uniform, so the steps are scalar branches
__device__ __forceinline__ float group_max(float v, int lanes) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    if (lanes > 2) v = fmaxf(v, dpp<kDppXor2>(v));
    if (lanes > 4) v = fmaxf(v, dpp<kDppHalfMirror>(v));
    return v;
}
__device__ __forceinline__ float group_min(float v, int lanes) {
    v = fminf(v, dpp<kDppXor1>(v));
    if (lanes > 2) v = fminf(v, dpp<kDppXor2>(v));
    if (lanes > 4) v = fminf(v, dpp<kDppHalfMirror>(v));
    return v;
}

// Quantize the 16 values x of this lane (channels 16 lane .. 16 lane + 15 of
// row drow) and store codes and metadata.  rint of each quotient comes from
// y = num * r with r = v_rcp_f32(den) (within 1 ulp of 1/den): y is within
// 1.5 * 2^-23 |q| of the exact quotient q and the IEEE quotient within
// 2^-24 |q|, so for |q| < 255 they differ by less than 2^-14 and rint(y)
// equals rint of the IEEE quotient unless y lies within 2^-14 of a
// half-integer, i.e. |y - rint(y)| > 0.5 - 2^-14 (quotients of 255 and more
// clamp to the top code either way).  Waves with such an element (about 1
// in 8000 elements) recompute those with the IEEE divide.
template <int DT, int FMT>
__device__ __forceinline__ void quant16(const RowPart& r, float x[kEpl], int64_t drow, int h, int lane,
                                        int D) {
    constexpr float kBand = 0.49993896484375f;    // 0.5 - 2^-14
    float y[kEpl];
    bool near = false;
    uint32_t pk[kEpl / 2];                        // 4-bit: pk[0..1]; 8-bit: pk[0..3]
    if constexpr (FMT == kFmtSym4) {
        if (r.bias) {
            const float* bb = r.bias + (int64_t)h * D + lane * kEpl;
#pragma unroll
            for (int k = 0; k < kEpl; ++k) x[k] = x[k] - bb[k];
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < kEpl; ++k) amax = fmaxf(amax, fabsf(x[k]));
        amax = fmaxf(amax, dpp<kDppXor1>(amax));     // 2 lanes per block of 32
        float dd = amax / 7.0f;
        dd = fmaxf(dd, kEps);
        const uint16_t d16 = f32_to_f16_bits(dd);
        const float df = f16_bits_to_f32(d16);
        const float rdf = __builtin_amdgcn_rcpf(df);
        float dev = 0.0f;                             // max |q - rint(q)|
#pragma unroll
        for (int k = 0; k < kEpl; ++k) {
            const float q = x[k] * rdf;
            y[k] = rintf(q);
            dev = fmaxf(dev, fabsf(q - y[k]));
        }
        near = dev > kBand;
        if (__builtin_amdgcn_ballot_w64(near) != 0) {
#pragma unroll
            for (int k = 0; k < kEpl; ++k) {
                const float q = x[k] * rdf;
                if (fabsf(q - rintf(q)) > kBand) y[k] = rintf(x[k] / df);
            }
        }
#pragma unroll
        for (int k = 0; k < kEpl; ++k) y[k] = fminf(fmaxf(y[k], -8.0f), 7.0f) + 8.0f;
        if ((lane & 1) == 0) static_cast<uint16_t*>(r.meta)[drow * (D >> 5) + (lane >> 1)] = d16;
    } else {
        constexpr int BITS = FMT == kFmtAff4 ? 4 : FMT == kFmtAff2 ? 2 : 8;
        constexpr float top = (float)((1 << BITS) - 1);
        const int gsh = __builtin_ctz(r.group);       // group sizes are powers of two
        const int lpg = r.group / kEpl;               // lanes per group (2, 4 or 8)
        const int lsh = gsh - 4;                      // log2(lanes per group)
        float mn = x[0], mx = x[0];
#pragma unroll
        for (int k = 1; k < kEpl; ++k) { mn = fminf(mn, x[k]); mx = fmaxf(mx, x[k]); }
        mn = group_min(mn, lpg);
        mx = group_max(mx, lpg);
        const float range = mx - mn;
        float sc = range / top;
        sc = fmaxf(sc, kEps);
        const uint16_t s16 = f32_to_f16_bits(sc);
        const uint16_t z16 = f32_to_f16_bits(mn);
        const float sf = f16_bits_to_f32(s16);
        const float zf = f16_bits_to_f32(z16);
        const float rs = __builtin_amdgcn_rcpf(sf);
        float dev = 0.0f;                             // max |q - rint(q)|
        // 4-bit codes: q = fma(x, rs, -zf rs) saves the subtract.  The exact
        // product inside the fma leaves the reciprocal's error (2^-23 |q|,
        // |q| <= 16) and the rounding of -zf rs (2^-24 |zf / sf|), together
        // below 2^-14.5 while |zf| <= 512 sf, so the near-tie band still
        // covers the difference to the IEEE quotient.  A lane whose zero
        // point lies further out sends all its elements to the exact path.
        const float c = -zf * rs;
        const bool far = BITS == 4 && !(fabsf(zf) <= 512.0f * sf);
#pragma unroll
        for (int k = 0; k < kEpl; ++k) {
            const float q = BITS == 4 ? fmaf(x[k], rs, c) : (x[k] - zf) * rs;
            y[k] = rintf(q);
            dev = fmaxf(dev, fabsf(q - y[k]));
        }
        if (far) dev = 1.0f;
        near = dev > kBand;
        if (__builtin_amdgcn_ballot_w64(near) != 0) {
#pragma unroll
            for (int k = 0; k < kEpl; ++k) {
                const float diff = x[k] - zf;
                const float q = BITS == 4 ? fmaf(x[k], rs, c) : diff * rs;
                if (far || fabsf(q - rintf(q)) > kBand) y[k] = rintf(diff / sf);
            }
        }
#pragma unroll
        for (int k = 0; k < kEpl; ++k) y[k] = __builtin_amdgcn_fmed3f(y[k], 0.0f, top);
        if ((lane & (lpg - 1)) == 0)
            static_cast<uint32_t*>(r.meta)[(drow << (__builtin_ctz(D) - gsh)) + (lane >> lsh)] =
                (uint32_t)s16 | ((uint32_t)z16 << 16);
    }
    // y holds integral codes in [0, top]; v_cvt_pk_u8_f32 converts one to a
    // byte lane of a packed word
    if constexpr (FMT == kFmtAff2) {
        // 2-bit codes: element i of the lane at bits 2i of one word
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < kEpl; ++k) w |= (uint32_t)y[k] << (2 * k);
        reinterpret_cast<uint32_t*>(r.codes)[drow * (D >> 4) + lane] = w;
    } else if constexpr (FMT == kFmtAff8) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) w = __builtin_amdgcn_cvt_pk_u8_f32(y[4 * k + i], i, w);
            pk[k] = w;
        }
        reinterpret_cast<uint4*>(r.codes)[drow * (D >> 4) + lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
        // even elements to the byte lanes of e, odd ones to o: e | o << 4 is
        // the nibble-packed word (element 2i low nibble of byte i)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t e = 0, o = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e = __builtin_amdgcn_cvt_pk_u8_f32(y[8 * k + 2 * i], i, e);
                o = __builtin_amdgcn_cvt_pk_u8_f32(y[8 * k + 2 * i + 1], i, o);
            }
            pk[k] = e | (o << 4);
        }
        reinterpret_cast<uint2*>(r.codes)[drow * (D >> 4) + lane] = make_uint2(pk[0], pk[1]);
    }
}

// Plain rows are copied (or, for the centering test seam, centered in fp32).
template <int DT>
__device__ __forceinline__ void copy_row16(const RowPart& r, int64_t row, int64_t drow, int h, int lane, int D) {
    const int d0 = lane * kEpl;
    if constexpr (DT == KVQ_F32) {
        const float4* x = reinterpret_cast<const float4*>(static_cast<const float*>(r.src) + row * D + d0);
        float4* y = reinterpret_cast<float4*>(static_cast<float*>(r.codes) + drow * D + d0);
        if (r.bias) {
            // test seam: centered keys kept at full precision (fp32 subtract)
            const float4* bb = reinterpret_cast<const float4*>(r.bias + (int64_t)h * D + d0);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 a = x[k], c = bb[k];
                y[k] = make_float4(a.x - c.x, a.y - c.y, a.z - c.z, a.w - c.w);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = x[k];
        }
    } else {
        const uint4* x = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(r.src) + row * D + d0);
        uint4* y = reinterpret_cast<uint4*>(static_cast<uint16_t*>(r.codes) + drow * D + d0);
        y[0] = x[0];
        y[1] = x[1];
    }
}

// Fused append of K rows (unless KIVI per-channel, FK == kFmtNone), V rows
// and positions.  Block (x = chunk, y = slice bh - bh0, z) covers rows
// [chunk * rows_per_chunk, +rows_per_chunk) of sequence slice bh, of K
// (z = 0) or V (z = 1, or z = 0 when K takes the channel path); a row is
// D / 16 = 2^lpr_sh lanes of 16 channels, and each thread takes kRowIter
// rows, all loaded before any is widened or quantized.  Blocks of bh = 0
// also write the positions of their rows.
// Positions of the appended slots.
struct PosWrite {
    int32_t* pos; const int32_t* src; int src_rows; int first; int per_head;
};

template <int DT, int FK, int FV>
__global__ __launch_bounds__(256) void row_append_kernel(RowQuantArgs a, RowPart kp, RowPart vp, int bh0,
                                                         int lpr_sh, PosWrite pw) {
    constexpr int ES = DT == KVQ_F32 ? 4 : 2;          // input bytes per element
    const int rpp_sh = 8 - lpr_sh;                    // log2 rows per pass
    const int rpc = kRowIter << rpp_sh;               // rows per chunk
    const int chunk = blockIdx.x;
    const int bh = bh0 + blockIdx.y;
    const bool is_v = FK == kFmtNone || blockIdx.z == 1;
    const int lane = threadIdx.x & ((1 << lpr_sh) - 1);
    const int i_base = chunk * rpc + (threadIdx.x >> lpr_sh);
    if (pw.pos && (pw.per_head || bh == 0) && !(FK != kFmtNone && is_v)) {
        const int i_end = min(a.n, (chunk + 1) * rpc);
        int32_t* P = pw.pos + (pw.per_head ? (int64_t)bh * a.cap : 0) + a.slot0;
        const int32_t* Ps = pw.src ? pw.src + (pw.per_head ? (int64_t)bh * pw.src_rows : 0) : nullptr;
        for (int i = chunk * rpc + threadIdx.x; i < i_end; i += 256) P[i] = Ps ? Ps[i] : pw.first + i;
    }
    const int64_t drow0 = (int64_t)bh * a.cap + a.slot0;
    auto run = [&](const RowPart& part, auto fmt_tag) {
        constexpr int FMT = decltype(fmt_tag)::value;
        if constexpr (FMT == kFmtPlain) {
            const int h = bh % a.H;
#pragma unroll
            for (int it = 0; it < kRowIter; ++it) {
                const int i = i_base + (it << rpp_sh);
                if (i < a.n) copy_row16<DT>(part, (int64_t)bh * a.src_rows + i, drow0 + i, h, lane, a.D);
            }
        } else {
            const char* src = static_cast<const char*>(part.src) + ((int64_t)bh * a.src_rows * a.D + lane * kEpl) * ES;
            const uint32_t row_bytes = (uint32_t)a.D * ES;
            Raw16<DT> raw[kRowIter];
#pragma unroll
            for (int it = 0; it < kRowIter; ++it) {
                // rows past the end load the last row (always valid) and are not stored
                const int i = min(i_base + (it << rpp_sh), a.n - 1);
                load_raw16<DT>(src + (uint64_t)(uint32_t)i * row_bytes, raw[it]);
            }
            const int h = FMT == kFmtSym4 && part.bias ? bh % a.H : 0;
#pragma unroll
            for (int it = 0; it < kRowIter; ++it) {
                const int i = i_base + (it << rpp_sh);
                if (i < a.n) {       // whole rows (hence groups) skip together
                    float x[kEpl];
                    widen16<DT>(raw[it], x);
                    quant16<DT, FMT>(part, x, drow0 + i, h, lane, a.D);
                }
            }
        }
    };
    if (is_v) {
        run(vp, std::integral_constant<int, FV>{});
    } else if constexpr (FK != kFmtNone) {
        run(kp, std::integral_constant<int, FK>{});
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
        return load_as_f32<DT>(a.k_new, (bh * a.src_rows + (tau - a.r0)) * D + c);
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
        if constexpr (BITS == 2) {
            // four 2-bit codes per byte: the even lane of a channel-pair pair writes it
            const uint32_t n = u0 | (u1 << 2);
            const uint32_t m = (uint32_t)__shfl_xor((int)n, 1);
            if ((dp & 1) == 0) static_cast<uint8_t*>(a.codes)[slot * (D >> 2) + (dp >> 1)] = (uint8_t)(n | (m << 4));
        } else if constexpr (BITS == 4) {
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
        static_cast<const T*>(a.k_new)[(bh * a.src_rows + i) * a.D + d];
}

int row_fmt(int kind, int bits) {
    if (kind == KVQ_PLAIN) return kFmtPlain;
    if (kind == KVQ_TOK_SYM4) return kFmtSym4;
    if (kind == KVQ_TOK_AFFINE) return bits == 4 ? kFmtAff4 : bits == 2 ? kFmtAff2 : kFmtAff8;
    return kFmtNone;   // KIVI per-channel keys take the channel path
}

template <int DT, int FK, int FV>
hipError_t launch_append_fv(const RowAppendArgs& a, hipStream_t s) {
    const int lpr_sh = __builtin_ctz(a.rows.D / kEpl);     // D in {32, 64, 128}
    const int rpc = (256 >> lpr_sh) * kRowIter;
    const int n_chunks = (a.rows.n + rpc - 1) / rpc;
    const int bh_total = a.rows.B * a.rows.H;
    // slices go on grid y (at most 65535 per launch)
    for (int bh0 = 0; bh0 < bh_total; bh0 += 65535) {
        const int nbh = bh_total - bh0 < 65535 ? bh_total - bh0 : 65535;
        dim3 grid((unsigned)n_chunks, (unsigned)nbh, FK == kFmtNone ? 1 : 2);
        hipLaunchKernelGGL((row_append_kernel<DT, FK, FV>), grid, dim3(256), 0, s, a.rows,
                           RowPart{a.k_src, a.k_codes, a.k_meta, a.k_bias, a.k_group},
                           RowPart{a.v_src, a.v_codes, a.v_meta, nullptr, a.v_group}, bh0, lpr_sh,
                           PosWrite{a.pos, a.pos_src, a.pos_src_rows, a.first_pos, a.pos_per_head});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DT, int FK>
hipError_t launch_append_fk(const RowAppendArgs& a, int fv, hipStream_t s) {
    switch (fv) {
        case kFmtPlain: return launch_append_fv<DT, FK, kFmtPlain>(a, s);
        case kFmtAff4: return launch_append_fv<DT, FK, kFmtAff4>(a, s);
        case kFmtAff2: return launch_append_fv<DT, FK, kFmtAff2>(a, s);
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
        case kFmtAff2: return launch_append_fk<DT, kFmtAff2>(a, fv, s);
        default: return launch_append_fk<DT, kFmtSym4>(a, fv, s);
    }
}

template <int DT>
hipError_t launch_channel_dt(const ChannelQuantArgs& a, hipStream_t s) {
    if (a.n_groups > 0) {
        dim3 grid((unsigned)a.n_groups, (unsigned)(a.B * a.H));
        if (a.bits == 2)
            hipLaunchKernelGGL((channel_close_kernel<DT, 2>), grid, dim3(64), 0, s, a);
        else if (a.bits == 4)
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

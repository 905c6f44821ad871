// decode_fast.hip -- decode attention for KIVI keys ("StreamingLLM + KIVI",
// "KIVI": per-channel 4-bit keys over 32-token groups, the open group kept in
// full precision) and per-token affine 4- or 8-bit values ("Low-bit KV caches
// on MLX", s.1) at head_dim 128 and 1-4 query heads per kv-head, on the VALU
// (gfx950).  Per-token 4-bit keys run on the matrix cores instead
// (decode_mfma.hip); both kernels use the split plan and the dispatch below.
//
// Decode streams the whole cache once per step ("Low-bit KV caches on MLX",
// s.5: decode spends its time reading the cache):
//
// * Workgroup = 4 waves on one (batch, kv-head[, token split]); each wave
//   owns a contiguous run of 32-token tiles with its own online softmax; the
//   waves merge through LDS (token splits merge in a combine kernel).
// * QK^T: lane (token t, quarter of head_dim) reads 16 bytes of codes per
//   token.  A channel's scale and zero live in the table row of the token's
//   group, so they cannot be factored out of the dot product: each wave
//   stages the table rows of a tile's first and last tokens in LDS (a tile
//   spans at most those two in an unevicted cache), every lane dequantizes
//   its token's 32 channels in fp32 (k = u s + z) and multiplies them by the
//   query with mixed-precision FMAs.  The query is held as fp16 pairs scaled
//   by a power of two shared by the head group (exact for bf16/fp16 queries).
//   Tokens whose row is neither staged row, and tokens of the open group,
//   take a per-lane path that reads their row or residual from memory.  The
//   four quarter partials of a head meet in lane quarter h by DPP rotations.
// * Softmax: lane (t, h) computes p for head h of tokens t and t+16 (one
//   exp each) and writes the fp16 weight pair (p_t s_t, p_t+16 s_t+16) 2^E to
//   LDS; the running max is rescaled only when a wave sees a larger logit,
//   so p <= 1.  The power of two 2^E follows the largest V scale the wave
//   has seen (the accumulators are rescaled when it changes), so weights
//   neither overflow nor fall into fp16's subnormal range when V is small;
//   it is taken out exactly at the end.
// * PV: lane (phase, 8-channel chunk) reads the codes of tokens t and t+16.
//   A 4-bit code left in place under a mask is an fp16 subnormal, which
//   v_dot2_f32_f16 multiplies exactly: one v_perm_b32 per byte position
//   gives the pair of whole bytes (b_t, b_t+16), b = u_2k + 16 u_2k+1, and
//   one AND its low nibbles; v_dot2_f32_f16 with the weight pair does two
//   token MACs on each, and the high-nibble channel is (byte sum - low sum)
//   / 16 at the end (8-bit codes: the whole bytes are the codes).  The zero
//   points and the fp16 rounding of the weights are accounted exactly in
//   fp32 (c = 8 for 4-bit codes, 128 for 8-bit):
//     o = sum_t w^_t u_t + sum_t p_t (z_t + c s_t) - c sum_t w^_t
//   so rounding a weight only perturbs w (u - c).
// * Tails need no clamping: loads go through buffer resources whose size is
//   the valid part of the tile, and out-of-range loads return zero.  Only the
//   last tile of a split can hold invalid tokens; it alone masks its logits.
//   Codes and per-token metadata, read once per step, load with the
//   non-temporal cache policy; table rows and positions use the default.
#include <math.h>

#include "bufload.h"
#include "dequant8.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kD = 128;
constexpr int kGQ = 4;          // query heads per kv-head
constexpr int kTileT = 32;      // tokens per wave tile
constexpr int kWaves = 4;
constexpr int kRowB = kD / 2;   // bytes of 4-bit K codes per token

using buf::rsrc;
using buf::u32x2;
using buf::u32x4;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}
// Round-to-nearest-even pack of two fp32 into an fp16 pair.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    half2_t h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}
// acc + (low / high fp16 half of h) * x in one v_fma_mix_f32.  Written out so
// that the compiler keeps the packed pair as the operand instead of hoisting
// loop-invariant widenings into separate registers.  The compiler does not
// add wait states around inline asm: never feed these a fresh transcendental
// result (v_exp_f32 and the like); the build checks the assembly for it.
__device__ __forceinline__ float fma_lo(uint32_t h, float x, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x), "v"(acc));
    return r;
}
__device__ __forceinline__ float fma_hi(uint32_t h, float x, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x), "v"(acc));
    return r;
}
// fp16 halves of a packed pair, widened (folds into v_fma_mix_f32 operands)
__device__ __forceinline__ float f16lo(uint32_t u) { return (float)__builtin_bit_cast(half2_t, u).x; }
__device__ __forceinline__ float f16hi(uint32_t u) { return (float)__builtin_bit_cast(half2_t, u).y; }
// (low fp16 half of h) * y: one v_fma_mix_f32 with a +0 addend (a -0
// product comes out as +0, which no caller distinguishes).  Plain code, not
// inline asm: its operands are often fresh v_exp_f32 results, and only code
// the compiler emits itself gets the wait states such a read needs.
__device__ __forceinline__ float mul_lo(uint32_t h, float y) { return __builtin_fmaf(f16lo(h), y, 0.0f); }
// DPP quad rotations: value of lane (l - k) mod 4 within the lane's quad.
template <int K>
__device__ __forceinline__ float quad_from_minus(float v) {
    constexpr int ctrl = K == 1 ? 0x93 : K == 2 ? 0x4E : 0x39;   // quad_perm [3,0,1,2] / [2,3,0,1] / [1,2,3,0]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
}

template <bool B>
struct Flag { static constexpr bool value = B; };

// Query element as fp32.
template <int QDT>
__device__ __forceinline__ float q_elem(uint32_t bits16) {
    if constexpr (QDT == KVQ_BF16) return bf16_bits_to_f32(bits16);
    else return f16_bits_to_f32(bits16);
}

template <int NVG>
struct VMeta { uint32_t m[2][NVG]; };   // (scale, zero) of tokens t, t+16 per V group

// Loads of one lane, issued a tile ahead of their use (ping-pong buffers).
// VW: 32-bit words of V codes per token and lane (8 channels: 1 at 4 bits, 2 at 8).
template <int NVG, int VW>
struct TileLoads {
    u32x4 k[2];          // codes of the lane's quarter for tokens t and t+16
    VMeta<NVG> vm;
    uint32_t v[4][2][VW];  // V code words (8 channels) of tokens ph+4j and ph+4j+16
    // table rows of tokens t, t+16; this lane's 8 bytes of the two staged
    // rows (the rows of the tile's first and last coded tokens, r0, r1)
    int32_t krow[2];
    u32x2 stg[2];
    int r0, r1;
};

// GV: channels per V group (32, 64 or 128); VB: bits per V code (4 or 8).
template <int QDT, int VB, int GV>
__global__ __launch_bounds__(256, 2) void decode_kivi_kernel(DecodeArgs a) {
    constexpr int NVG = kD / GV;      // V groups per row
    constexpr int VW = VB / 4;        // V code words per token and lane
    constexpr int kVRowB = kD * VB / 8;   // bytes of V codes per token
    constexpr float kVCenter = VB == 4 ? 8.0f : 128.0f;          // codes are centered on this
    constexpr uint32_t kVCenterNeg = VB == 4 ? 0xC800C800u : 0xD800D800u;   // fp16 (-c, -c)

    // the wave index is uniform across the wave; say so, so that tile bases and
    // buffer descriptors stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * a.Hkv + hk;
    const int t_lo = split * a.split_len;
    const int t_hi = min(a.T, t_lo + a.split_len);
    const int n_tiles = (t_hi - t_lo + kTileT - 1) / kTileT;
    const int tile0 = (n_tiles * wave) / kWaves, tile1 = (n_tiles * (wave + 1)) / kWaves;

    __shared__ uint32_t wbuf[kWaves][16][NVG][kGQ];           // fp16 weight pairs of a tile
    __shared__ __align__(16) uint32_t kst[kWaves][2][kD];     // staged table rows
    __shared__ float comb_o[kWaves][kGQ][kD];
    __shared__ float comb_ml[kWaves][kGQ][2];

    // QK role: token t16 (and t16 + 16), quarter q4 of head_dim; after the
    // reduce-scatter the lane owns query head hq = q4.
    const int t16 = lane >> 2, q4 = lane & 3;
    // PV role: phase ph (tokens ph + 4j, j < 4, and +16), chunk c (channels 8c..8c+7)
    const int ph = lane >> 4, c = lane & 15;
    const int vg_c = (8 * c) / GV;

    // ---- query: fp16 pairs for this lane's quarter, scaled by 2^-e (shared by the group)
    // (gq query heads share the kv-head; heads gq .. 3 hold zeros and are not written)
    const int gq = a.Hq / a.Hkv;
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + hk * gq) * kD;
    float qmax = 0.0f;
#pragma unroll
    for (int h = 0; h < kGQ; ++h) {
        if (h >= gq) continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 x = *reinterpret_cast<const uint4*>(q16 + h * kD + 32 * q4 + 8 * k);
            const uint32_t e4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qmax = fmaxf(qmax, fmaxf(fabsf(q_elem<QDT>(e4[i] & 0xFFFFu)), fabsf(q_elem<QDT>(e4[i] >> 16))));
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, off));
    // scale so the largest |q| lands in [2^14, 2^15): exact fp16 for bf16/fp16 inputs
    int qexp = 0;
    if (qmax > 0.0f) { frexpf(qmax, &qexp); qexp -= 15; }
    const float qscale = ldexpf(1.0f, -qexp);
    // register j of this lane holds query head (q4 + j) % 4, so that the four
    // quarter partials of head h meet in lane quarter h by quad rotations
    // only; channel pairs (8k+2i, 8k+2i+1)
    uint32_t qv[kGQ][16];
#pragma unroll
    for (int j = 0; j < kGQ; ++j) {
        const int h = (q4 + j) & 3;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float x[8];
            if (h < gq) {
                const uint4 xx = *reinterpret_cast<const uint4*>(q16 + h * kD + 32 * q4 + 8 * k);
                const uint32_t e4[4] = {xx.x, xx.y, xx.z, xx.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = q_elem<QDT>(e4[i] & 0xFFFFu);
                    x[2 * i + 1] = q_elem<QDT>(e4[i] >> 16);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) qv[j][4 * k + i] = pack_f16(x[2 * i] * qscale, x[2 * i + 1] * qscale);
        }
    }
    // logit (base 2) = scale_log2 2^qexp (q' . k)
    const float kC = ldexpf(a.scale_log2, qexp);

    const uint8_t* kcodes = static_cast<const uint8_t*>(a.k_codes) + bh * a.cap * kRowB;
    const uint8_t* vcodes = static_cast<const uint8_t*>(a.v_codes) + bh * a.cap * kVRowB;
    const uint32_t* vmeta = static_cast<const uint32_t*>(a.v_meta) + bh * a.cap * NVG;
    // the (batch, kv-head)'s table [rows][kD] of (scale, zero) fp16 pairs
    const int rows_t = a.cap / a.Gt + 3;
    const uint8_t* ktab = static_cast<const uint8_t*>(a.k_meta) + bh * rows_t * kD * 4;

    float m_lane = -INFINITY;     // running max of head q4
    float l_lane = 0.0f;          // running sum of head q4 (this lane's tokens)
    // fp16 weights are p s 2^wexp: wexp follows the largest V scale the wave
    // has seen (vsmax 2^wexp in [2^13, 2^14)), so with p <= 1 no weight
    // overflows, and any weight above 2^-27 of vsmax stays a normal fp16
    // with full relative precision.  acc and corr are in these units.
    float vsmax = 0.0f;
    int wexp = 0;
    float wmul = 1.0f;            // 2^wexp
    float corr[NVG];              // head q4, per V group
#pragma unroll
    for (int g = 0; g < NVG; ++g) corr[g] = 0.0f;
    float acc[kGQ][8];            // PV: head h; i = 2k: channel 8c+2k, i = 2k+1: byte k (scaled 2^-24)
#pragma unroll
    for (int h = 0; h < kGQ; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.0f;

    auto load_tile = [&](int tile, TileLoads<NVG, VW>& L) {
        const int tb = t_lo + tile * kTileT;
        // valid tokens in the tile (0 past the end: those loads return zeros);
        // kept in a scalar register so the buffer descriptors stay uniform
        const uint32_t nv = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(kTileT, t_hi - tb)));
        const __amdgpu_buffer_rsrc_t rk = rsrc(kcodes + (int64_t)tb * kRowB, nv * kRowB);
        const __amdgpu_buffer_rsrc_t rvm = rsrc(vmeta + (int64_t)tb * NVG, nv * NVG * 4);
        const __amdgpu_buffer_rsrc_t rv = rsrc(vcodes + (int64_t)tb * kVRowB, nv * kVRowB);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t tt = ph + 4 * j;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t off = (tt + 16 * e) * kVRowB + 4 * VW * c;
                if constexpr (VW == 1) {
                    L.v[j][e][0] = buf::stream32(rv, off);
                } else {
                    const u32x2 x = buf::stream64(rv, off);
                    L.v[j][e][0] = x.x; L.v[j][e][1] = x.y;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t tok = t16 + 16 * p;
            L.k[p] = buf::stream128(rk, tok * kRowB + 16 * q4);
            // the token's table row (slots past the tile's valid part read 0)
            const __amdgpu_buffer_rsrc_t rrow = rsrc(a.k_row + tb, nv * 4);
            L.krow[p] = (int32_t)buf::load32(rrow, tok * 4);
            if constexpr (NVG == 1) {
                L.vm.m[p][0] = buf::stream32(rvm, tok * 4);
            } else if constexpr (NVG == 2) {
                const u32x2 x = buf::stream64(rvm, tok * 8);
                L.vm.m[p][0] = x.x; L.vm.m[p][1] = x.y;
            } else {
                const u32x4 x = buf::stream128(rvm, tok * 16);
                L.vm.m[p][0] = x.x; L.vm.m[p][1] = x.y; L.vm.m[p][2] = x.z; L.vm.m[p][3] = x.w;
            }
        }
        // the table rows of the tile's first and last coded tokens, staged
        // through registers: lane l loads channels 2l, 2l+1 of each (the
        // table buffer covers the whole table, so any row index is safe)
        const int nq = max(0, min(tb + (int)nv, a.n_quant) - tb);
        int r0 = 0, r1 = 0;
        if (nq > 0) {
            r0 = a.k_row[tb];
            r1 = a.k_row[tb + nq - 1];
        }
        L.r0 = __builtin_amdgcn_readfirstlane(r0);
        L.r1 = __builtin_amdgcn_readfirstlane(r1);
        const __amdgpu_buffer_rsrc_t rtab = rsrc(ktab, (uint32_t)rows_t * kD * 4);
        L.stg[0] = buf::load64(rtab, (uint32_t)L.r0 * kD * 4 + 8 * lane);
        L.stg[1] = buf::load64(rtab, (uint32_t)L.r1 * kD * 4 + 8 * lane);
    };

    auto process = [&](const TileLoads<NVG, VW>& L, int tile, auto tail) {
        constexpr bool kTail = decltype(tail)::value;     // the tile may hold invalid tokens
        const int tb = t_lo + tile * kTileT;
        // -------------------------------------------- QK^T, two passes (t16, t16 + 16)
        float xs[2];
        // stage the two table rows; kst[wave][r][c] = (scale, zero) of channel c
        *reinterpret_cast<u32x2*>(&kst[wave][0][2 * lane]) = L.stg[0];
        *reinterpret_cast<u32x2*>(&kst[wave][1][2 * lane]) = L.stg[1];
        wave_lds_sync();
        // every token of the wave valid-and-coded with a staged row: the common case
        bool fast = true;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int t = tb + t16 + 16 * p;
            const bool staged = L.krow[p] == L.r0 || L.krow[p] == L.r1;
            fast = fast && (t >= t_hi || (t < a.n_quant && staged));
        }
        const bool all_fast = __builtin_amdgcn_ballot_w64(!fast) == 0;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int t = tb + t16 + 16 * p;
            const uint32_t kw[4] = {L.k[p].x, L.k[p].y, L.k[p].z, L.k[p].w};
            // register j: query head (q4 + j) % 4 over this quarter; eight
            // channels at a time, exact fp16 x fp32 products
            float part[kGQ];
#pragma unroll
            for (int j = 0; j < kGQ; ++j) part[j] = 0.0f;
            auto chunk = [&](int k, const float xk[8]) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < kGQ; ++j)
#pragma unroll
                    for (int i = 0; i < 8; i += 2) {
                        part[j] = fma_lo(qv[j][4 * k + i / 2], xk[i], part[j]);
                        part[j] = fma_hi(qv[j][4 * k + i / 2], xk[i + 1], part[j]);
                    }
            };
            // keys of channels 8k .. 8k+7 of the quarter: k = u s + z from the row's (scale, zero) pairs
            auto deq = [&](int k, const uint32_t m[8], float xk[8]) __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < 8; ++i) xk[i] = fmaf((float)((kw[k] >> (4 * i)) & 0xFu), f16lo(m[i]), f16hi(m[i]));
            };
            if (all_fast) {
                const uint32_t* row = &kst[wave][L.krow[p] == L.r0 ? 0 : 1][32 * q4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint4 m0 = *reinterpret_cast<const uint4*>(row + 8 * k);
                    const uint4 m1 = *reinterpret_cast<const uint4*>(row + 8 * k + 4);
                    const uint32_t m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
                    float xk[8];
                    deq(k, m, xk);
                    chunk(k, xk);
                }
            } else {
                // per lane: past the split (zeros), the open group (the
                // full-precision residual), a staged row, or a row in memory
                const bool staged = L.krow[p] == L.r0 || L.krow[p] == L.r1;
                const uint32_t* row = staged ? &kst[wave][L.krow[p] == L.r0 ? 0 : 1][32 * q4]
                                             : reinterpret_cast<const uint32_t*>(ktab) + (int64_t)L.krow[p] * kD + 32 * q4;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float xk[8];
                    if (t >= t_hi) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) xk[i] = 0.0f;
                    } else if (t >= a.n_quant) {
                        dq::load8(a.k_resid, (bh * a.Gt + (t - a.n_quant)) * kD + 32 * q4 + 8 * k, a.in_dtype, xk);
                    } else {
                        const uint4 m0 = *reinterpret_cast<const uint4*>(row + 8 * k);
                        const uint4 m1 = *reinterpret_cast<const uint4*>(row + 8 * k + 4);
                        const uint32_t m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
                        deq(k, m, xk);
                    }
                    chunk(k, xk);
                }
            }
            const float xl = (part[0] + quad_from_minus<1>(part[1]) + quad_from_minus<2>(part[2]) +
                              quad_from_minus<3>(part[3])) * kC;
            if constexpr (kTail) xs[p] = t < t_hi ? xl : -INFINITY;
            else xs[p] = xl;
        }

        // -------------------------------------------- online softmax (rescale on a new max)
        const bool grow = (xs[0] > m_lane) || (xs[1] > m_lane);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            float mt = fmaxf(xs[0], xs[1]);
#pragma unroll
            for (int off = 4; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
            const float m_new = fmaxf(m_lane, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_lane - m_new);
            m_lane = m_new;
            l_lane *= alpha;
#pragma unroll
            for (int g = 0; g < NVG; ++g) corr[g] *= alpha;
#pragma unroll
            for (int h = 0; h < kGQ; ++h) {
                // lane h owns head h
                const float ah = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] *= ah;
            }
        }
        // -------------------------------------------- weight scale (rescale on a new largest V scale)
        // lanes of equal q4 hold the V scales of all the tile's tokens
        float sl = 0.0f;
#pragma unroll
        for (int g = 0; g < NVG; ++g) sl = fmaxf(sl, fmaxf(f16lo(L.vm.m[0][g]), f16lo(L.vm.m[1][g])));
        if (__builtin_amdgcn_ballot_w64(sl > vsmax) != 0) {
#pragma unroll
            for (int off = 4; off < 64; off <<= 1) sl = fmaxf(sl, __shfl_xor(sl, off));
            vsmax = fmaxf(vsmax, sl);
            int e;
            frexpf(vsmax, &e);                        // vsmax in [2^(e-1), 2^e)
            const float f = ldexpf(1.0f, 14 - e - wexp);
            wexp = 14 - e;
            wmul = ldexpf(1.0f, wexp);
#pragma unroll
            for (int g = 0; g < NVG; ++g) corr[g] *= f;
#pragma unroll
            for (int h = 0; h < kGQ; ++h)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] *= f;
        }
        // v_exp_f32: weights below 2^-126 of the running max may flush to zero
        const float p0 = __builtin_amdgcn_exp2f(xs[0] - m_lane);
        const float p1 = __builtin_amdgcn_exp2f(xs[1] - m_lane);
        l_lane += p0 + p1;
        const float pw0 = p0 * wmul, pw1 = p1 * wmul;   // exact: a power of two
#pragma unroll
        for (int g = 0; g < NVG; ++g) {
            const uint32_t m0 = L.vm.m[0][g], m1 = L.vm.m[1][g];
            const uint32_t pair = pack_f16(mul_lo(m0, pw0), mul_lo(m1, pw1));
            float cg = corr[g];
            cg = fmaf(pw0, fmaf(kVCenter, f16lo(m0), f16hi(m0)), cg);
            cg = fmaf(pw1, fmaf(kVCenter, f16lo(m1), f16hi(m1)), cg);
            corr[g] = dot2_f16(pair, kVCenterNeg /* (-c, -c) */, cg);
            wbuf[wave][t16][g][q4] = pair;
        }
        wave_lds_sync();

        // -------------------------------------------- PV
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 wp = *reinterpret_cast<const uint4*>(&wbuf[wave][ph + 4 * j][vg_c][0]);
            const uint32_t wpair[kGQ] = {wp.x, wp.y, wp.z, wp.w};
            uint32_t cp[8];
            if constexpr (VB == 4) {
                const uint32_t w0 = L.v[j][0][0], w1 = L.v[j][1][0];
                // byte k of both tokens as an fp16 subnormal pair (b_t, b_t+16),
                // b = u_2k + 16 u_2k+1, and its low nibbles (u_2k of both tokens);
                // the high-nibble channel is separated once at the end
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t P = __builtin_amdgcn_perm(w1, w0, 0x0C040C00u + 0x00010001u * k);
                    cp[2 * k] = P & 0x000F000Fu;
                    cp[2 * k + 1] = P;
                }
            } else {
                // 8-bit codes: byte i of both tokens is channel 8c + i
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    cp[i] = __builtin_amdgcn_perm(L.v[j][1][i >> 2], L.v[j][0][i >> 2], 0x0C040C00u + 0x00010001u * (i & 3));
            }
#pragma unroll
            for (int h = 0; h < kGQ; ++h)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] = dot2_f16(wpair[h], cp[i], acc[h][i]);
        }
        wave_lds_sync();
    };

    // two load buffers in ping-pong: the next tile's loads are in flight while
    // the current tile is computed
    // Full tiles run in a ping-pong loop with unconditional prefetches (a
    // prefetch past the end reads zeros and is never used); only the split's
    // last tile can be partial and is processed with token masking.
    TileLoads<NVG, VW> A, B2;
    const int full_end = min(tile1, (t_hi - t_lo) / kTileT);
    int tile = tile0;
    load_tile(tile, A);
    for (; tile + 1 < full_end; tile += 2) {
        load_tile(tile + 1, B2);
        process(A, tile, Flag<false>{});
        load_tile(tile + 2, A);
        process(B2, tile + 1, Flag<false>{});
    }
    if (tile < full_end) {                // one full tile left
        process(A, tile, Flag<false>{});
        ++tile;
        if (tile < tile1) load_tile(tile, A);
    }
    if (tile < tile1) process(A, tile, Flag<true>{});

    // ---------------------------------------------------- wave-level reduction
    // PV: sum the 4 phases (lanes c, c+16, c+32, c+48), undo the 2^-24 code
    // scale and split each byte sum into its two channels:
    // u_2k+1 = (b - u_2k) / 16
#pragma unroll
    for (int h = 0; h < kGQ; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = acc[h][i];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[h][i] = v;
        }
    // undo the code scale 2^-24 and the weight scale 2^wexp (exact)
    const float unit = ldexpf(1.0f, 24 - wexp), unit16 = ldexpf(1.0f, 20 - wexp), unitc = ldexpf(1.0f, -wexp);
#pragma unroll
    for (int h = 0; h < kGQ; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float lo = acc[h][2 * k], whole = acc[h][2 * k + 1];
            if constexpr (VB == 4) {
                acc[h][2 * k] = lo * unit;
                acc[h][2 * k + 1] = (whole - lo) * unit16;      // / 16
            } else {
                acc[h][2 * k] = lo * unit;
                acc[h][2 * k + 1] = whole * unit;
            }
        }
    // head q4 sums over the lane's tokens: reduce over lanes with equal q4
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) {
        l_lane += __shfl_xor(l_lane, off);
#pragma unroll
        for (int g = 0; g < NVG; ++g) corr[g] += __shfl_xor(corr[g], off);
    }
#pragma unroll
    for (int h = 0; h < kGQ; ++h) {
        // corrections of head h for this chunk's V group live in lane h
        float cv = 0.0f;
#pragma unroll
        for (int g = 0; g < NVG; ++g) {
            const float cg = __shfl(corr[g], h);
            cv = (g == vg_c) ? cg : cv;
        }
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < 8; ++i) comb_o[wave][h][c * 8 + i] = fmaf(cv, unitc, acc[h][i]);
        }
    }
    if (lane < kGQ) {
        comb_ml[wave][lane][0] = m_lane;
        comb_ml[wave][lane][1] = l_lane;
    }
    __syncthreads();
    // ---------------------------------------------------- merge the 4 waves
    const int ns = a.n_splits;
    for (int idx = threadIdx.x; idx < kGQ * kD; idx += 256) {
        const int h = idx / kD, d = idx % kD;
        if (h >= gq) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, comb_ml[w][h][0]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = comb_ml[w][h][0];
            const float f = mw == -INFINITY ? 0.0f : exp2f(mw - M);
            num = fmaf(f, comb_o[w][h][d], num);
            den = fmaf(f, comb_ml[w][h][1], den);
        }
        const int64_t row = (int64_t)b * a.Hq + hk * gq + h;
        if (ns == 1) {
            a.out[row * kD + d] = num / den;
        } else {
            a.ws_o[(row * ns + split) * kD + d] = num;
            if (d == 0) {
                a.ws_ml[(row * ns + split) * 2 + 0] = M;
                a.ws_ml[(row * ns + split) * 2 + 1] = den;
            }
        }
    }
}

}  // namespace

// The fast decode covers D = 128, bf16 or fp16 queries, affine 4- or 8-bit V
// and no RoPE on read, with per-token 4-bit K (affine groups or symmetric
// blocks, 4 query heads per kv-head: decode_mfma.hip; a per-key rotation
// would undo the factored scale) or KIVI 4-bit K (1-4 query heads per
// kv-head: this file).
bool decode_fast_applies(const DecodeArgs& a) {
    if (decode_mfma_applies(a)) return true;
    const bool v_ok = a.v_kind == KVQ_TOK_AFFINE && (a.v_bits == 4 || a.v_bits == 8);
    const bool heads_ok = a.Hq % a.Hkv == 0 && a.Hq >= a.Hkv && a.Hq <= kGQ * a.Hkv;
    return a.k_kind == KVQ_KIVI_CH && a.k_bits == 4 && v_ok && heads_ok && a.D == kD &&
           (a.q_dtype == KVQ_BF16 || a.q_dtype == KVQ_F16) && !a.rope;
}

// Split plan: one workgroup per (batch, kv-head) when that fills the chip
// twice over, otherwise split the tokens so that about 512 workgroups run.
void decode_fast_plan(int B, int Hkv, int T, int* n_splits, int* split_len) {
    const int units = B * Hkv;
    int ns = (512 + units - 1) / units;
    // at least 2 tiles per wave, so that each wave's second tile loads while
    // its first is computed (the best latency for small batches)
    const int min_len = kWaves * kTileT * 2;
    const int max_ns = (T + min_len - 1) / min_len;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    int len = (T + ns - 1) / ns;
    len = ((len + kTileT - 1) / kTileT) * kTileT;
    *split_len = len;
    *n_splits = (T + len - 1) / len;
}

template <int QDT, int VB>
static hipError_t launch_kivi_v(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.n_splits, (unsigned)a.Hkv, (unsigned)a.B);
    switch (a.v_group) {
        case 32: hipLaunchKernelGGL((decode_kivi_kernel<QDT, VB, 32>), grid, dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL((decode_kivi_kernel<QDT, VB, 64>), grid, dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL((decode_kivi_kernel<QDT, VB, 128>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int QDT>
static hipError_t launch_kivi_q(const DecodeArgs& a, hipStream_t s) {
    return a.v_bits == 8 ? launch_kivi_v<QDT, 8>(a, s) : launch_kivi_v<QDT, 4>(a, s);
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s) {
    if (decode_mfma_applies(a)) return launch_decode_mfma(a, s);
    if (a.q_dtype == KVQ_BF16) return launch_kivi_q<KVQ_BF16>(a, s);
    return launch_kivi_q<KVQ_F16>(a, s);
}

}  // namespace kvq

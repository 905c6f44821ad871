// decode_mfma.hip -- decode attention for per-token 4-bit K (affine groups,
// mlx-lm style, "Low-bit KV caches on MLX", s.1; or symmetric blocks of 32,
// "kv-cache: optional per-channel K-cache mean-centering for Q4_0") and
// per-token affine 4- or 8-bit V at head_dim 128 and 4 query heads per
// kv-head, with both products on the matrix cores (gfx950,
// v_mfma_f32_16x16x32_f16).
//
// Work split: 4 waves per (batch, kv-head[, token split]) (8 for KIVI keys
// in splits of at most 8 tiles), each with its own online softmax over
// every fourth (eighth) 32-token tile of the split (so the waves of a
// workgroup stream one region of the cache together, which keeps fewer DRAM
// streams open than separate runs), merged through LDS
// (token splits merge in a combine kernel).  What changes is where the multiply-adds run.  A 4-bit code left
// in place under a mask is an fp16 subnormal (u 2^-24 for a low nibble,
// u 2^-20 for a high one), and the matrix cores multiply subnormal fp16
// operands exactly, so the codes feed the MFMA B operand with one AND each.
// Lane l below is (r, n) = (l >> 4, l & 15).
//
// * Scores, per 16-token block: C = A B over the 128 channels in 4 MFMAs of
//   32 channels.  B column n is token n; lane (r, n) supplies channels
//   32r .. 32r+31 of it (one 16-byte load).  A row i = 4qq + h holds query
//   head h restricted to channel quarter qq (zero elsewhere), so C row
//   (qq, h) is the partial dot product of head h over quarter qq, and lane
//   (r, n) ends with the quarter-r partials of all four heads for token n.
//   Each lane applies its token's (scale, zero) of the quarter's group:
//     q . k = sum_qq [ s (q . u)_qq + z (sum q)_qq ]
//   and two cross-row exchanges sum the quarters, leaving lane (r, n) with
//   the logit of head r for token n.  The query is held as fp16 scaled by a
//   power of two (exact for bf16 and fp16 queries), high-nibble channels
//   pre-divided by 16.
// * Softmax: lane (h, n) owns head h for tokens n and n + 16 of the tile,
//   with a lazily rescaled running max as in the VALU decode, and writes the
//   fp16 weight pairs w^ = fp16(p s 2^E) per V group to LDS.  E is the wave's
//   weight exponent: it follows the largest V scale seen so far (rescaling
//   the accumulators when it changes, as for a new running max), so that
//   small V scales do not push the weights into fp16's subnormal range,
//   and it is taken out exactly at the end.
// * Values: O = W V over the tile's 32 tokens in one MFMA per code byte
//   position and kind.  W row i = 4g + h holds head h's weights for V group
//   g (one 16-byte LDS read per lane); V column n is code word n (4-bit:
//   channels 8n .. 8n+7), and one v_perm_b32 per token pair gives the whole
//   bytes b = u_2k + 16 u_2k+1 of tokens (t, t + 16) as subnormal fp16
//   pairs, one AND their low nibbles.  The high-nibble channel is (byte sum -
//   low sum) / 16 at the end.  8-bit codes are whole bytes already: words n
//   and n + 16 (channels 4n .. 4n+3 and 64 + 4n ..) give one MFMA per byte;
//   their tile is fetched with 16-byte loads and staged in LDS, from where
//   each lane reads its words (16 single-dword fetches per lane and tile
//   would cost more).
//   Only the rows of a column's own V group are kept.  The zero points and
//   the rounding of the weights are accounted exactly in fp32 as in the VALU
//   decode (c = 8 for 4-bit codes, 128 for 8-bit):
//     o = sum_t w^_t u_t + sum_t p_t (z_t + c s_t) - c sum_t w^_t
// * Symmetric K blocks (value (u - 8) d) are the affine case with s = d and
//   z = -8 d.
// * Loads go through buffer resources sized to the valid part of a tile, so
//   tail tokens read zeros; the last tile of a split masks their logits.
//   They carry the non-temporal cache policy: the cache is read once per
//   step.
#include <math.h>

#include "bufload.h"
#include "dequant8.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using buf::u32x4;

constexpr int kD = 128;
constexpr int kGQ = 4;          // query heads per kv-head
constexpr int kTileT = 32;      // tokens per wave tile
constexpr int kWaves = 4;
constexpr int kRowB = kD / 2;   // bytes of 4-bit K codes per token
constexpr int kKAff4 = 0;       // per-token affine K groups: (scale, zero) fp16 pairs
constexpr int kKSym4 = 1;       // symmetric K blocks of 32: one fp16 scale d, value (u - 8) d
constexpr int kKKivi = 2;       // KIVI per-channel K: (scale, zero) per channel from the token's group row

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma16(u32x4 a, u32x4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0,
                                                  0);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    half2_t h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float f16lo(uint32_t u) { return (float)__builtin_bit_cast(half2_t, u).x; }
__device__ __forceinline__ float f16hi(uint32_t u) { return (float)__builtin_bit_cast(half2_t, u).y; }
template <int QDT>
__device__ __forceinline__ float q_elem(uint32_t bits16) {
    if constexpr (QDT == KVQ_BF16) return bf16_bits_to_f32(bits16);
    else return f16_bits_to_f32(bits16);
}
template <bool B>
struct Flag { static constexpr bool value = B; };


// The four code-word nibble masks as the B operand of one 32-channel MFMA:
// fp16 slots (c0, c4, c1, c5, c2, c6, c3, c7) of the word's eight channels,
// odd channels 16x (their query slots carry 1/16).
__device__ __forceinline__ u32x4 nibble_operand(uint32_t w) {
    const uint32_t w8 = w >> 8;
    return u32x4{w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
}

// Loads of one lane for one tile, issued a tile ahead of their use.
// VH: V code words per token and lane (1 at 4 bits, 2 at 8).
template <int NVG, int VH>
struct MTile {
    u32x4 k[2];          // K codes of channels 32r .. 32r+31, tokens n and n + 16
    uint32_t km[2];      // K (scale, zero) of that quarter's group (symmetric: d), tokens n and n + 16
    uint32_t vm[2][NVG]; // V (scale, zero) per group, tokens n and n + 16
    uint32_t v[4][2][VH];  // V code words n (and n + 16) of tokens 4r + j and 4r + j + 16
    u32x4 vraw[4];         // 8-bit V codes of the tile, 16-byte units lane + 64 q
    int32_t krow[2];       // KIVI: table rows of tokens n and n + 16
    buf::u32x2 stg[2];     // KIVI: this lane's 8 bytes of table rows r0, r1
    int r0, r1;            // KIVI: rows of the tile's first and last coded tokens
};

// KF: K format (kKAff4; kKSym4 or kKKivi with GK = 32); GK, GV: channels
// per K / V group (32, 64 or 128); VB: bits per V code (4 or 8); NW: waves
// per workgroup (4, two workgroups per CU; 8, one, for splits of at most 8
// tiles, where a wave's second tile would only lengthen the latency chain).
template <int QDT, int KF, int GK, int VB, int GV, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void decode_mfma_kernel(DecodeArgs a) {
    static_assert(KF == kKAff4 || GK == 32, "symmetric and KIVI keys take GK = 32");
    constexpr int NKG = kD / GK;
    constexpr int NVG = kD / GV;
    constexpr int VH = VB / 4;
    constexpr int kVRowB = kD * VB / 8;              // bytes of V codes per token
    constexpr int kKMetaB = KF == kKSym4 ? 2 : 4;    // bytes per K group and token
    constexpr float kVCenter = VB == 4 ? 8.0f : 128.0f;                       // V codes are centered on this
    constexpr uint32_t kVCenterNeg = VB == 4 ? 0xC800C800u : 0xD800D800u;     // fp16 (-c, -c)

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 15, r = lane >> 4;
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * a.Hkv + hk;
    const int t_lo = split * a.split_len;
    const int t_hi = min(a.T, t_lo + a.split_len);
    const int n_tiles = (t_hi - t_lo + kTileT - 1) / kTileT;

    __shared__ __align__(16) uint32_t wbuf[NW][NVG][kGQ][16];   // fp16 weight pairs (t, t + 16)
    __shared__ __align__(16) uint32_t vst[VB == 8 ? NW : 1][kTileT][36];     // 8-bit V code rows (32 words + pad)
    __shared__ float comb_o[NW][kGQ][kD];
    __shared__ float comb_ml[NW][kGQ][2];
    // KIVI keys: the staged table rows r0, r1 ((scale, zero) per channel),
    // the A operands built from one of them ([hi | lo][head][channel chunk]),
    // and the query of all heads for tokens that take the per-lane path
    constexpr int KW = KF == kKKivi ? NW : 1;
    __shared__ __align__(16) uint32_t kst[KW][2][kD];
    __shared__ __align__(16) u32x4 abuf[KW][2][kGQ][16];
    __shared__ __align__(16) float qbuf[KF == kKKivi ? kGQ : 1][kD];

    // ---- query: lane (r, n) reads channels 32r .. 32r+31 of head n & 3
    // (gq query heads per kv-head; the rows of heads gq .. 3 are zero)
    const int gq = a.Hq / a.Hkv;
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + hk * gq) * kD;
    float x[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint4 xx = make_uint4(0u, 0u, 0u, 0u);
        if ((n & 3) < gq) xx = *reinterpret_cast<const uint4*>(q16 + (n & 3) * kD + 32 * r + 8 * k);
        const uint32_t e4[4] = {xx.x, xx.y, xx.z, xx.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[8 * k + 2 * i] = q_elem<QDT>(e4[i] & 0xFFFFu);
            x[8 * k + 2 * i + 1] = q_elem<QDT>(e4[i] >> 16);
        }
    }
    float qmax = 0.0f, qpart = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        qmax = fmaxf(qmax, fabsf(x[i]));
        qpart += x[i];
    }
    qmax = wave64_max(qmax);
    // scale so the largest |q| lands in [2^14, 2^15): exact fp16 for bf16/fp16 inputs
    int qexp = 0;
    if (qmax > 0.0f) { frexpf(qmax, &qexp); qexp -= 15; }
    const float qscale = ldexpf(1.0f, -qexp);
    // A operands of the score MFMAs: row n = (quarter n >> 2, head n & 3) is
    // nonzero only in the lanes of its own quarter (r == n >> 2)
    const bool own = (n >> 2) == r;
    u32x4 qa[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float* xc = x + 8 * c;
        const float s = own ? qscale : 0.0f, s16 = s * 0.0625f;
        qa[c] = u32x4{pack_f16(xc[0] * s, xc[4] * s), pack_f16(xc[1] * s16, xc[5] * s16),
                      pack_f16(xc[2] * s, xc[6] * s), pack_f16(xc[3] * s16, xc[7] * s16)};
    }
    // zero-point terms: sum of head h's query over quarter r (lane (r, h) holds it), / 2^(qexp + 24)
    float qsk[kGQ];
    // lane (r, h) of this lane's row, by DPP row broadcasts
    qsk[0] = ldexpf(__uint_as_float(dpp_u32<0x150>(__float_as_uint(qpart))), -(qexp + 24));
    qsk[1] = ldexpf(__uint_as_float(dpp_u32<0x151>(__float_as_uint(qpart))), -(qexp + 24));
    qsk[2] = ldexpf(__uint_as_float(dpp_u32<0x152>(__float_as_uint(qpart))), -(qexp + 24));
    qsk[3] = ldexpf(__uint_as_float(dpp_u32<0x153>(__float_as_uint(qpart))), -(qexp + 24));
    // logit (base 2) = kC sum_quarters (s C + z qsk)
    const float kC = ldexpf(a.scale_log2, qexp + 24);
    const int kg = (32 * r) / GK;   // K group of this lane's quarter

    // KIVI: lane l builds the A operands of head l >> 4 over channels
    // 8 (l & 15) .. +7 (qx8); eq: qmax < 2^eq
    float qx8[8];
    int eq = 0;
    const uint32_t* ktab = nullptr;
    int rows_t = 0;
    if constexpr (KF == kKKivi) {
        const int hh = lane >> 4, c8 = 8 * (lane & 15);
        uint4 xx = make_uint4(0u, 0u, 0u, 0u);
        if (hh < gq) xx = *reinterpret_cast<const uint4*>(q16 + hh * kD + c8);
        const uint32_t e4[4] = {xx.x, xx.y, xx.z, xx.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qx8[2 * i] = q_elem<QDT>(e4[i] & 0xFFFFu);
            qx8[2 * i + 1] = q_elem<QDT>(e4[i] >> 16);
        }
        if (qmax > 0.0f) frexpf(qmax, &eq);
        if (wave == 0 && n < kGQ) {
#pragma unroll
            for (int i = 0; i < 32; ++i) qbuf[n][32 * r + i] = x[i];
        }
        __syncthreads();
        rows_t = a.cap / a.Gt + 3;
        ktab = static_cast<const uint32_t*>(a.k_meta) + bh * rows_t * kD;
    }

    const uint8_t* kcodes = static_cast<const uint8_t*>(a.k_codes) + bh * a.cap * kRowB;
    const uint8_t* vcodes = static_cast<const uint8_t*>(a.v_codes) + bh * a.cap * kVRowB;
    const uint8_t* kmeta = static_cast<const uint8_t*>(a.k_meta) + bh * a.cap * NKG * kKMetaB;
    const uint8_t* vmeta = static_cast<const uint8_t*>(a.v_meta) + bh * a.cap * NVG * 4;

    float m_lane = -INFINITY;     // running max of head r
    float l_lane = 0.0f;          // running sum of head r over this lane's tokens
    // fp16 weights are p s 2^wexp: wexp follows the largest V scale the wave
    // has seen (vsmax 2^wexp in [2^13, 2^14)), so with p <= 1 no weight
    // overflows, and any weight above 2^-27 of vsmax stays a normal fp16
    // with full relative precision.  acc and corr are in these units.
    float vsmax = 0.0f;
    int wexp = 0;
    float wmul = 1.0f;            // 2^wexp
    float corr[NVG];              // head r, per V group: (sum p (z + c s) - c sum w^) 2^wexp
#pragma unroll
    for (int g = 0; g < NVG; ++g) corr[g] = 0.0f;
    // PV: row (g = r, h = i) of column n, scaled 2^-24.  4-bit codes: acc[k]
    // the whole bytes k, acc[4 + k] their low nibbles; 8-bit: acc[4 hb + k]
    // byte k of word n + 16 hb
    f4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    auto load_tile = [&](int tile, MTile<NVG, VH>& L) {
        const int tb = t_lo + tile * kTileT;
        // valid tokens in the tile (0 past the end: those loads return zeros),
        // in a scalar register so that the descriptors stay uniform
        const uint32_t nv = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(kTileT, t_hi - tb)));
        const __amdgpu_buffer_rsrc_t rk = buf::rsrc(kcodes + (int64_t)tb * kRowB, nv * kRowB);
        const __amdgpu_buffer_rsrc_t rkm = buf::rsrc(kmeta + (int64_t)tb * NKG * kKMetaB, nv * NKG * kKMetaB);
        const __amdgpu_buffer_rsrc_t rvm = buf::rsrc(vmeta + (int64_t)tb * NVG * 4, nv * NVG * 4);
        const __amdgpu_buffer_rsrc_t rv = buf::rsrc(vcodes + (int64_t)tb * kVRowB, nv * kVRowB);
        if constexpr (VB == 8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) L.vraw[q] = buf::stream128(rv, 16 * (lane + 64 * q));
        } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int hb = 0; hb < VH; ++hb)
                    L.v[j][e][hb] = buf::stream32(rv, (4 * r + j + 16 * e) * kVRowB + 4 * (n + 16 * hb));
        }
        if constexpr (KF == kKKivi) {
            // each token's table row (past the tile's valid part: 0), and the
            // rows of its first and last coded tokens, staged through registers
            // (lane l: channels 2l, 2l + 1; the table resource covers every row)
            const __amdgpu_buffer_rsrc_t rrow = buf::rsrc(a.k_row + tb, nv * 4);
#pragma unroll
            for (int p = 0; p < 2; ++p) L.krow[p] = (int32_t)buf::load32(rrow, (n + 16 * p) * 4);
            const int nq = max(0, min(tb + (int)nv, a.n_quant) - tb);
            int q0 = 0, q1 = 0;
            if (nq > 0) {
                q0 = a.k_row[tb];
                q1 = a.k_row[tb + nq - 1];
            }
            L.r0 = __builtin_amdgcn_readfirstlane(q0);
            L.r1 = __builtin_amdgcn_readfirstlane(q1);
            const __amdgpu_buffer_rsrc_t rtab = buf::rsrc(ktab, (uint32_t)rows_t * kD * 4);
            L.stg[0] = buf::load64(rtab, (uint32_t)L.r0 * kD * 4 + 8 * lane);
            L.stg[1] = buf::load64(rtab, (uint32_t)L.r1 * kD * 4 + 8 * lane);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t tok = n + 16 * p;
            L.k[p] = buf::stream128(rk, tok * kRowB + 16 * r);
            if constexpr (KF == kKSym4) L.km[p] = buf::stream16(rkm, (tok * NKG + kg) * 2);
            else if constexpr (KF == kKAff4) L.km[p] = buf::stream32(rkm, (tok * NKG + kg) * 4);
            if constexpr (NVG == 1) {
                L.vm[p][0] = buf::stream32(rvm, tok * 4);
            } else if constexpr (NVG == 2) {
                const buf::u32x2 v2 = buf::stream64(rvm, tok * 8);
                L.vm[p][0] = v2.x; L.vm[p][1] = v2.y;
            } else {
                const u32x4 v4 = buf::stream128(rvm, tok * 16);
                L.vm[p][0] = v4.x; L.vm[p][1] = v4.y; L.vm[p][2] = v4.z; L.vm[p][3] = v4.w;
            }
        }
    };

    // KIVI keys.  A 16-token block whose coded tokens share a table row g
    // runs on the matrix cores: with the row's (s, z) per channel,
    //   q . k = sum_c (q_c s_c) u_c + sum_c q_c z_c,
    // so the A operand is q o s, held as an exact fp16 pair hi + lo (q and s
    // carry at most 11 significant bits each, so q_c s_c has at most 22 and
    // hi takes the top 11, lo the rest), scaled by 2^E so that the largest
    // element stays below 2^15; odd channels carry a further 1/16 for the
    // high-nibble operand.  The tile's first and last coded tokens name the
    // two staged rows; tokens of another row or of the open group (the
    // full-precision residual) take a per-lane path.
    auto kivi_scores = [&](const MTile<NVG, VH>& L, int tb, float (&y)[2][kGQ]) __attribute__((always_inline)) {
        *reinterpret_cast<buf::u32x2*>(&kst[wave][0][2 * lane]) = L.stg[0];
        *reinterpret_cast<buf::u32x2*>(&kst[wave][1][2 * lane]) = L.stg[1];
        wave_lds_sync();
        // 0: coded with row r0; 1: coded with row r1 (!= r0); 2: the per-lane
        // path; 3: past the split (codes read as zero, logit masked)
        int cls[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int t = tb + n + 16 * p;
            cls[p] = t >= t_hi ? 3 : t >= a.n_quant ? 2 : L.krow[p] == L.r0 ? 0 : L.krow[p] == L.r1 ? 1 : 2;
#pragma unroll
            for (int h = 0; h < kGQ; ++h) y[p][h] = 0.0f;
        }
        const uint32_t kw[2][4] = {{L.k[0].x, L.k[0].y, L.k[0].z, L.k[0].w},
                                   {L.k[1].x, L.k[1].y, L.k[1].z, L.k[1].w}};
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if (__builtin_amdgcn_ballot_w64(cls[0] == g || cls[1] == g) == 0) continue;
            // A operands of row g: lane l takes head l >> 4, channels 8 ci .. 8 ci + 7
            const int hh = lane >> 4, ci = lane & 15;
            const uint4 m0 = *reinterpret_cast<const uint4*>(&kst[wave][g][8 * ci]);
            const uint4 m1 = *reinterpret_cast<const uint4*>(&kst[wave][g][8 * ci + 4]);
            const uint32_t mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            float smax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) smax = fmaxf(smax, f16lo(mm[i]));
            smax = row16_max(smax);
            int es = 0;
            frexpf(smax, &es);                    // |q s| < 2^(eq + es)
            const int E = 15 - eq - es;
            const float se = ldexpf(1.0f, E), so = ldexpf(1.0f, E - 4);
            float hv[8], lv[8];
            float qzp = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = qx8[i] * f16lo(mm[i]) * ((i & 1) ? so : se);   // exact
                hv[i] = (float)(_Float16)v;
                lv[i] = v - hv[i];                                            // exact
                qzp = fmaf(qx8[i], f16hi(mm[i]), qzp);
            }
            // fp16 slot order of nibble_operand: channels (0, 4, 1, 5, 2, 6, 3, 7)
            abuf[wave][0][hh][ci] = u32x4{pack_f16(hv[0], hv[4]), pack_f16(hv[1], hv[5]), pack_f16(hv[2], hv[6]),
                                          pack_f16(hv[3], hv[7])};
            abuf[wave][1][hh][ci] = u32x4{pack_f16(lv[0], lv[4]), pack_f16(lv[1], lv[5]), pack_f16(lv[2], lv[6]),
                                          pack_f16(lv[3], lv[7])};
            qzp = row16_sum(qzp);                 // q . z of head hh
            float qz[kGQ];
#pragma unroll
            for (int h = 0; h < kGQ; ++h)
                qz[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qzp), 16 * h));
            wave_lds_sync();
            // row n = (quarter, head n & 3) carries the head's operand over
            // every quarter (the scales are folded into it), so each row of
            // the product is the head's whole dot product
            u32x4 ah[4], al[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ah[c] = abuf[wave][0][n & 3][4 * r + c];
                al[c] = abuf[wave][1][n & 3][4 * r + c];
            }
            wave_lds_sync();                      // abuf is rebuilt for the next row
            const float fu = ldexpf(1.0f, 24 - E);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const bool mem = cls[p] == g;
                f4 cq = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 bw = nibble_operand(mem ? kw[p][c] : 0u);   // zero codes: no term
                    cq = mfma16(ah[c], bw, cq);
                    cq = mfma16(al[c], bw, cq);
                }
                if (mem) {
#pragma unroll
                    for (int h = 0; h < kGQ; ++h) y[p][h] = fmaf(cq[h], fu, qz[h]);
                }
            }
        }
        if (__builtin_amdgcn_ballot_w64(cls[0] == 2 || cls[1] == 2) != 0) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                float part[kGQ];
#pragma unroll
                for (int h = 0; h < kGQ; ++h) part[h] = 0.0f;
                if (cls[p] == 2) {
                // keys of channels 32r .. 32r+31: the residual row, or u s + z from the token's row
                const int t = tb + n + 16 * p;
                float kv[32];
                if (t >= a.n_quant) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        dq::load8(a.k_resid, (bh * a.Gt + (t - a.n_quant)) * kD + 32 * r + 8 * k, a.in_dtype,
                                  kv + 8 * k);
                } else {
                    const uint32_t* row = ktab + (int64_t)L.krow[p] * kD + 32 * r;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint4 m0 = *reinterpret_cast<const uint4*>(row + 8 * k);
                        const uint4 m1 = *reinterpret_cast<const uint4*>(row + 8 * k + 4);
                        const uint32_t mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            kv[8 * k + i] = fmaf((float)((kw[p][k] >> (4 * i)) & 0xFu), f16lo(mm[i]), f16hi(mm[i]));
                    }
                }
#pragma unroll
                for (int h = 0; h < kGQ; ++h) {
                    float acc = 0.0f;
#pragma unroll
                    for (int i = 0; i < 32; ++i) acc = fmaf(qbuf[h][32 * r + i], kv[i], acc);
                    part[h] = acc;
                }
                }
                // the whole dot products: add the four quarters (lanes r = 0 .. 3 of the token)
#pragma unroll
                for (int h = 0; h < kGQ; ++h) {
                    part[h] = swap16_sum(part[h], part[h]);
                    part[h] = swap32_sum(part[h], part[h]);
                }
                if (cls[p] == 2) {
#pragma unroll
                    for (int h = 0; h < kGQ; ++h) y[p][h] = part[h];
                }
            }
        }
    };

    auto process = [&](const MTile<NVG, VH>& L, int tile, auto tail) {
        constexpr bool kTail = decltype(tail)::value;     // the tile may hold invalid tokens
        const int tb = t_lo + tile * kTileT;
        // -------------------------------------------- scores of tokens n and n + 16
        // y[p][h]: quarter r of head h's dot product for token n + 16 p (KIVI:
        // the whole dot product, in every lane)
        float y[2][kGQ];
        if constexpr (KF == kKKivi) {
            kivi_scores(L, tb, y);
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                f4 cq = f4{0.0f, 0.0f, 0.0f, 0.0f};
                const uint32_t kw[4] = {L.k[p].x, L.k[p].y, L.k[p].z, L.k[p].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) cq = mfma16(qa[c], nibble_operand(kw[c]), cq);
                // quarter r of the four heads: s C + z qsk
                const float sk = f16lo(L.km[p]);
                const float zk = KF == kKSym4 ? -8.0f * sk : f16hi(L.km[p]);
#pragma unroll
                for (int h = 0; h < kGQ; ++h) y[p][h] = fmaf(sk, cq[h], zk * qsk[h]);
            }
        }
        // scaled units (per-token formats) or plain q . k (KIVI) to base-2 logits
        const float kCx = KF == kKKivi ? a.scale_log2 : kC;
        float xs[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float xh;
            if constexpr (KF == kKKivi) {
                xh = r == 0 ? y[p][0] : (r == 1 ? y[p][1] : (r == 2 ? y[p][2] : y[p][3]));   // head r
            } else {
                // sum the quarters: rows r and r ^ 2 first (keeping heads r & 1
                // and (r & 1) + 2 of this row pair), then r and r ^ 1 (keeping head r)
                const float z0 = swap32_sum(y[p][0], y[p][2]);
                const float z1 = swap32_sum(y[p][1], y[p][3]);
                xh = swap16_sum(z0, z1);
            }
            const float xl = xh * kCx;
            if constexpr (kTail) xs[p] = (tb + n + 16 * p < t_hi) ? xl : -INFINITY;
            else xs[p] = xl;
        }

        // -------------------------------------------- online softmax (rescale on a new max)
        const bool grow = (xs[0] > m_lane) || (xs[1] > m_lane);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            float mt = fmaxf(xs[0], xs[1]);
            mt = row16_max(mt);
            const float m_new = fmaxf(m_lane, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_lane - m_new);
            m_lane = m_new;
            l_lane *= alpha;
#pragma unroll
            for (int g = 0; g < NVG; ++g) corr[g] *= alpha;
#pragma unroll
            for (int h = 0; h < kGQ; ++h) {
                // row h owns head h
                const float ah =
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 16 * h));
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k][h] *= ah;
            }
        }
        // -------------------------------------------- weight scale (rescale on a new largest V scale)
        // the lanes of a row hold the V scales of all the tile's tokens
        float sl = 0.0f;
#pragma unroll
        for (int g = 0; g < NVG; ++g) sl = fmaxf(sl, fmaxf(f16lo(L.vm[0][g]), f16lo(L.vm[1][g])));
        if (__builtin_amdgcn_ballot_w64(sl > vsmax) != 0) {
            sl = row16_max(sl);
            vsmax = fmaxf(vsmax, sl);
            int e;
            frexpf(vsmax, &e);                        // vsmax in [2^(e-1), 2^e)
            const float f = ldexpf(1.0f, 14 - e - wexp);
            wexp = 14 - e;
            wmul = ldexpf(1.0f, wexp);
#pragma unroll
            for (int g = 0; g < NVG; ++g) corr[g] *= f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] *= f;
        }
        // v_exp_f32: weights below 2^-126 of the running max may flush to zero
        const float p0 = __builtin_amdgcn_exp2f(xs[0] - m_lane);
        const float p1 = __builtin_amdgcn_exp2f(xs[1] - m_lane);
        l_lane += p0 + p1;
        const float pw0 = p0 * wmul, pw1 = p1 * wmul;   // exact: a power of two
#pragma unroll
        for (int g = 0; g < NVG; ++g) {
            const uint32_t m0 = L.vm[0][g], m1 = L.vm[1][g];
            const uint32_t pair = pack_f16(__builtin_fmaf(f16lo(m0), pw0, 0.0f), __builtin_fmaf(f16lo(m1), pw1, 0.0f));
            float cg = corr[g];
            cg = fmaf(pw0, fmaf(kVCenter, f16lo(m0), f16hi(m0)), cg);
            cg = fmaf(pw1, fmaf(kVCenter, f16lo(m1), f16hi(m1)), cg);
            corr[g] = dot2_f16(pair, kVCenterNeg /* (-8, -8) */, cg);
            wbuf[wave][g][r][n] = pair;
        }
        wave_lds_sync();

        // -------------------------------------------- values
        uint32_t vw[4][2][VH];
        if constexpr (VB == 8) {
            // stage the tile's codes (unit u: token u / 8, words 4 (u % 8) ..) and
            // read words n and n + 16 of tokens 4r + j and 4r + j + 16
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = lane + 64 * q;
                *reinterpret_cast<u32x4*>(&vst[wave][u >> 3][4 * (u & 7)]) = L.vraw[q];
            }
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int hb = 0; hb < VH; ++hb) vw[j][e][hb] = vst[wave][4 * r + j + 16 * e][n + 16 * hb];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int hb = 0; hb < VH; ++hb) vw[j][e][hb] = L.v[j][e][hb];
        }
        // A: row n = (group n >> 2, head n & 3), tokens (4r + j, 4r + j + 16) for j < 4
        u32x4 aw = u32x4{0u, 0u, 0u, 0u};
        if ((n >> 2) < NVG) aw = *reinterpret_cast<const u32x4*>(&wbuf[wave][n >> 2][n & 3][4 * r]);
#pragma unroll
        for (int hb = 0; hb < VH; ++hb)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                u32x4 bw, bl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // byte k of the word for tokens 4r + j and 4r + j + 16
                    const uint32_t P =
                        __builtin_amdgcn_perm(vw[j][1][hb], vw[j][0][hb], 0x0C040C00u + 0x00010001u * k);
                    bw[j] = P;
                    bl[j] = P & 0x000F000Fu;
                }
                if constexpr (VB == 4) {
                    acc[k] = mfma16(aw, bw, acc[k]);
                    acc[4 + k] = mfma16(aw, bl, acc[4 + k]);
                } else {
                    acc[4 * hb + k] = mfma16(aw, bw, acc[4 * hb + k]);
                }
            }
        wave_lds_sync();
    };

    // this wave's tiles wave, wave + NW, ...; two load buffers in ping-pong:
    // the next tile's loads are in flight while the current tile is computed
    // (a prefetch past the split reads zeros and is never used); only the
    // split's last tile can be partial
    MTile<NVG, VH> A, B2;
    const int n_full = (t_hi - t_lo) / kTileT;
    const int n_mine = n_tiles > wave ? (n_tiles - wave + NW - 1) / NW : 0;
    const int n_mine_full = n_full > wave ? (n_full - wave + NW - 1) / NW : 0;
    auto tl = [&](int i) { return wave + NW * i; };
    int i = 0;
    if (n_mine > 0) load_tile(tl(0), A);
    for (; i + 1 < n_mine_full; i += 2) {
        load_tile(tl(i + 1), B2);
        process(A, tl(i), Flag<false>{});
        load_tile(tl(i + 2), A);
        process(B2, tl(i + 1), Flag<false>{});
    }
    if (i < n_mine_full) {
        process(A, tl(i), Flag<false>{});
        ++i;
        if (i < n_mine) load_tile(tl(i), A);
    }
    if (i < n_mine) process(A, tl(i), Flag<true>{});

    // ---------------------------------------------------- wave-level reduction
    // head r sums over the row's tokens
    l_lane = row16_sum(l_lane);
#pragma unroll
    for (int g = 0; g < NVG; ++g) corr[g] = row16_sum(corr[g]);
    // undo the code scale 2^-24 and the weight scale 2^wexp (exact)
    const float unit = ldexpf(1.0f, 24 - wexp), unit16 = ldexpf(1.0f, 20 - wexp), unitc = ldexpf(1.0f, -wexp);
#pragma unroll
    for (int h = 0; h < kGQ; ++h) {
        // correction of head h (row h) for V group r
        float cv = 0.0f;
#pragma unroll
        for (int g = 0; g < NVG; ++g) {
            const float cg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, corr[g]), 16 * h));
            cv = (g == r) ? cg : cv;
        }
        // a column is kept in the row of its own V group
        if constexpr (VB == 4) {
            if (r == (8 * n) / GV) {      // channels 8n .. 8n+7
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float whole = acc[k][h], lo = acc[4 + k][h];
                    comb_o[wave][h][8 * n + 2 * k] = fmaf(lo, unit, cv * unitc);
                    comb_o[wave][h][8 * n + 2 * k + 1] = fmaf(whole - lo, unit16, cv * unitc);   // / 16
                }
            }
        } else {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int c0 = 4 * (n + 16 * hb);     // channels c0 .. c0 + 3
                if (r == c0 / GV) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) comb_o[wave][h][c0 + k] = fmaf(acc[4 * hb + k][h], unit, cv * unitc);
                }
            }
        }
    }
    if (n == 0) {
        comb_ml[wave][r][0] = m_lane;
        comb_ml[wave][r][1] = l_lane;
    }
    __syncthreads();
    // ---------------------------------------------------- merge the waves
    const int ns = a.n_splits;
    for (int idx = threadIdx.x; idx < kGQ * kD; idx += NW * 64) {
        const int h = idx / kD, d = idx % kD;
        if (h >= gq) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, comb_ml[w][h][0]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
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

template <int QDT, int KF, int GK, int VB, int NW>
hipError_t launch_mfma_v(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.n_splits, (unsigned)a.Hkv, (unsigned)a.B);
    const dim3 block(NW * 64);
    switch (a.v_group) {
        case 32: hipLaunchKernelGGL((decode_mfma_kernel<QDT, KF, GK, VB, 32, NW>), grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL((decode_mfma_kernel<QDT, KF, GK, VB, 64, NW>), grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((decode_mfma_kernel<QDT, KF, GK, VB, 128, NW>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int QDT, int KF, int GK>
hipError_t launch_mfma_k(const DecodeArgs& a, hipStream_t s) {
    if (a.v_bits == 8) return launch_mfma_v<QDT, KF, GK, 8, 4>(a, s);
    // KIVI keys in short splits (at most 8 tiles: one per wave of 8): the
    // latency-bound small-batch case
    if constexpr (KF == kKKivi)
        if (a.split_len <= 8 * kTileT) return launch_mfma_v<QDT, KF, GK, 4, 8>(a, s);
    return launch_mfma_v<QDT, KF, GK, 4, 4>(a, s);
}

template <int QDT>
hipError_t launch_mfma_q(const DecodeArgs& a, hipStream_t s) {
    if (a.k_kind == KVQ_TOK_SYM4) return launch_mfma_k<QDT, kKSym4, 32>(a, s);
    if (a.k_kind == KVQ_KIVI_CH) return launch_mfma_k<QDT, kKKivi, 32>(a, s);
    switch (a.k_group) {
        case 32: return launch_mfma_k<QDT, kKAff4, 32>(a, s);
        case 64: return launch_mfma_k<QDT, kKAff4, 64>(a, s);
        case 128: return launch_mfma_k<QDT, kKAff4, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Applies to 4-bit K -- per-token affine groups, symmetric blocks, or KIVI
// per-channel groups -- with affine 4- or 8-bit V at head_dim 128, 1 to 4
// query heads per kv-head, bf16 or fp16 queries and no RoPE on read (a
// per-key rotation would undo the factored scales).
bool decode_mfma_applies(const DecodeArgs& a) {
    const bool k_ok = (a.k_kind == KVQ_TOK_AFFINE && a.k_bits == 4) || a.k_kind == KVQ_TOK_SYM4 ||
                      (a.k_kind == KVQ_KIVI_CH && a.k_bits == 4);
    const bool v_ok = a.v_kind == KVQ_TOK_AFFINE && (a.v_bits == 4 || a.v_bits == 8);
    const bool heads_ok = a.Hq % a.Hkv == 0 && a.Hq >= a.Hkv && a.Hq <= kGQ * a.Hkv;
    return k_ok && v_ok && heads_ok && a.D == kD && (a.q_dtype == KVQ_BF16 || a.q_dtype == KVQ_F16) && !a.rope;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
    if (a.q_dtype == KVQ_BF16) return launch_mfma_q<KVQ_BF16>(a, s);
    return launch_mfma_q<KVQ_F16>(a, s);
}

// The fast path is the matrix-core decode.
bool decode_fast_applies(const DecodeArgs& a) { return decode_mfma_applies(a); }

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s) { return launch_decode_mfma(a, s); }

// Split plan: one workgroup per (batch, kv-head) when that fills the chip
// twice over, otherwise split the tokens so that about 512 workgroups run,
// with at least 2 tiles per wave, so that each wave's second tile loads
// while its first is computed (the best latency for small batches).  With
// 8-bit values and at least 64 (batch, kv-head) units the target is 256:
// a wave's tile then carries about half again as many bytes, and longer
// splits stream better (Q4_0 keys with 8-bit values, B=16, T=16384: 2
// splits 68.8 us, 4 splits 70.1 us, 8 splits 71.3 us).
void decode_fast_plan(int B, int Hkv, int T, int v_bits, int* n_splits, int* split_len) {
    const int units = B * Hkv;
    const int target = (v_bits == 8 && units >= 64) ? 256 : 512;
    int ns = (target + units - 1) / units;
    const int min_len = kWaves * kTileT * 2;
    const int max_ns = (T + min_len - 1) / min_len;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    int len = (T + ns - 1) / ns;
    len = ((len + kTileT - 1) / kTileT) * kTileT;
    *split_len = len;
    *n_splits = (T + len - 1) / len;
}

}  // namespace kvq

// prefill_attn.hip -- multi-query attention over the packed cache (gfx950).
//
// A prefill chunk of n_q queries per head attends to the compressed cache
// ("Low-bit KV caches on MLX", s.5: the multi-query microbenchmark shape of
// 128 queries with GQA 4:1 over 2K-64K cached tokens, where attention is a
// dense contraction).  Per (batch, kv-head) the G * n_q query rows of the
// head group share every key and value, so the work is two products per
// 64-token tile on the matrix cores:
//
//   S^T = K Q^T      (64 tokens x 32 query rows per wave, K-dim = head_dim)
//   O^T += V^T P^T   (head_dim x 32 query rows per wave, K-dim = 64 tokens)
//
// with v_mfma_f32_32x32x16_f16.  The workgroup unpacks each tile once into LDS
// for all its waves, into one of two buffers, so the next tile is unpacked
// while the current one is computed.  4-bit per-token affine keys in groups
// of 64 or 128 channels (with fp16 or bf16 queries) enter the score product
// as their codes, and the group scales and zero points are applied to the
// sums (the factored scores below); other keys are held as an fp16 pair
// (x_hi + x_lo, x_lo the rounding residual), with the fp16 or bf16 query row
// scaled by a power of two into fp16 exactly, so the scores take
// K_hi Q + K_lo Q (an fp32 query is a pair as well: K_hi Q_hi + K_lo Q_hi +
// K_hi Q_lo).  Either way the logits are fp32-accurate even where large keys
// (outlier channels) would make a single fp16 rounding move the softmax;
// values and probabilities enter the second product as single fp16 (their
// rounding stays relative to the output).  The online softmax runs in fp32 on
// the score accumulators, where each lane holds one query column.  Tokens
// are handed to the second product in the order the score accumulators hold
// them, and the value tile is stored in that order, so probabilities go from
// registers to the matrix cores without a shuffle.  Splits over the tokens
// write partials (m, l, o / l in fp16) that a log-sum-exp combine merges.
#include <math.h>

#include "bufload.h"
#include "dequant8.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kPT = 64;          // tokens per tile
constexpr int kXcds = 8;         // XCDs (L2 domains) of the device
constexpr int kWaves = 8;        // waves per workgroup, 32 query rows each
constexpr int kRows = 32 * kWaves;
// Waves per workgroup of the factored-score kernel.  Four waves (two
// workgroups of 128 rows per CU, with separate barriers) measured slower than
// eight: each workgroup then unpacks every tile for half the rows.
constexpr int kFactWaves = 8;
constexpr int kPad = 8;          // halfs of padding per LDS row (bank spread)
constexpr float kSlack = 8.0f;   // log2 headroom of the lazily moved softmax reference point
constexpr float kSlackP = 256.0f; // 2^kSlack

// Row of the 32x32 block held by accumulator element v of lane half kh.
__device__ __forceinline__ int acc_row(int v, int kh) { return 8 * (v >> 2) + 4 * kh + (v & 3); }

// Column of token t (0..63) in the transposed value tile.  For K-step s of
// the second product, lane half kh supplies the probabilities of tokens
// 16s + 8(j >> 2) + 4kh + (j & 3), j < 8 (the score accumulator layout);
// storing that token at column 16s + 8kh + j lines the value rows up with them.
__device__ __forceinline__ int v_col(int t) {
    const int s = t >> 4, r = t & 15;
    return 16 * s + 8 * ((r & 7) >> 2) + 4 * (r >> 3) + (r & 3);
}

// Physical column of (row, col) in the value tile: the 16-byte chunk index
// (col bits 3..5) is XORed with (row >> 4) & 7, so the rows 8c + j that one
// store instruction writes (c = 0..15) spread over the banks, while the
// 16-byte operand reads of a row stay contiguous.
__device__ __forceinline__ int vswz(int row, int col) { return col ^ (((row >> 4) & 7) << 3); }

__device__ __forceinline__ int wave_min(int v) { return lane_reduce<true>(v, [](int x, int y) { return min(x, y); }); }

__device__ __forceinline__ half8 to_half8(const float x[8]) {
    half8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)x[j];
    return h;
}
// fp16 pair with x = hi + lo to about 2^-22 relative
__device__ __forceinline__ void split_half8(const float x[8], half8& hi, half8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        hi[j] = (_Float16)x[j];
        lo[j] = (_Float16)(x[j] - (float)hi[j]);
    }
}

// The eight 4-bit codes of a code word as floats: even channels are the bytes
// of w & 0x0F0F0F0F, odd channels those of (w >> 4) & 0x0F0F0F0F (one
// byte-to-float conversion each).
__device__ __forceinline__ void nib8(uint32_t w, float u[8]) {
    const uint32_t e = w & 0x0F0F0F0Fu, o = (w >> 4) & 0x0F0F0F0Fu;
    u[0] = (float)(e & 0xFFu);
    u[1] = (float)(o & 0xFFu);
    u[2] = (float)((e >> 8) & 0xFFu);
    u[3] = (float)((o >> 8) & 0xFFu);
    u[4] = (float)((e >> 16) & 0xFFu);
    u[5] = (float)((o >> 16) & 0xFFu);
    u[6] = (float)(e >> 24);
    u[7] = (float)(o >> 24);
}

using buf::rsrc;
// Loads of `bytes` (2, 4 or 8) bytes at a buffer offset; past the buffer's end they read zero.
__device__ __forceinline__ void bload_codes(__amdgpu_buffer_rsrc_t r, uint32_t off, int bytes, dq::Pre8& p) {
    if (bytes == 2) {
        p.c0 = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    } else if (bytes == 4) {
        p.c0 = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
        p.c0 = w.x; p.c1 = w.y;
    }
}

// Block (split, hk * n_rb + rb, b): query rows [rb * kRows, +kRows) of kv-head
// hk's group (row r = h * n_q + i: query head hk * G + h, query i), tokens of
// the split.  Causal rows see slots t <= T - n_q + i.
//
// QX: the query is fp16 or bf16.  Each row is then scaled by a power of two
// so that its largest element lies in [2^14, 2^15): every element down to
// 2^-28 of the largest is exact in fp16 (smaller ones, far below the fp32
// rounding of the dot product, may lose low bits), the scores need only
// K_hi Q + K_lo Q, and the row's factor (softmax scale times the power of
// two) is applied to the fp32 scores.  Otherwise (fp32 queries) the query is
// an fp16 pair as the keys are.
//
// C4: per-token 4-bit keys and values.  The code widths are then constants,
// so each tile's fetch is one straight run of loads whose results are first
// used one tile later (with widths known only at run time, the branches
// around the loads cost a wait on each of them).
//
// FG > 0: factored scores for 4-bit per-token affine keys with FG groups per
// row (group 64 or 128 at head_dim 128).  A key is u s_g + z_g, so
//   q.k = sum_g s_g (q_g . u_g) + sum_g z_g Q_g,    Q_g = sum of q over group g.
// The key tile holds the codes themselves as MFMA operands: a code left in
// place under a nibble mask is the fp16 subnormal u 2^-24 (low nibble) or
// u 2^-20 (high nibble), and the query operand carries the matching channel
// order and a 1/16 on the high-nibble channels, so every product is exact and
// only the fp32 accumulation rounds.  One accumulator per group takes the
// q_g . u_g sums; the zero-point term is one bf16 product per 32-token block
// (z as an exact bf16 pair, Q_g 2^-24 as an exact bf16 triple); the lane then
// scales each group's sum by its token's s_g.  There is no key residual and
// no second key product.
template <int KK, int VK, int D, bool QX, bool C4, int FG>
__global__ __launch_bounds__((FG > 0 ? kFactWaves : kWaves) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_attn_kernel(DecodeArgs a, int n_q, int n_rb, int causal) {
    static_assert(!C4 || ((KK == KVQ_TOK_AFFINE || KK == KVQ_TOK_SYM4) && VK == KVQ_TOK_AFFINE),
                  "constant code widths: per-token layouts");
    static_assert(FG == 0 || (C4 && QX && KK == KVQ_TOK_AFFINE && D == 128 && FG <= 2),
                  "factored scores: 4-bit affine keys at head_dim 128, fp16/bf16 queries, 1 or 2 groups per row");
    constexpr bool kFact = FG > 0;
    constexpr int NW = kFact ? kFactWaves : kWaves;      // waves per workgroup
    constexpr int NT = NW * 64;
    constexpr int RW = 32 * NW;                          // query rows per workgroup
    if constexpr (C4) {
        a.k_bits = 4;
        a.v_bits = 4;
    }
    constexpr int NK = D / 16;               // K-steps of the score product
    constexpr int ND = D / 32;               // 32-row blocks of the output
    constexpr int C8 = D / 8;                // 8-channel chunks per row
    // Workgroup x runs on XCD x % 8.  Work item p = (x % 8) * per_xcd + x / 8
    // (split fastest, then row block, kv-head, batch) puts the splits of a row
    // block, and the row blocks of a kv-head, on one XCD, where they share its
    // L2 copy of the query rows and of the cache tiles; the grid is padded to
    // a multiple of 8 and the padding exits.
    const int per_xcd = (int)(gridDim.x / kXcds);
    const int p = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    const int n_units = a.Hkv * n_rb;
    if (p >= a.n_splits * n_units * a.B) return;
    const int split = p % a.n_splits;
    const int unit = p / a.n_splits;
    const int b = unit / n_units;
    const int hk = (unit - b * n_units) / n_rb, rb = unit - b * n_units - hk * n_rb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int kh = lane >> 5, l32 = lane & 31;
    const int G = a.Hq / a.Hkv;
    const int R = G * n_q;
    const int64_t bh = (int64_t)b * a.Hkv + hk;
    const int T = a.T;

    // LDS: two tile buffers, each keys (fp16 high part and rounding residual,
    // token-major) and the transposed value tile; after the last tile the
    // same space holds each wave's output block for a row-major write-out
    constexpr int kKeyHalfs = kPT * (D + kPad);
    // factored: group scales [kPT] u32 and zero-point operands [kPT][2] uint4
    // in place of the key residual
    constexpr int kResHalfs = kFact ? 2 * kPT + kPT * 2 * 8 : kKeyHalfs;
    constexpr int kTileHalfs = kKeyHalfs + kResHalfs + D * (kPT + kPad);
    constexpr int kOutHalfs = NW * 32 * 33 * 2;              // [wave][32 rows][32 dims + pad] fp32
    __shared__ __align__(16) _Float16 lds[2 * kTileHalfs > kOutHalfs ? 2 * kTileHalfs : kOutHalfs];
    auto k_lds = [&](int buf) { return reinterpret_cast<_Float16 (*)[D + kPad]>(lds + buf * kTileHalfs); };
    auto kl_lds = [&](int buf) {
        return reinterpret_cast<_Float16 (*)[D + kPad]>(lds + buf * kTileHalfs + kKeyHalfs);
    };
    auto v_lds = [&](int buf) {
        return reinterpret_cast<_Float16 (*)[kPT + kPad]>(lds + buf * kTileHalfs + kKeyHalfs + kResHalfs);
    };
    // factored scores: the residual's space holds each token's group scales
    // (fp16 s_0 | s_1 << 16) and its zero-point operands ([token][group] 8 bf16)
    auto sc_lds = [&](int buf) { return reinterpret_cast<uint32_t*>(lds + buf * kTileHalfs + kKeyHalfs); };
    auto zo_lds = [&](int buf) {
        return reinterpret_cast<uint4 (*)[2]>(lds + buf * kTileHalfs + kKeyHalfs + 2 * kPT);
    };

    // this lane's query row: fragments for every K-step
    const int r = rb * RW + wave * 32 + l32;
    const bool row_ok = r < R;
    const int h = row_ok ? r / n_q : 0, i = row_ok ? r - (r / n_q) * n_q : 0;
    const int64_t grow = ((int64_t)b * a.Hq + hk * G + h) * n_q + i;     // global query row
    // the query operands, prepared while the first tile's codes are in flight
    half8 qf[NK], qfl[NK];
    uint4 zq = make_uint4(0u, 0u, 0u, 0u);   // factored: B operand of the zero-point product
    float qc = 1.0f;                         // factor from score accumulators to base-2 logits
    auto prepare_query = [&]() {
        if constexpr (QX) {
            // All of the row's loads first (16 bytes each, whatever the
            // type; a row past the group reads row 0 and is zeroed).  For
            // finite fp16 and bf16 values |x| grows with the integer bits & 0x7FFF,
            // so the row's largest magnitude is found on the bits.
            uint4 raw[NK];
            const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (row_ok ? grow : 0) * D + kh * 8;
#pragma unroll
            for (int q = 0; q < NK; ++q) raw[q] = *reinterpret_cast<const uint4*>(qrow + q * 16);
            uint32_t mbits = 0;
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                if (!row_ok) raw[q] = make_uint4(0u, 0u, 0u, 0u);
                const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) mbits = max(mbits, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
            }
            const bool f16in = a.q_dtype == KVQ_F16;
            // both conversions, then a select: no branch per element
            auto elem = [&](uint32_t b16) {
                const float h = f16_bits_to_f32(b16), bf = bf16_bits_to_f32(b16);
                return f16in ? h : bf;
            };
            float amax = elem(mbits);
            amax = fmaxf(amax, lane_xor<32>(amax));
            int ex = 0;
            if (amax > 0.0f) frexpf(amax, &ex);                  // amax in [2^(ex-1), 2^ex)
            const float up = ldexpf(1.0f, 15 - ex);              // largest |q| -> [2^14, 2^15)
            qc = ldexpf(a.scale_log2, kFact ? ex + 9 : ex - 15); // factored sums carry 2^-24
            float qsum[2] = {0.0f, 0.0f};        // factored: this lane's half of each group's query sum
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[2 * j] = elem(w[j] & 0xFFFFu) * up;
                    x[2 * j + 1] = elem(w[j] >> 16) * up;
                }
                if constexpr (kFact) {
                    // operand element e holds channel {0,4,1,5,2,6,3,7}[e] of the
                    // chunk; high-nibble channels (odd) arrive 16x larger
                    constexpr int ch[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
                    for (int e = 0; e < 8; ++e) qf[q][e] = (_Float16)((ch[e] & 1) ? x[ch[e]] * 0.0625f : x[ch[e]]);
                    // K-step q covers channels 16q .. 16q + 15, all in group q / (NK / FG)
#pragma unroll
                    for (int e = 0; e < 8; ++e) qsum[FG == 2 && q >= NK / 2 ? 1 : 0] += x[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) qf[q][e] = (_Float16)x[e];
                }
            }
            if constexpr (kFact) {
                // Lane half kh supplies group kh's term (FG = 2), or the low
                // half the whole row's (FG = 1); the partner lane holds the
                // other half of every group's channels.
                const float send = FG == 2 ? qsum[1 - kh] : qsum[0];
                const float other = lane_xor<32>(send);
                const float Q = (FG == 2 ? qsum[kh] : qsum[0]) + other;
                // Q 2^-24 as an exact bf16 triple (truncating splits)
                const float Qs = Q * 0x1p-24f;
                const uint32_t hb = __float_as_uint(Qs) & 0xFFFF0000u;
                const float r1 = Qs - __uint_as_float(hb);
                const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
                const float r2 = r1 - __uint_as_float(mb);
                const uint32_t h = hb >> 16, mdl = mb >> 16, lw = __float_as_uint(r2) >> 16;
                const bool live = FG == 2 || kh == 0;
                zq = live ? make_uint4(h | (mdl << 16), lw | (h << 16), mdl | (lw << 16), 0u) : make_uint4(0u, 0u, 0u, 0u);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                float x[8] = {};
                if (row_ok) dq::load8(a.q, grow * D + q * 16 + kh * 8, a.q_dtype, x);
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] *= a.scale_log2;
                split_half8(x, qf[q], qfl[q]);
            }
        }
    };
    const int lim = causal ? T - n_q + i : T - 1;   // last visible slot
    const int t_lo = split * a.split_len;
    const int t_hi = min(T, t_lo + a.split_len);
    float m = -INFINITY, l = 0.0f;
    floatx16 o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = floatx16{};

    // Each thread owns kItems (token, 8-channel chunk) items of a tile.  Tile
    // t + 1 is unpacked into the other LDS buffer while tile t is computed,
    // and the codes and metadata of tile t + 2 are fetched into registers
    // behind it: one barrier per tile.
    constexpr int kItems = (kPT * C8 + NT - 1) / NT;
    dq::Pre8 pk[kItems], pv[kItems];
    // Per-token layouts put every item of a tile at a fixed byte offset from
    // the tile's first slot: each tile only rebuilds buffer resources (scalar
    // work) sized to its valid rows.
    constexpr bool kTokK = KK == KVQ_TOK_AFFINE || KK == KVQ_TOK_SYM4;
    constexpr bool kTokV = VK == KVQ_TOK_AFFINE;
    // 4-bit affine keys and values at head_dim 128: items 2p and 2p + 1 of a
    // thread are tokens 2u and 2u + 1 of one 8-channel chunk, whose transposed
    // values sit in adjacent columns (one 32-bit LDS store per channel)
    constexpr bool kPair = C4 && KK == KVQ_TOK_AFFINE && D == 128 && kItems % 2 == 0 && kPT * C8 == kItems * NT;
    auto item_tc = [&](int j, int& t, int& c) {
        if constexpr (kPair) {
            c = tid % C8;
            t = 2 * (tid / C8 + (j >> 1) * (NT / C8)) + (j & 1);
        } else {
            const int it = tid + j * NT;
            t = it / C8;
            c = it - t * C8;
        }
    };
    const int kb = KK == KVQ_TOK_SYM4 ? 4 : a.k_bits;                 // code bytes per 8 channels
    const int k_row_b = D * kb / 8;
    const int k_meta_b = KK == KVQ_TOK_SYM4 ? (D / 32) * 2 : (kTokK ? (D / a.k_group) * 4 : 0);
    const int v_row_b = D * a.v_bits / 8;
    const int v_meta_b = kTokV ? (D / a.v_group) * 4 : 0;
    auto fetch = [&](int tb, dq::Pre8 (&pkd)[kItems], dq::Pre8 (&pvd)[kItems]) {
        // rows of the tile inside the split (0 past its end: every load then reads zero)
        const uint32_t nt = (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(kPT, t_hi - tb)));
        const int64_t slot0 = bh * a.cap + tb;
        if constexpr (kTokK) {
            const __amdgpu_buffer_rsrc_t rk = rsrc(static_cast<const uint8_t*>(a.k_codes) + slot0 * k_row_b, nt * k_row_b);
            const __amdgpu_buffer_rsrc_t rm = rsrc(static_cast<const uint8_t*>(a.k_meta) + slot0 * k_meta_b, nt * k_meta_b);
#pragma unroll
            for (int j = 0; j < kItems; ++j) {
                if (!kPair && tid + j * NT >= kPT * C8) break;
                int t, c;
                item_tc(j, t, c);
                bload_codes(rk, (uint32_t)(t * k_row_b + c * kb), kb, pkd[j]);
                pkd[j].meta = KK == KVQ_TOK_SYM4
                                 ? __builtin_amdgcn_raw_buffer_load_b16(rm, (t * (D / 32) + (8 * c) / 32) * 2, 0, 0)
                                 : __builtin_amdgcn_raw_buffer_load_b32(rm, (t * (D / a.k_group) + (8 * c) / a.k_group) * 4, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kItems; ++j) {
                const int it = tid + j * NT;
                const int t = it / C8, c = it - t * C8;
                if (it < kPT * C8 && tb + t < t_hi) dq::k_fetch8<KK>(a, bh, tb + t, c, pkd[j]);
            }
        }
        if constexpr (kTokV) {
            const __amdgpu_buffer_rsrc_t rv = rsrc(static_cast<const uint8_t*>(a.v_codes) + slot0 * v_row_b, nt * v_row_b);
            const __amdgpu_buffer_rsrc_t rm = rsrc(static_cast<const uint8_t*>(a.v_meta) + slot0 * v_meta_b, nt * v_meta_b);
#pragma unroll
            for (int j = 0; j < kItems; ++j) {
                if (!kPair && tid + j * NT >= kPT * C8) break;
                int t, c;
                item_tc(j, t, c);
                bload_codes(rv, (uint32_t)(t * v_row_b + c * a.v_bits), a.v_bits, pvd[j]);
                pvd[j].meta = __builtin_amdgcn_raw_buffer_load_b32(rm, (t * (D / a.v_group) + (8 * c) / a.v_group) * 4, 0, 0);
            }
        }
    };
    // unpack the fetched tile at tb into buffer buf; rows past the split are zero
    auto unpack = [&](int tb, int buf, const dq::Pre8 (&pks)[kItems], const dq::Pre8 (&pvs)[kItems]) {
        const int nt = min(kPT, t_hi - tb);
        _Float16 (*kd)[D + kPad] = k_lds(buf);
        _Float16 (*kld)[D + kPad] = kl_lds(buf);
        _Float16 (*vd)[kPT + kPad] = v_lds(buf);
        if constexpr (kPair) {
            // rows past the split were fetched as zero codes and metadata: zero keys and values
#pragma unroll
            for (int pp = 0; pp < kItems / 2; ++pp) {    // item pairs (2pp, 2pp + 1)
                const int c = tid % C8, t0 = 2 * (tid / C8 + pp * (NT / C8));
#pragma unroll
                for (int jj2 = 0; jj2 < 2; ++jj2) {
                    const int j = 2 * pp + jj2;
                    if constexpr (kFact) {
                        // the code word under nibble masks: channels (0,4), (1,5)*16,
                        // (2,6), (3,7)*16 as fp16 subnormal pairs
                        const uint32_t w = pks[j].c0, w8 = w >> 8;
                        *reinterpret_cast<uint4*>(&kd[t0 + jj2][8 * c]) =
                            make_uint4(w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u);
                        constexpr int kCg = 128 / FG / 8;    // 8-channel chunks per group
                        if (c % kCg == 0) {
                            // first chunk of group g: the token's s_g, and z_g as an
                            // exact bf16 pair (zh keeps the top 8 significant bits)
                            const int g = c / kCg;
                            reinterpret_cast<uint16_t*>(sc_lds(buf))[2 * (t0 + jj2) + g] = (uint16_t)(pks[j].meta & 0xFFFFu);
                            const float z = f16_bits_to_f32(pks[j].meta >> 16);
                            const uint32_t zhb = __float_as_uint(z) & 0xFFFF0000u;
                            const uint32_t zh = zhb >> 16, zl = __float_as_uint(z - __uint_as_float(zhb)) >> 16;
                            zo_lds(buf)[t0 + jj2][g] = make_uint4(zh | (zh << 16), zh | (zl << 16), zl | (zl << 16), 0u);
                            if (FG == 1) zo_lds(buf)[t0 + jj2][1] = make_uint4(0u, 0u, 0u, 0u);
                        }
                    } else {
                        float u[8];
                        nib8(pks[j].c0, u);
                        const float sk = f16_bits_to_f32(pks[j].meta & 0xFFFFu), zk = f16_bits_to_f32(pks[j].meta >> 16);
                        half8 kh8, kl8;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const float x = fmaf(u[i], sk, zk);
                            kh8[i] = (_Float16)x;
                            kl8[i] = (_Float16)(x - (float)kh8[i]);
                        }
                        *reinterpret_cast<half8*>(&kd[t0 + jj2][8 * c]) = kh8;
                        *reinterpret_cast<half8*>(&kld[t0 + jj2][8 * c]) = kl8;
                    }
                }
                // Values as (token t0, token t0 + 1) fp16 pairs, straight from the
                // code bytes: byte i of both code words gives channels 2i (low
                // nibbles) and 2i + 1 (high nibbles); 0x6400 | u is the fp16
                // 1024 + u, so subtracting 1024 leaves u exactly, and one packed
                // fp16 fma rounds u s + z once.
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                const uint32_t w0 = pvs[2 * pp].c0, w1 = pvs[2 * pp + 1].c0;
                const uint32_t m0 = pvs[2 * pp].meta, m1 = pvs[2 * pp + 1].meta;
                const h2 s2 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(m1, m0, 0x05040100u));
                const h2 z2 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(m1, m0, 0x07060302u));
                const h2 m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
                // rows 8c .. 8c + 7 share (row >> 4) & 7 = (c >> 1) & 7: one swizzled
                // column for all eight stores (token t0 + 1 is the next column)
                _Float16* vrow = &vd[8 * c][vswz(8 * c, v_col(t0))];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x = __builtin_amdgcn_perm(w1, w0, (uint32_t)i | 0x0C000C00u | ((uint32_t)(4 + i) << 16));
                    const uint32_t e = (x & 0x000F000Fu) | 0x64006400u, od = ((x >> 4) & 0x000F000Fu) | 0x64006400u;
                    const h2 ve = __builtin_elementwise_fma(__builtin_bit_cast(h2, e) + m1024, s2, z2);
                    const h2 vo = __builtin_elementwise_fma(__builtin_bit_cast(h2, od) + m1024, s2, z2);
                    *reinterpret_cast<h2*>(vrow + (2 * i) * (kPT + kPad)) = ve;
                    *reinterpret_cast<h2*>(vrow + (2 * i + 1) * (kPT + kPad)) = vo;
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const int it = tid + j * NT;
            if (it >= kPT * C8) break;
            const int t = it / C8, c = it - t * C8;
            float xk[8] = {}, xv[8] = {};
            if (kTokK && kTokV) {
                // rows past the split were fetched as zero codes and zero
                // metadata, which dequantize to zero: no branch
                dq::k_finish8<KK>(a, bh, tb + t, c, pks[j], xk);
                dq::v_finish8<VK>(a, bh, tb + t, c, pvs[j], xv);
            } else if (t < nt) {
                dq::k_finish8<KK>(a, bh, tb + t, c, pks[j], xk);
                dq::v_finish8<VK>(a, bh, tb + t, c, pvs[j], xv);
            }
            half8 kh8, kl8;
            split_half8(xk, kh8, kl8);
            *reinterpret_cast<half8*>(&kd[t][8 * c]) = kh8;
            *reinterpret_cast<half8*>(&kld[t][8 * c]) = kl8;
            const int col = v_col(t);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) vd[8 * c + jj][vswz(8 * c + jj, col)] = (_Float16)xv[jj];
        }
    };
    // the first two tiles' codes are in flight while the query is prepared
    {
        dq::Pre8 pk0[kItems], pv0[kItems];
        if (t_lo < t_hi) fetch(t_lo, pk0, pv0);
        if (t_lo + kPT < t_hi) fetch(t_lo + kPT, pk, pv);
        prepare_query();
        if (t_lo < t_hi) unpack(t_lo, 0, pk0, pv0);
    }
    __syncthreads();

    const int lim_min = __builtin_amdgcn_readfirstlane(wave_min(row_ok ? lim : T - 1));
    // S^T for this wave's 32 rows over the tile in buffer bf: two 32-token blocks
    floatx16 s[2];
    auto scores = [&](int bf) {
        _Float16 (*kd)[D + kPad] = k_lds(bf);
        if constexpr (kFact) {
            const uint32_t* scl = sc_lds(bf);
            uint4 (*zo)[2] = zo_lds(bf);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const uint4 za = zo[blk * 32 + l32][kh];
                s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, za),
                                                                 __builtin_bit_cast(bf16x8, zq), floatx16{}, 0, 0, 0);
                // one group at a time: its K-steps into one accumulator, then
                // each element scaled by its token's s_g (token 8j + 4kh + i of
                // the block is accumulator element 4j + i)
#pragma unroll
                for (int g = 0; g < FG; ++g) {
                    constexpr int kQ = NK / FG;
                    floatx16 sg = floatx16{};
#pragma unroll
                    for (int q = 0; q < kQ; ++q) {
                        const half8 ka = *reinterpret_cast<const half8*>(&kd[blk * 32 + l32][(g * kQ + q) * 16 + kh * 8]);
                        sg = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[g * kQ + q], sg, 0, 0, 0);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 sv = *reinterpret_cast<const uint4*>(&scl[blk * 32 + 8 * j + 4 * kh]);
                        const uint32_t w[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            s[blk][4 * j + i] = fmaf(f16_bits_to_f32(g == 0 ? w[i] & 0xFFFFu : w[i] >> 16), sg[4 * j + i], s[blk][4 * j + i]);
                    }
                }
                // the block's logits are complete here (keeps the next block's
                // products from running ahead of this block's scaling)
                asm volatile("" : "+v"(s[blk]));
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            _Float16 (*kld)[D + kPad] = kl_lds(bf);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                s[blk] = floatx16{};
#pragma unroll
                for (int q = 0; q < NK; ++q) {
                    const half8 ka = *reinterpret_cast<const half8*>(&kd[blk * 32 + l32][q * 16 + kh * 8]);
                    const half8 kl = *reinterpret_cast<const half8*>(&kld[blk * 32 + l32][q * 16 + kh * 8]);
                    s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kl, qf[q], s[blk], 0, 0, 0);
                    if constexpr (!QX) s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qfl[q], s[blk], 0, 0, 0);
                    s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[q], s[blk], 0, 0, 0);
                }
            }
        }
    };
    // the tile after t0 goes into buffer nb (without a branch for per-token
    // layouts, so that the score products and the unpacking are one block the
    // scheduler can interleave; past the split's end the unpack writes zero
    // rows and the fetch reads zeros)
    auto next_tile = [&](int t0, int nb) {
        if constexpr (kFact) __builtin_amdgcn_sched_barrier(0);
        if constexpr (kTokK && kTokV) {
            unpack(t0 + kPT, nb, pk, pv);
            fetch(t0 + 2 * kPT, pk, pv);
        } else if (t0 + kPT < t_hi) {
            unpack(t0 + kPT, nb, pk, pv);
            if (t0 + 2 * kPT < t_hi) fetch(t0 + 2 * kPT, pk, pv);
        }
    };
    // softmax of the scores s of the tile at t0, and its values (buffer bf)
    auto finish = [&](int t0, int bf) {
        _Float16 (*vd)[kPT + kPad] = v_lds(bf);
        // P^T fragments: K-step st takes accumulator elements 8 (st & 1) .. +7
        // of block st >> 1 (v_exp_f32: results below 2^-126 flush to 0); the
        // return value is this lane's sum of the fp16 probabilities the value
        // product uses, two per instruction
        half8 pf[4];
        auto probs = [&](float mu) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pf[st][j] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[st >> 1][8 * (st & 1) + j], qc, -mu));
            typedef _Float16 half2v __attribute__((ext_vector_type(2)));
            const half2v one2 = {(_Float16)1.0f, (_Float16)1.0f};
            float sum = 0.0f;
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2v pr = {pf[st][2 * j], pf[st][2 * j + 1]};
                    sum = __builtin_amdgcn_fdot2(pr, one2, sum, false);
                }
            return sum;
        };
        // online softmax, base 2.  A row's reference point m moves only when
        // the row sees a logit more than kSlack above it (and on its first
        // visible slot); only then are its output accumulators rescaled.  The
        // probabilities are then at most 2^kSlack, well inside fp16, and the
        // split's (m, l) stay consistent with its outputs.  A tile that needs
        // no mask (every slot visible to every row of the wave) and a wave
        // whose rows all have a reference point first take the probabilities
        // against the current m: a lane sum below 2^kSlack bounds every one
        // of them, so no logit is more than kSlack above m and m stays
        // (the same decision as from the tile's maximum, which is then not
        // needed); otherwise the tile takes the general path below.
        const bool no_mask = t0 + kPT <= t_hi && t0 + kPT - 1 <= lim_min;
        bool general = !no_mask || __builtin_amdgcn_ballot_w64(m == -INFINITY) != 0;
        float ps = 0.0f;
        if (!general) {
            ps = probs(m);
            general = __builtin_amdgcn_ballot_w64(!(ps < kSlackP)) != 0;
        }
        if (general) {
            // mask (past the split or the row's last visible slot) -- only
            // tiles that reach either boundary for some row of the wave need
            // it (the row factor qc > 0 is applied to the max and inside the
            // exponent)
            float mt = -INFINITY;
            if (no_mask) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[blk][v]);
            } else {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int tok = t0 + blk * 32 + acc_row(v, kh);
                        const float x = (tok < t_hi && tok <= lim) ? s[blk][v] : -INFINITY;
                        s[blk][v] = x;
                        mt = fmaxf(mt, x);
                    }
            }
            mt = fmaxf(mt, lane_xor<32>(mt)) * qc;
            const float m_new = mt > m + kSlack ? mt : m;
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // nothing visible yet
            if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
                const float alpha = __builtin_amdgcn_exp2f(m - m_use);
                l *= alpha;
#pragma unroll
                for (int d = 0; d < ND; ++d) o[d] *= alpha;
            }
            m = m_new;
            ps = probs(m_use);
        }
        ps = swap32_sum(ps, ps);
        l += ps;
        // O^T += V^T P^T.  Row d * 32 + l32, 16-byte chunk 2 st + kh XORed with
        // (row >> 4) & 7 = 2 d + (l32 >> 4) is chunk 2 (st ^ d) + (kh ^ (l32 >> 4)):
        // a lane base plus a constant offset per (d, st).
        const _Float16* vbase = &vd[l32][8 * (kh ^ (l32 >> 4))];
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const half8 va = *reinterpret_cast<const half8*>(vbase + d * 32 * (kPT + kPad) + 16 * (st ^ (d & 3)));
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[st], o[d], 0, 0, 0);
            }
    };
    int buf = 0;
    for (int t0 = t_lo; t0 < t_hi; t0 += kPT, buf ^= 1) {
        scores(buf);
        next_tile(t0, buf ^ 1);
        finish(t0, buf);
        __syncthreads();                 // this buffer is read, the other one written
    }

    // partials of the split: o[dim] / l as fp16 and (m, l) of each row in
    // fp32 (a row that saw no slot here has l = 0 and writes zeros).  The
    // accumulators hold O^T (lane = row); each 32-dim block goes through the
    // wave's own LDS rows so that rows are written as contiguous 64-byte runs
    // (only the wave's lanes exchange data there: wave-level syncs; the
    // loop's last barrier has freed the tile buffers).
    const int ns = a.n_splits;
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    float (*tr)[33] = reinterpret_cast<float (*)[33]>(lds) + wave * 32;      // [32 rows][32 dims + pad]
    const int wr = lane >> 1, wh = lane & 1;                                // row, 16-dim half it writes
    const int r_w = rb * RW + wave * 32 + wr;
    int64_t grow_w = 0;
    if (r_w < R) {
        const int hw = r_w / n_q, iw = r_w - hw * n_q;
        grow_w = ((int64_t)b * a.Hq + hk * G + hw) * n_q + iw;
    }
    uint16_t* ws_h = reinterpret_cast<uint16_t*>(a.ws_o);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        if (d > 0) wave_lds_sync();          // the previous block's reads are done
#pragma unroll
        for (int v = 0; v < 16; ++v) tr[l32][acc_row(v, kh)] = o[d][v] * inv_l;
        wave_lds_sync();
        if (r_w < R) {
            uint32_t hw2[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                _Float16 lo = (_Float16)tr[wr][wh * 16 + 2 * k], hi = (_Float16)tr[wr][wh * 16 + 2 * k + 1];
                hw2[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
            u32x4n* dst = reinterpret_cast<u32x4n*>(ws_h + (grow_w * ns + split) * D + d * 32 + wh * 16);
            __builtin_nontemporal_store(u32x4n{hw2[0], hw2[1], hw2[2], hw2[3]}, dst);
            __builtin_nontemporal_store(u32x4n{hw2[4], hw2[5], hw2[6], hw2[7]}, dst + 1);
        }
    }
    if (row_ok && kh == 0) {
        a.ws_ml[(grow * ns + split) * 2 + 0] = m;
        a.ws_ml[(grow * ns + split) * 2 + 1] = l;
    }
}

template <int KK, int VK, bool QX, bool C4>
hipError_t launch_prefill_kvq(const DecodeArgs& a, int n_q, int n_rb, int causal, hipStream_t s) {
    const int64_t n_wg = (int64_t)a.n_splits * a.Hkv * n_rb * a.B;
    const dim3 grid((unsigned)(((n_wg + kXcds - 1) / kXcds) * kXcds));
    const dim3 blk(kWaves * 64), blk_f(kFactWaves * 64);
    switch (a.D) {
        case 32: hipLaunchKernelGGL((prefill_attn_kernel<KK, VK, 32, QX, C4, 0>), grid, blk, 0, s, a, n_q, n_rb, causal); break;
        case 64: hipLaunchKernelGGL((prefill_attn_kernel<KK, VK, 64, QX, C4, 0>), grid, blk, 0, s, a, n_q, n_rb, causal); break;
        default:
            if constexpr (C4 && QX && KK == KVQ_TOK_AFFINE) {
                // factored scores for key groups of 64 or 128 channels (the
                // cases prefill_factored names)
                if (a.k_group == 64) {
                    hipLaunchKernelGGL((prefill_attn_kernel<KK, VK, 128, QX, C4, 2>), grid, blk_f, 0, s, a, n_q, n_rb, causal);
                    break;
                }
                if (a.k_group == 128) {
                    hipLaunchKernelGGL((prefill_attn_kernel<KK, VK, 128, QX, C4, 1>), grid, blk_f, 0, s, a, n_q, n_rb, causal);
                    break;
                }
            }
            hipLaunchKernelGGL((prefill_attn_kernel<KK, VK, 128, QX, C4, 0>), grid, blk, 0, s, a, n_q, n_rb, causal);
            break;
    }
    return hipGetLastError();
}

template <int KK, int VK, bool QX>
hipError_t launch_prefill_kvq_c(const DecodeArgs& a, int n_q, int n_rb, int causal, hipStream_t s) {
    if constexpr ((KK == KVQ_TOK_AFFINE || KK == KVQ_TOK_SYM4) && VK == KVQ_TOK_AFFINE) {
        if ((KK == KVQ_TOK_SYM4 || a.k_bits == 4) && a.v_bits == 4)
            return launch_prefill_kvq<KK, VK, QX, true>(a, n_q, n_rb, causal, s);
    }
    return launch_prefill_kvq<KK, VK, QX, false>(a, n_q, n_rb, causal, s);
}

template <int KK, int VK>
hipError_t launch_prefill_kv(const DecodeArgs& a, int n_q, int n_rb, int causal, hipStream_t s) {
    return a.q_dtype == KVQ_F32 ? launch_prefill_kvq_c<KK, VK, false>(a, n_q, n_rb, causal, s)
                                : launch_prefill_kvq_c<KK, VK, true>(a, n_q, n_rb, causal, s);
}

template <int KK>
hipError_t launch_prefill_k(const DecodeArgs& a, int n_q, int n_rb, int causal, hipStream_t s) {
    return a.v_kind == KVQ_PLAIN ? launch_prefill_kv<KK, KVQ_PLAIN>(a, n_q, n_rb, causal, s)
                                 : launch_prefill_kv<KK, KVQ_TOK_AFFINE>(a, n_q, n_rb, causal, s);
}

}  // namespace

// Split count before rounding the split length: about 256 workgroups, each
// split at least two tiles long, at most 1024 splits.  The planned count
// never exceeds it, and it grows with T, so its value at the capacity bounds
// every plan of that cache (the workspace size).
int prefill_max_splits(int B, int Hkv, int Hq, int n_q, int T) {
    const int R = (Hq / Hkv) * n_q;
    const int64_t units = (int64_t)B * Hkv * ((R + kRows - 1) / kRows);
    // one round of workgroups: each holds two tile buffers (about 106 KB of
    // LDS at head_dim 128), so one fits per CU and 256 cover the chip
    int64_t ns = (256 + units - 1) / units;
    const int64_t max_ns = ((int64_t)T + 2 * kPT - 1) / (2 * kPT);
    if (ns > max_ns) ns = max_ns;
    if (ns > 1024) ns = 1024;
    if (ns < 1) ns = 1;
    return (int)ns;
}

// Whether a call takes the factored-score kernel (4-bit per-token affine keys
// in groups of 64 or 128 and 4-bit affine values at head_dim 128, fp16 or
// bf16 queries), which works on kFactWaves * 32 rows per workgroup.
bool prefill_factored(const DecodeArgs& a) {
    return a.D == 128 && a.k_kind == KVQ_TOK_AFFINE && a.k_bits == 4 && (a.k_group == 64 || a.k_group == 128) &&
           a.v_kind == KVQ_TOK_AFFINE && a.v_bits == 4 && a.q_dtype != KVQ_F32;
}

// Row blocks per kv-head and token splits (at most prefill_max_splits).  The
// plan aims at one round of workgroups: 256 of kWaves waves, or as many more
// as the factored kernel's smaller workgroups allow.
void prefill_plan(int B, int Hkv, int Hq, int n_q, int T, bool factored, int* n_rb, int* n_splits, int* split_len) {
    const int R = (Hq / Hkv) * n_q;
    const int rows = factored ? 32 * kFactWaves : kRows;
    *n_rb = (R + rows - 1) / rows;
    int64_t ns = prefill_max_splits(B, Hkv, Hq, n_q, T);
    if (factored && kFactWaves < kWaves) {
        const int64_t units = (int64_t)B * Hkv * *n_rb;
        const int64_t want = (256 * (kWaves / kFactWaves) + units - 1) / units;
        if (want < ns) ns = want;
    }
    int len = (int)(((int64_t)T + ns - 1) / ns);
    len = ((len + kPT - 1) / kPT) * kPT;
    *split_len = len;
    *n_splits = (T + len - 1) / len;
    if (*n_splits < 1) *n_splits = 1;
}

hipError_t launch_prefill_attention(const DecodeArgs& a, int n_q, int n_rb, int causal, hipStream_t s) {
    hipError_t e;
    switch (a.k_kind) {
        case KVQ_PLAIN: e = launch_prefill_k<KVQ_PLAIN>(a, n_q, n_rb, causal, s); break;
        case KVQ_KIVI_CH: e = launch_prefill_k<KVQ_KIVI_CH>(a, n_q, n_rb, causal, s); break;
        case KVQ_TOK_AFFINE: e = launch_prefill_k<KVQ_TOK_AFFINE>(a, n_q, n_rb, causal, s); break;
        default: e = launch_prefill_k<KVQ_TOK_SYM4>(a, n_q, n_rb, causal, s); break;
    }
    if (e != hipSuccess) return e;
    return launch_decode_combine_f16(reinterpret_cast<const uint16_t*>(a.ws_o), a.ws_ml, a.out,
                                     (int64_t)a.B * a.Hq * n_q, a.D, a.n_splits, s);
}

}  // namespace kvq

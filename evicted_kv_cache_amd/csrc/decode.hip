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
// bandwidth-tuned kernels for 4-bit-key layouts live in decode_mfma.hip.
#include <math.h>

#include "dequant8.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using dq::k_values8;
using dq::v_values8;

constexpr int kTile = 64;       // tokens per tile
constexpr int kMaxGroup = 8;    // query heads per kv-head
constexpr int kMaxD = 128;

__device__ __forceinline__ float wave_max(float v) { return wave64_max(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave64_sum(v); }

// Generic split-T decode for every layout (D <= 128, up to 8 query heads
// per kv-head).  Per 64-token tile the block dequantizes K and V into LDS as
// fp32 (8 consecutive channels per work item: one code load and one
// metadata load; both token-major, keys with a 4-float row pad so that
// consecutive tokens fall in different banks), computes the logits (thread =
// token x head slot, 16-byte key reads), updates the online softmax per head,
// and accumulates P V (thread = channel x token range, so each value is read
// once for all heads).
//
// C4: 4-bit key and value codes.  The widths are then constants, so a tile's
// fetch is a straight run of loads whose results are first used one tile
// later (with widths known only at run time, the branches around the loads
// cost a wait on each of them).
template <int KK, int VK, int D, bool C4>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a) {
    static_assert(!C4 || (KK != KVQ_PLAIN && VK == KVQ_TOK_AFFINE), "constant code widths: coded layouts");
    if constexpr (C4) {
        a.k_bits = 4;
        a.v_bits = 4;
    }
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    constexpr int c8 = D / 8;
    constexpr int kItems = kTile * c8 / 256;     // 8-channel items per thread and tile (1, 2 or 4)
    const int gq = a.Hq / a.Hkv;
    const int64_t bh = (int64_t)b * a.Hkv + hk;

    __shared__ __align__(16) float q_s[kMaxGroup][kMaxD];
    constexpr int KS = D + 4;                 // key row stride (floats)
    __shared__ __align__(16) float k_s[kTile * (kMaxD + 4)];   // [token][KS]; also the final reduction
    __shared__ __align__(16) float v_s[kTile * kMaxD];
    __shared__ __align__(16) float p_s[kMaxGroup][kTile];
    __shared__ float m_s[kMaxGroup], l_s[kMaxGroup], alpha_s[kMaxGroup];

    for (int idx = tid; idx < gq * D; idx += 256) {
        const int h = idx / D, d = idx - h * D;
        const int64_t qi = ((int64_t)b * a.Hq + hk * gq + h) * D + d;
        float qv;
        if (a.q_dtype == KVQ_F32) qv = static_cast<const float*>(a.q)[qi];
        else if (a.q_dtype == KVQ_F16) qv = f16_bits_to_f32(static_cast<const uint16_t*>(a.q)[qi]);
        else qv = bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[qi]);
        q_s[h][d] = qv * a.scale_log2;
    }
    if (tid < kMaxGroup) { m_s[tid] = -INFINITY; l_s[tid] = 0.0f; alpha_s[tid] = 1.0f; }
    constexpr int hd = D / 2;                 // RoPE pairs (x_j, x_{j + D/2})
    const float2* rope = reinterpret_cast<const float2*>(a.rope);
    if (rope) {
        // the query turns at its own position
        __syncthreads();
        const float2* cs = rope + (int64_t)a.q_pos * hd;
        for (int idx = tid; idx < gq * hd; idx += 256) {
            const int h = idx / hd, j = idx - h * hd;
            const float2 r = cs[j];
            const float x0 = q_s[h][j], x1 = q_s[h][j + hd];
            q_s[h][j] = x0 * r.x - x1 * r.y;
            q_s[h][j + hd] = x0 * r.y + x1 * r.x;
        }
    }

    const int t_begin = split * a.split_len;
    const int t_end = min(a.T, t_begin + a.split_len);
    // PV role: channel d, token range `part` of the tile
    constexpr int TH = 256 / D;             // token ranges per tile (2, 4 or 8)
    const int pd = tid % D, part = tid / D;
    constexpr int tpp = kTile / TH;         // tokens per range
    float acc[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.0f;
    // QK role: token t, head slot (heads slot and slot + 4)
    const int qt = tid & 63, slot = tid >> 6;

    // keys: thread = token (tid % 64) x channel chunks tid / 64 + 4 r, so
    // consecutive lanes write consecutive tokens of the transposed tile;
    // values: consecutive lanes take consecutive channel chunks of a token.
    // The codes and metadata of the next tile are fetched into registers
    // while the current one is computed (the fetch/finish form of the
    // dequantization); kinds without codes load in the finish stage.
    const int kt = tid & 63;
    dq::Pre8 pk[kItems], pv[kItems];
    auto fetch = [&](int tb) {
        const int ntb = min(kTile, t_end - tb);
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            if (kt < ntb) dq::k_fetch8<KK>(a, bh, tb + kt, (tid >> 6) + 4 * r, pk[r]);
            const int it = tid + 256 * r, vt = it / c8, vc = it - vt * c8;
            if (vt < ntb) dq::v_fetch8<VK>(a, bh, tb + vt, vc, pv[r]);
        }
    };
    if (t_begin < t_end) fetch(t_begin);

    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        const int nt = min(kTile, t_end - t0);
        __syncthreads();                    // previous tile's reads of k_s / v_s / p_s are done
        {
            float xk[kItems][8], xv[kItems][8];
#pragma unroll
            for (int r = 0; r < kItems; ++r) {
                if (kt < nt) dq::k_finish8<KK>(a, bh, t0 + kt, (tid >> 6) + 4 * r, pk[r], xk[r]);
                const int it = tid + 256 * r, vt = it / c8, vc = it - vt * c8;
                if (vt < nt) dq::v_finish8<VK>(a, bh, t0 + vt, vc, pv[r], xv[r]);
            }
            if (t0 + kTile < t_end) fetch(t0 + kTile);
#pragma unroll
            for (int r = 0; r < kItems; ++r) {
                if (kt < nt) {
                    const int c = (tid >> 6) + 4 * r;
                    *reinterpret_cast<float4*>(&k_s[kt * KS + 8 * c]) = make_float4(xk[r][0], xk[r][1], xk[r][2], xk[r][3]);
                    *reinterpret_cast<float4*>(&k_s[kt * KS + 8 * c + 4]) = make_float4(xk[r][4], xk[r][5], xk[r][6], xk[r][7]);
                }
                const int it = tid + 256 * r, vt = it / c8, vc = it - vt * c8;
                if (vt < nt) {
                    *reinterpret_cast<float4*>(&v_s[vt * D + 8 * vc]) = make_float4(xv[r][0], xv[r][1], xv[r][2], xv[r][3]);
                    *reinterpret_cast<float4*>(&v_s[vt * D + 8 * vc + 4]) = make_float4(xv[r][4], xv[r][5], xv[r][6], xv[r][7]);
                }
            }
        }
        __syncthreads();
        if (rope) {
            // keys turn at their slot index (the position in the compressed cache)
            static_assert(kTile == 64, "token = idx & 63");
            for (int idx = tid; idx < kTile * hd; idx += 256) {
                const int t = idx & 63, j = idx >> 6;
                if (t < nt) {
                    const float2 r = rope[(int64_t)(t0 + t) * hd + j];
                    const float x0 = k_s[t * KS + j], x1 = k_s[t * KS + j + hd];
                    k_s[t * KS + j] = x0 * r.x - x1 * r.y;
                    k_s[t * KS + j + hd] = x0 * r.y + x1 * r.x;
                }
            }
            __syncthreads();
        }
        {
            float lg0 = 0.0f, lg1 = 0.0f;
            const int h0 = slot, h1 = slot + 4;
            if (qt >= nt) {
                lg0 = lg1 = -INFINITY;
            } else if (gq > 4) {
#pragma unroll 4
                for (int d = 0; d < D; d += 4) {
                    const float4 qa = *reinterpret_cast<const float4*>(&q_s[h0][d]);
                    const float4 qb = *reinterpret_cast<const float4*>(&q_s[h1][d]);
                    const float4 kk = *reinterpret_cast<const float4*>(&k_s[qt * KS + d]);
                    const float k0 = kk.x, k1 = kk.y, k2 = kk.z, k3 = kk.w;
                    lg0 = fmaf(qa.x, k0, lg0); lg0 = fmaf(qa.y, k1, lg0); lg0 = fmaf(qa.z, k2, lg0); lg0 = fmaf(qa.w, k3, lg0);
                    lg1 = fmaf(qb.x, k0, lg1); lg1 = fmaf(qb.y, k1, lg1); lg1 = fmaf(qb.z, k2, lg1); lg1 = fmaf(qb.w, k3, lg1);
                }
            } else if (h0 < gq) {
                // at most 4 query heads: one per wave, the second slot is idle
#pragma unroll 4
                for (int d = 0; d < D; d += 4) {
                    const float4 qa = *reinterpret_cast<const float4*>(&q_s[h0][d]);
                    const float4 kk = *reinterpret_cast<const float4*>(&k_s[qt * KS + d]);
                    lg0 = fmaf(qa.x, kk.x, lg0); lg0 = fmaf(qa.y, kk.y, lg0); lg0 = fmaf(qa.z, kk.z, lg0); lg0 = fmaf(qa.w, kk.w, lg0);
                }
            }
            if (h0 < gq) p_s[h0][qt] = lg0;
            if (h1 < gq) p_s[h1][qt] = lg1;
        }
        __syncthreads();
        {
            const int wave = tid >> 6, lane = tid & 63;
            for (int h = wave; h < gq; h += 4) {
                const float lg = p_s[h][lane];
                const float m_old = m_s[h];
                const float m_new = fmaxf(m_old, wave_max(lg));
                const float e = exp2f(lg - m_new);
                p_s[h][lane] = e;
                const float sum = wave_sum(e);
                if (lane == 0) {
                    const float alpha = exp2f(m_old - m_new);
                    l_s[h] = l_s[h] * alpha + sum;
                    m_s[h] = m_new;
                    alpha_s[h] = alpha;
                }
            }
        }
        __syncthreads();
        {
#pragma unroll
            for (int h = 0; h < kMaxGroup; ++h) acc[h] *= alpha_s[h];
            // four tokens at a time: weights of a head as one 16-byte LDS read
            // (weights past nt are zero: exp2 of -inf; values past tb read as 0)
            const int ta = part * tpp, tb = min(nt, ta + tpp);
            for (int t = ta; t < tb; t += 4) {
                float vv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) vv[u] = t + u < tb ? v_s[(t + u) * D + pd] : 0.0f;   // rows past nt are stale
#pragma unroll
                for (int h = 0; h < kMaxGroup; ++h) {
                    if (h < gq) {
                        const float4 pw = *reinterpret_cast<const float4*>(&p_s[h][t]);
                        acc[h] = fmaf(pw.x, vv[0], acc[h]);
                        acc[h] = fmaf(pw.y, vv[1], acc[h]);
                        acc[h] = fmaf(pw.z, vv[2], acc[h]);
                        acc[h] = fmaf(pw.w, vv[3], acc[h]);
                    }
                }
            }
        }
    }
    // sum the token ranges (reusing k_s) and write the split's partials
    __syncthreads();
    float* red = k_s;                       // [TH][gq][D]
    for (int h = 0; h < gq; ++h) red[(part * gq + h) * D + pd] = acc[h];
    __syncthreads();
    const int ns = a.n_splits;
    for (int idx = tid; idx < gq * D; idx += 256) {
        const int h = idx / D, d = idx - h * D;
        float o = 0.0f;
        for (int pp = 0; pp < TH; ++pp) o += red[(pp * gq + h) * D + d];
        a.ws_o[(((int64_t)b * a.Hq + hk * gq + h) * ns + split) * D + d] = o;
    }
    if (tid < gq) {
        float* ml = a.ws_ml + (((int64_t)b * a.Hq + hk * gq + tid) * ns + split) * 2;
        ml[0] = m_s[tid];
        ml[1] = l_s[tid];
    }
}

// out[row][d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s.  The
// per-split (m, l) pairs are staged in LDS by the block; the partial outputs
// are read eight splits at a time.
constexpr int kCombineMaxSplits = 1024;
// Log-sum-exp merge of the splits of each row: the partials are unnormalized
// sums o, weighted exp2(m - M).
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* ws_o, const float* ws_ml,
                                                             float* out, int D, int ns) {
    // Every load goes out first: the first kPre partial outputs of this
    // thread's channel and this thread's (max, sum) pairs; none depends on
    // the merged max, so the kernel waits for memory once.
    constexpr int kPre = 32;
    const int64_t row = blockIdx.x;
    const int d = threadIdx.x;
    __shared__ float w_s[kCombineMaxSplits];
    __shared__ float red[2][4];
    const float* ml = ws_ml + row * ns * 2;
    const float* o = ws_o + row * ns * D + d;
    // unconditional loads (a split index past ns reads split ns - 1 and gets weight 0)
    float v[kPre];
    if (d < D) {
#pragma unroll
        for (int u = 0; u < kPre; ++u) v[u] = o[(int64_t)min(u, ns - 1) * D];
    }
    float2 mlv[kCombineMaxSplits / 128];
#pragma unroll
    for (int k = 0; k < kCombineMaxSplits / 128; ++k) {
        const int sidx = d + 128 * k;
        mlv[k] = sidx < ns ? reinterpret_cast<const float2*>(ml)[sidx] : make_float2(-INFINITY, 0.0f);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombineMaxSplits / 128; ++k) mloc = fmaxf(mloc, mlv[k].x);
    mloc = wave64_max(mloc);
    if ((d & 63) == 0) red[0][d >> 6] = mloc;
    __syncthreads();
    const float M = fmaxf(red[0][0], red[0][1]);
    float dloc = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombineMaxSplits / 128; ++k) {
        const int sidx = d + 128 * k;
        if (sidx < ns) {
            const float w = exp2f(mlv[k].x - M);
            w_s[sidx] = w;
            dloc = fmaf(w, mlv[k].y, dloc);
        }
    }
    dloc = wave64_sum(dloc);
    if ((d & 63) == 0) red[1][d >> 6] = dloc;
    if (d >= ns && d < kPre) w_s[d] = 0.0f;    // the padding of the prefetch
    __syncthreads();
    const float den = red[1][0] + red[1][1];
    if (d >= D) return;
    float num = 0.0f;
#pragma unroll
    for (int u = 0; u < kPre; ++u) num = fmaf(w_s[u], v[u], num);
    int s = kPre;
    for (; s + 8 <= ns; s += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = o[(int64_t)(s + u) * D];
#pragma unroll
        for (int u = 0; u < 8; ++u) num = fmaf(w_s[s + u], x[u], num);
    }
    for (; s < ns; ++s) num = fmaf(w_s[s], o[(int64_t)s * D], num);
    out[row * D + d] = num / den;
}

// The same merge over fp16 partials o / l (weight exp2(m - M) l), D in {32,
// 64, 128}.  Thread t takes channel pair t % (D/2) (one 32-bit load per
// split) of the splits s = t / (D/2) mod 128 / (D/2); the phases meet in LDS.
__global__ __launch_bounds__(128) void combine_f16_kernel(const uint16_t* ws_o, const float* ws_ml, float* out,
                                                          int D, int ns) {
    constexpr int kPre = 16;                      // splits prefetched per thread
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const int P = D / 2, Q = 128 / P;
    const int c2 = t % P, q = t / P;
    __shared__ float w_s[kCombineMaxSplits];
    __shared__ float red[2][2];
    __shared__ float2 part[128];
    const float* ml = ws_ml + row * ns * 2;
    const uint32_t* o = reinterpret_cast<const uint32_t*>(ws_o + row * ns * D) + c2;     // split s: o[s * P]
    uint32_t v[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) v[u] = o[(int64_t)min(q + Q * u, ns - 1) * P];
    float2 mlv[kCombineMaxSplits / 128];
#pragma unroll
    for (int k = 0; k < kCombineMaxSplits / 128; ++k) {
        const int sidx = t + 128 * k;
        mlv[k] = sidx < ns ? reinterpret_cast<const float2*>(ml)[sidx] : make_float2(-INFINITY, 0.0f);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombineMaxSplits / 128; ++k) mloc = fmaxf(mloc, mlv[k].x);
    mloc = wave64_max(mloc);
    if ((t & 63) == 0) red[0][t >> 6] = mloc;
    __syncthreads();
    const float M = fmaxf(red[0][0], red[0][1]);
    float dloc = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombineMaxSplits / 128; ++k) {
        const int sidx = t + 128 * k;
        if (sidx < ns) {
            const float wl = exp2f(mlv[k].x - M) * mlv[k].y;
            w_s[sidx] = wl;
            dloc += wl;
        }
    }
    dloc = wave64_sum(dloc);
    if ((t & 63) == 0) red[1][t >> 6] = dloc;
    __syncthreads();
    const float den = red[1][0] + red[1][1];
    float nx = 0.0f, ny = 0.0f;
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int sidx = q + Q * u;
        const float w = sidx < ns ? w_s[sidx] : 0.0f;
        nx = fmaf(w, (float)__builtin_bit_cast(_Float16, (uint16_t)(v[u] & 0xFFFFu)), nx);
        ny = fmaf(w, (float)__builtin_bit_cast(_Float16, (uint16_t)(v[u] >> 16)), ny);
    }
    for (int sidx = q + Q * kPre; sidx < ns; sidx += Q) {
        const uint32_t x = o[(int64_t)sidx * P];
        nx = fmaf(w_s[sidx], (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xFFFFu)), nx);
        ny = fmaf(w_s[sidx], (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16)), ny);
    }
    part[t] = make_float2(nx, ny);
    __syncthreads();
    if (t < P) {
        float sx = 0.0f, sy = 0.0f;
        for (int qq = 0; qq < Q; ++qq) { sx += part[qq * P + t].x; sy += part[qq * P + t].y; }
        reinterpret_cast<float2*>(out + row * D)[t] = make_float2(sx / den, sy / den);
    }
}

// (cos, sin) of pos * base^(-2j/D) for pos < n_pos, j < D/2, computed in fp64.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* table, int n_pos, int hd, double base) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n_pos * hd) return;
    const int p = (int)(idx / hd), j = (int)(idx - (int64_t)p * hd);
    const double theta = pow(base, -(double)j / (double)hd);
    double sn, cs;
    sincos((double)p * theta, &sn, &cs);
    table[idx] = make_float2((float)cs, (float)sn);
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

template <int KK, int VK, bool C4>
hipError_t launch_generic_kvc(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.n_splits, (unsigned)a.Hkv, (unsigned)a.B);
    switch (a.D) {
        case 32: hipLaunchKernelGGL((decode_generic_kernel<KK, VK, 32, C4>), grid, dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL((decode_generic_kernel<KK, VK, 64, C4>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((decode_generic_kernel<KK, VK, 128, C4>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int KK, int VK>
hipError_t launch_generic_kv(const DecodeArgs& a, hipStream_t s) {
    if constexpr (KK != KVQ_PLAIN && VK == KVQ_TOK_AFFINE) {
        if ((KK == KVQ_TOK_SYM4 || a.k_bits == 4) && a.v_bits == 4) return launch_generic_kvc<KK, VK, true>(a, s);
    }
    return launch_generic_kvc<KK, VK, false>(a, s);
}

template <int KK>
hipError_t launch_generic_v(const DecodeArgs& a, hipStream_t s) {
    if (a.v_kind == KVQ_PLAIN) return launch_generic_kv<KK, KVQ_PLAIN>(a, s);
    return launch_generic_kv<KK, KVQ_TOK_AFFINE>(a, s);
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
    if (a.n_splits > kCombineMaxSplits) return hipErrorInvalidValue;   // both plans stay <= 512
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

hipError_t launch_rope_table(float* table, int n_pos, int D, double base, hipStream_t s) {
    const int64_t n = (int64_t)n_pos * (D / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<float2*>(table), n_pos, D / 2, base);
    return hipGetLastError();
}

hipError_t launch_decode_combine_f16(const uint16_t* ws_o, const float* ws_ml, float* out, int64_t rows, int D,
                                     int ns, hipStream_t s) {
    if (ns > kCombineMaxSplits || rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (D != 32 && D != 64 && D != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_f16_kernel, dim3((unsigned)rows), dim3(128), 0, s, ws_o, ws_ml, out, D, ns);
    return hipGetLastError();
}

hipError_t launch_decode_combine(const float* ws_o, const float* ws_ml, float* out, int64_t rows, int D, int ns,
                                 hipStream_t s) {
    if (ns > kCombineMaxSplits || rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)rows), dim3(128), 0, s, ws_o, ws_ml, out, D, ns);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace kvq

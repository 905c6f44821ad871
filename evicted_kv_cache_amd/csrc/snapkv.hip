// snapkv.hip -- SnapKV prefill scoring, selection and gather (gfx950).
//
// "SnapKV -- Prefill Observation-Window Token Eviction", section "How it
// works": the last w key rows act as queries; scores are the window mean of
// softmax(K_w K^T / sqrt(D)) rows; the first n_sink positions are always
// kept; the top (budget - n_sink) of the rest are added; kept rows are
// gathered in their original order.
//
// The w x S logit block is a dense fp16 contraction, computed with
// v_mfma_f32_32x32x16_f16 in two passes over the keys: pass 1 (stats) gives
// each window row's max and exp-sum over a stats chunk (keys as MFMA rows, so
// the per-window-row reductions stay inside a lane; a chunk is one to four
// 128-key sub-chunks, more only past 32768 keys, so that at most 64 partials
// per row are left), pass 2 (scores) merges the chunk stats and recomputes the
// logits with window rows as MFMA rows, so each key's sum over window rows
// stays inside a lane.  Recomputing the block is cheaper than storing the
// w x S fp32 logits.
//
// Selection works on order-preserving 32-bit keys of the fp32 scores, one
// workgroup per head: for S <= 32768 the keys stay in registers and the
// threshold (k-th largest key) is found by nested 4096-bucket LDS histograms
// over the candidate key range, finished by ranking the keys of the
// threshold bucket directly once it holds at most 64; longer sequences use an
// MSB-first radix select (4 passes of 8 bits, LDS histograms).  Ties at the
// threshold go to the lower positions, and the kept set is emitted in
// ascending order through block prefix scans.  No floating-point atomics are
// used, so results are reproducible.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 128;          // keys per block (4 waves x 32)
constexpr int kMaxWindow = 128;
constexpr int kStatTarget = 64;      // stats partials per window row (more only past S = 4 * 64 * 128)

__device__ __forceinline__ half8 load_half8(const uint16_t* p) {
    return __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(p));
}

// acc row index (within a 32-row tile) of accumulator element v for lane half kh.
__device__ __forceinline__ int acc_row(int v, int kh) { return 8 * (v >> 2) + 4 * kh + (v & 3); }

// Pass 1: the (max, exp-sum) of every window row over one stats chunk of
// F * a.stat_reps consecutive 128-key sub-chunks (each wave takes 32 keys of
// a sub-chunk, keys as MFMA rows, so the per-window-row reductions stay
// inside a lane).  Sub-chunks are merged online; long sequences take several
// sub-chunks per workgroup so that the scores pass merges few partials.
template <int D, int F>
__global__ __launch_bounds__(256) void snap_stats_kernel(SnapArgs a) {
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int kh = lane >> 5, l32 = lane & 31;
    const int S = a.S;
    const int wc = a.n_rows;
    const uint16_t* K = a.k + ((int64_t)b * a.H + h) * a.kv_stride;
    const uint16_t* O = a.obs + ((int64_t)b * a.H + h) * a.obs_stride;   // observation rows
    const float c = 1.4426950408889634f / sqrtf((float)D);
    __shared__ float sm[4][kMaxWindow], sl[4][kMaxWindow];
    constexpr int NK = D / 16;
    constexpr int NT = kMaxWindow / 32;
    // running (max, sum) of window row nt * 32 + l32, both lane halves alike
    float M[NT], L[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) { M[nt] = -INFINITY; L[nt] = 0.0f; }

    for (int rep = 0; rep < a.stat_reps; ++rep) {
        const int sub0 = (chunk * a.stat_reps + rep) * F;     // first 128-key sub-chunk of this step
        // this lane's key fragments of all F sub-chunks: all loads in flight together
        half8 A[F][NK];
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int key = (sub0 + f) * kChunk + wave * 32 + l32;
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                A[f][q] = half8{};
                if (key < S) A[f][q] = load_half8(K + (int64_t)key * D + q * 16 + kh * 8);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt * 32 >= wc) break;
            const int wr = nt * 32 + l32;
            half8 Bv[NK];
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                Bv[q] = half8{};
                if (wr < wc) Bv[q] = load_half8(O + (int64_t)wr * D + q * 16 + kh * 8);
            }
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const int key_base = (sub0 + f) * kChunk + wave * 32;
                if (key_base >= S) break;                  // uniform: the rest is past the end
                floatx16 acc = {};
#pragma unroll
                for (int q = 0; q < NK; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[f][q], Bv[q], acc, 0, 0, 0);
                // acc[v] = logit(key_base + acc_row(v, kh), window row wr)
                float mx = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (key_base + acc_row(v, kh) < S) mx = fmaxf(mx, acc[v] * c);
                mx = fmaxf(mx, lane_xor<32>(mx));
                const float Mn = fmaxf(M[nt], mx);           // finite: key_base < S
                float sum = 0.0f;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (key_base + acc_row(v, kh) < S) sum += exp2f(acc[v] * c - Mn);
                sum = swap32_sum(sum, sum);
                L[nt] = (M[nt] == -INFINITY ? 0.0f : L[nt] * exp2f(M[nt] - Mn)) + sum;
                M[nt] = Mn;
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int wr = nt * 32 + l32;
        if (kh == 0 && wr < wc) { sm[wave][wr] = M[nt]; sl[wave][wr] = L[nt]; }
    }
    __syncthreads();
    if (tid < wc) {
        float Mx = -INFINITY;
        for (int w = 0; w < 4; ++w) Mx = fmaxf(Mx, sm[w][tid]);
        float Lx = 0.0f;
        for (int w = 0; w < 4; ++w)
            if (sm[w][tid] > -INFINITY) Lx += sl[w][tid] * exp2f(sm[w][tid] - Mx);
        float* st = a.stats + ((((int64_t)b * a.H + h) * a.n_stat + chunk) * wc + tid) * 2;
        st[0] = Mx;
        st[1] = Lx;
    }
}

template <int D>
__global__ __launch_bounds__(256) void snap_scores_kernel(SnapArgs a) {
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int kh = lane >> 5, l32 = lane & 31;
    const int S = a.S;
    const int wc = a.n_rows;
    const uint16_t* K = a.k + ((int64_t)b * a.H + h) * a.kv_stride;
    const uint16_t* O = a.obs + ((int64_t)b * a.H + h) * a.obs_stride;   // observation rows
    const float c = 1.4426950408889634f / sqrtf((float)D);
    __shared__ float Mrow[kMaxWindow], invL[kMaxWindow];
    // Loads in the order they are needed: the first batch of chunk stats
    // (their merge runs while the key and window fragments are in flight),
    // then this lane's key fragments, then the first window tile.
    const int tpr = wc <= 32 ? 8 : (wc <= 64 ? 4 : 2);     // threads per window row in the merge
    const int r = tid / tpr, j = tid % tpr;
    const float* st = a.stats + (((int64_t)b * a.H + h) * a.n_stat * wc + r) * 2;
    float2 ml[8];
    auto load_stats = [&](int ch0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int ch = ch0 + u * tpr;
            ml[u] = (r < wc && ch < a.n_stat) ? *reinterpret_cast<const float2*>(st + (int64_t)ch * wc * 2)
                                              : make_float2(-INFINITY, 0.0f);
        }
    };
    load_stats(j);
    const int key = chunk * kChunk + wave * 32 + l32;
    constexpr int NK = D / 16;
    half8 Bk[NK];
#pragma unroll
    for (int q = 0; q < NK; ++q) {
        Bk[q] = half8{};
        if (key < S) Bk[q] = load_half8(K + (int64_t)key * D + q * 16 + kh * 8);
    }
    half8 A[NK];
#pragma unroll
    for (int q = 0; q < NK; ++q) {
        A[q] = half8{};
        if (l32 < wc) A[q] = load_half8(O + (int64_t)l32 * D + q * 16 + kh * 8);
    }
    {
        // merge the per-chunk (max, sum) of every window row: tpr threads per
        // row stride over the chunks (eight at a time, one common max per
        // batch), then combine with lane shuffles
        float M = -INFINITY, L = 0.0f;
        for (int ch0 = j;;) {
            float mb = M;
#pragma unroll
            for (int u = 0; u < 8; ++u) mb = fmaxf(mb, ml[u].x);
            if (mb > -INFINITY) {
                float Ln = M == -INFINITY ? 0.0f : L * exp2f(M - mb);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (ml[u].x > -INFINITY) Ln += ml[u].y * exp2f(ml[u].x - mb);
                L = Ln;
                M = mb;
            }
            ch0 += 8 * tpr;
            if (ch0 >= a.n_stat) break;
            load_stats(ch0);
        }
        auto merge_pair = [&](float m2, float l2) {
            const float Mn = fmaxf(M, m2);
            L = (M == -INFINITY ? 0.0f : L * exp2f(M - Mn)) + (m2 == -INFINITY ? 0.0f : l2 * exp2f(m2 - Mn));
            M = Mn;
        };
        // lanes j = 0 .. tpr - 1 of a row (tpr in {2, 4, 8}) merge by lane distances 1, 2, 4
        if (tpr > 1) { const float m2 = lane_xor<1>(M), l2 = lane_xor<1>(L); merge_pair(m2, l2); }
        if (tpr > 2) { const float m2 = lane_xor<2>(M), l2 = lane_xor<2>(L); merge_pair(m2, l2); }
        if (tpr > 4) { const float m2 = lane_xor<4>(M), l2 = lane_xor<4>(L); merge_pair(m2, l2); }
        if (r < wc && j == 0) {
            Mrow[r] = M;
            invL[r] = 1.0f / L;
        }
    }
    __syncthreads();
    float score = 0.0f;
    for (int mt = 0; mt * 32 < wc; ++mt) {
        const int wr = mt * 32 + l32;
        if (mt > 0) {
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                A[q] = half8{};
                if (wr < wc) A[q] = load_half8(O + (int64_t)wr * D + q * 16 + kh * 8);
            }
        }
        floatx16 acc = {};
#pragma unroll
        for (int q = 0; q < NK; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[q], Bk[q], acc, 0, 0, 0);
        // acc[v] = logit(window row mt*32 + acc_row(v, kh), key)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = mt * 32 + acc_row(v, kh);
            if (i < wc) score += exp2f(acc[v] * c - Mrow[i]) * invL[i];
        }
    }
    score = swap32_sum(score, score);
    if (kh == 0 && key < S)
        a.scores[((int64_t)b * a.H + h) * S + key] = score / (float)wc;
}

// ---------------------------------------------------------------- one-read scores
//
// The keys are read once.  Workgroup (chunk, h, b) computes the logits of its
// one_chunk keys against every observation row (keys as MFMA rows, as in
// pass 1) and keeps them in registers, publishes its per-row (max, exp-sum),
// waits until every chunk of its head has published, merges the head's
// statistics and turns its own logits into scores.  The exchange uses
// agent-coherent stores and loads: a workgroup's partials are stored and
// complete before its ready flag takes the call's tag.  The wait is bounded:
// a workgroup that gives up (when not every chunk of the head could be
// resident at once, for instance) recomputes every chunk's partials itself
// with the same code, so the statistics, and the scores, are the same bits
// either way.  The select-gather launch that follows clears the flags.

__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): this lane's stores have completed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, int F, int NT>
__global__ __launch_bounds__(256) void snap_one_read_kernel(SnapArgs a) {
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int kh = lane >> 5, l32 = lane & 31;
    const int S = a.S, wc = a.n_rows, n_c = a.n_one, ck = a.one_chunk;
    const int64_t bh = (int64_t)b * a.H + h;
    const uint16_t* K = a.k + bh * a.kv_stride;
    const uint16_t* O = a.obs + bh * a.obs_stride;   // observation rows
    float* part = a.stats + bh * (int64_t)n_c * wc * 2;   // [n_c][wc] (max, sum)
    uint64_t* flag = a.flags + bh * n_c;
    const float c = 1.4426950408889634f / sqrtf((float)D);
    constexpr int NK = D / 16;
    __shared__ float sm[4][kMaxWindow], sl[4][kMaxWindow];
    __shared__ float Mrow[kMaxWindow], invL[kMaxWindow];

    // acc[f][nt][v] = logit(key kb(f) + acc_row(v, kh), observation row nt * 32 + l32)
    auto key_base = [&](int ch, int f) { return ch * ck + (f * 4 + wave) * 32; };
    auto logits = [&](int ch, floatx16 (&acc)[F][NT]) {
        half8 A[F][NK];
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int key = key_base(ch, f) + l32;
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                A[f][q] = half8{};
                if (key < S) A[f][q] = load_half8(K + (int64_t)key * D + q * 16 + kh * 8);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int wr = nt * 32 + l32;
            half8 Bv[NK];
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                Bv[q] = half8{};
                if (wr < wc) Bv[q] = load_half8(O + (int64_t)wr * D + q * 16 + kh * 8);
            }
#pragma unroll
            for (int f = 0; f < F; ++f) {
                floatx16 x = {};
#pragma unroll
                for (int q = 0; q < NK; ++q) x = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[f][q], Bv[q], x, 0, 0, 0);
                acc[f][nt] = x;
            }
        }
    };
    // (max, exp-sum) of every observation row over chunk ch's keys, stored
    // agent-coherent into the chunk's partials
    auto publish = [&](int ch, const floatx16 (&acc)[F][NT]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float M = -INFINITY, L = 0.0f;
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const int kb = key_base(ch, f);
                if (kb >= S) break;                        // uniform: the rest is past the end
                float mx = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (kb + acc_row(v, kh) < S) mx = fmaxf(mx, acc[f][nt][v] * c);
                mx = fmaxf(mx, lane_xor<32>(mx));
                const float Mn = fmaxf(M, mx);
                float sum = 0.0f;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (kb + acc_row(v, kh) < S) sum += exp2f(acc[f][nt][v] * c - Mn);
                sum = swap32_sum(sum, sum);
                L = (M == -INFINITY ? 0.0f : L * exp2f(M - Mn)) + sum;
                M = Mn;
            }
            const int wr = nt * 32 + l32;
            if (kh == 0 && wr < wc) { sm[wave][wr] = M; sl[wave][wr] = L; }
        }
        __syncthreads();
        if (tid < wc) {
            float Mx = -INFINITY;
            for (int w = 0; w < 4; ++w) Mx = fmaxf(Mx, sm[w][tid]);
            float Lx = 0.0f;
            for (int w = 0; w < 4; ++w)
                if (sm[w][tid] > -INFINITY) Lx += sl[w][tid] * exp2f(sm[w][tid] - Mx);
            st_agent(part + ((int64_t)ch * wc + tid) * 2, Mx);
            st_agent(part + ((int64_t)ch * wc + tid) * 2 + 1, Lx);
        }
        __syncthreads();
    };

    floatx16 acc[F][NT];
    logits(chunk, acc);
    publish(chunk, acc);
    if (tid < wc) wait_vmem();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flag + chunk, a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool late = false;
    if (tid < n_c) {
        const uint64_t t0 = wall_clock64();
        while (__hip_atomic_load(flag + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.tag) {
            if ((int64_t)(wall_clock64() - t0) > a.wait_ticks) { late = true; break; }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    if (__syncthreads_or(late)) {
        // not every chunk of the head published in time: compute them all here
        for (int ch = 0; ch < n_c; ++ch) {
            logits(ch, acc);
            publish(ch, acc);
        }
        if (tid < wc) wait_vmem();
        __syncthreads();
        logits(chunk, acc);
    }
    {
        // merge the head's per-chunk (max, sum) of every observation row: tpr
        // threads per row stride over the chunks (eight at a time, one common
        // max per batch), then combine with lane shuffles
        const int tpr = wc <= 32 ? 8 : (wc <= 64 ? 4 : 2);
        const int r = tid / tpr, j = tid % tpr;
        float M = -INFINITY, L = 0.0f;
        for (int ch0 = j; ch0 < n_c; ch0 += 8 * tpr) {
            float pm[8], pl[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int ch = ch0 + u * tpr;
                pm[u] = -INFINITY;
                pl[u] = 0.0f;
                if (r < wc && ch < n_c) {
                    pm[u] = ld_agent(part + ((int64_t)ch * wc + r) * 2);
                    pl[u] = ld_agent(part + ((int64_t)ch * wc + r) * 2 + 1);
                }
            }
            float mb = M;
#pragma unroll
            for (int u = 0; u < 8; ++u) mb = fmaxf(mb, pm[u]);
            if (mb > -INFINITY) {
                float Ln = M == -INFINITY ? 0.0f : L * exp2f(M - mb);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (pm[u] > -INFINITY) Ln += pl[u] * exp2f(pm[u] - mb);
                L = Ln;
                M = mb;
            }
        }
        auto merge_pair = [&](float m2, float l2) {
            const float Mn = fmaxf(M, m2);
            L = (M == -INFINITY ? 0.0f : L * exp2f(M - Mn)) + (m2 == -INFINITY ? 0.0f : l2 * exp2f(m2 - Mn));
            M = Mn;
        };
        // lanes j = 0 .. tpr - 1 of a row (tpr in {2, 4, 8}) merge by lane distances 1, 2, 4
        if (tpr > 1) { const float m2 = lane_xor<1>(M), l2 = lane_xor<1>(L); merge_pair(m2, l2); }
        if (tpr > 2) { const float m2 = lane_xor<2>(M), l2 = lane_xor<2>(L); merge_pair(m2, l2); }
        if (tpr > 4) { const float m2 = lane_xor<4>(M), l2 = lane_xor<4>(L); merge_pair(m2, l2); }
        if (r < wc && j == 0) {
            Mrow[r] = M;
            invL[r] = 1.0f / L;
        }
    }
    __syncthreads();
    // scores: each lane sums its observation rows' weights for its 16 keys,
    // then the 32 lanes of a half add up (reduce-scatter over 16 lanes, then
    // the two 16-lane groups), leaving key acc_row(l32 & 15, kh) in lane l32
    float mrow[NT], ilr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int wr = nt * 32 + l32;
        mrow[nt] = wr < wc ? Mrow[wr] : 0.0f;
        ilr[nt] = wr < wc ? invL[wr] : 0.0f;
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
        const int kb = key_base(chunk, f);
        if (kb >= S) break;                                // uniform
        float x[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float sacc = 0.0f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                if (nt * 32 + l32 < wc) sacc += exp2f(acc[f][nt][v] * c - mrow[nt]) * ilr[nt];
            x[v] = sacc;
        }
        float x8[8], x4[4], x2[2];
        {
            const bool hi = (l32 & 8) != 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) x8[i] = (hi ? x[i + 8] : x[i]) + lane_xor<8>(hi ? x[i] : x[i + 8]);
        }
        {
            const bool hi = (l32 & 4) != 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) x4[i] = (hi ? x8[i + 4] : x8[i]) + lane_xor<4>(hi ? x8[i] : x8[i + 4]);
        }
        {
            const bool hi = (l32 & 2) != 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) x2[i] = (hi ? x4[i + 2] : x4[i]) + lane_xor<2>(hi ? x4[i] : x4[i + 2]);
        }
        const bool hi = (l32 & 1) != 0;
        float sc = (hi ? x2[1] : x2[0]) + lane_xor<1>(hi ? x2[0] : x2[1]);
        sc = swap16_sum(sc, sc);
        const int key = kb + acc_row(l32 & 15, kh);
        if (l32 < 16 && key < S) a.scores[bh * S + key] = sc / (float)wc;
    }
}

// ---------------------------------------------------------------- selection

__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;                 // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one value per thread over a block of nthreads (<= 1024)
// threads; returns the inclusive prefix, and *total the block sum.  Wave
// scans by shuffles; the (<= 16) wave totals are scanned by wave 0.
__device__ uint32_t block_scan(uint32_t v, uint32_t* lds16, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) lds16[wave] = x;
    __syncthreads();
    if (wave == 0) {
        const uint32_t t = lane < nw ? lds16[lane] : 0u;
        uint32_t incl = t;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane < nw) lds16[lane] = incl - t;      // exclusive prefix of the wave totals
        if (lane == nw - 1) lds16[16] = incl;
    }
    __syncthreads();
    const uint32_t res = x + lds16[wave];
    *total = lds16[16];
    __syncthreads();
    return res;
}

// Radix select for long sequences (S > 16384): 4 passes of 8 bits over the
// keys, read from global memory on every pass, with per-wave LDS histograms.
__global__ __launch_bounds__(1024) void snap_select_radix_kernel(const float* scores, int S, int n_sink,
                                                                 int budget, int32_t* kept_all) {
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int n_keep = min(budget, S);
    const int n_s = min(n_sink, n_keep);
    const int k = n_keep - n_s;
    const int C = S - n_s;
    const float* sc = scores + bh * S;
    int32_t* kept = kept_all + bh * n_keep;
    if (k == C || k == 0) {                       // all candidates, or sinks only
        for (int i = tid; i < n_keep; i += blockDim.x) kept[i] = i;
        return;
    }
    auto key_of = [&](int j) -> uint32_t { return order_key(sc[j]); };
    __shared__ uint32_t whist[16][256];     // one histogram per wave: no cross-wave contention
    __shared__ uint32_t lds16[17];
    __shared__ uint32_t s_prefix, s_krem;
    uint32_t prefix = 0, mask = 0, krem = (uint32_t)k;
    const int wv = tid >> 6;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 16 * 256; i += blockDim.x) (&whist[0][0])[i] = 0;
        __syncthreads();
        for (int j = n_s + tid; j < S; j += blockDim.x) {
            const uint32_t key = key_of(j);
            if ((key & mask) == prefix) atomicAdd(&whist[wv][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // bins from the top: thread t holds bin 255 - t, summed over the waves
        uint32_t cnt = 0;
        if (tid < 256) {
#pragma unroll
            for (int w = 0; w < 16; ++w) cnt += whist[w][255 - tid];
        }
        uint32_t tot;
        const uint32_t incl = block_scan(cnt, lds16, &tot);
        if (tid < 256 && incl - cnt < krem && incl >= krem) {
            s_prefix = prefix | ((uint32_t)(255 - tid) << shift);
            s_krem = krem - (incl - cnt);
        }
        __syncthreads();
        prefix = s_prefix;
        krem = s_krem;
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t tau = prefix;   // k-th largest key; krem of the keys equal to tau are taken
    const int per = (S + (int)blockDim.x - 1) / (int)blockDim.x;
    const int j0 = min(S, tid * per), j1 = min(S, j0 + per);
    uint32_t nties = 0;
    for (int j = max(j0, n_s); j < j1; ++j) nties += (key_of(j) == tau);
    uint32_t tot;
    uint32_t tie_rank = block_scan(nties, lds16, &tot) - nties;
    uint32_t nsel = 0;
    for (int j = j0; j < j1; ++j) {
        bool sel;
        if (j < n_s) sel = true;
        else {
            const uint32_t key = key_of(j);
            if (key > tau) sel = true;
            else if (key == tau) sel = (tie_rank++ < krem);
            else sel = false;
        }
        nsel += sel;
    }
    uint32_t out = block_scan(nsel, lds16, &tot) - nsel;
    tie_rank -= nties;
    for (int j = j0; j < j1; ++j) {
        bool sel;
        if (j < n_s) sel = true;
        else {
            const uint32_t key = key_of(j);
            if (key > tau) sel = true;
            else if (key == tau) sel = (tie_rank++ < krem);
            else sel = false;
        }
        if (sel && out < (uint32_t)n_keep) kept[out++] = j;
    }
}

// Register-resident select for S <= 1024 * KPT: thread t holds the keys of
// positions t*KPT .. t*KPT+KPT-1 (sinks and positions past S as key 0, below
// every real key).  The threshold tau -- the k-th largest candidate key -- is
// found by bucketing: the candidate range [min, max] is split into 4096
// equal buckets (an LDS histogram; keys are order-preserving float bits, so
// buckets are close to logarithmic in the score and atomics rarely collide),
// a scan from the top finds the bucket holding the k-th largest key, and the
// search repeats inside that bucket with 12 more bits until a bucket is a
// single key value (at most three levels).  One block scan of the packed
// per-thread counts (sinks or above tau, equal to tau) then gives every kept
// position its output slot: positions above tau keep their order, and the
// first krem positions equal to tau are taken.
constexpr int kSelThreads = 1024;    // select block: 16 waves
constexpr int kSelBits = 12;
constexpr int kSelBuckets = 1 << kSelBits;              // 16 KB LDS histogram
constexpr int kSelPer = kSelBuckets / kSelThreads;      // buckets per thread (4)

// Inclusive wave scan with DPP: row shifts 1, 2, 4, 8 scan each row of 16
// lanes, then row broadcasts of lanes 15 and 31 carry the row totals.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
    return x;
}

// Exclusive scan of v over the 1024 threads with one barrier: a wave scan,
// then every wave reads the 16 wave totals.  `tot16` must not be reused
// before the next barrier.
__device__ __forceinline__ uint32_t scan1024(uint32_t v, uint32_t* tot16, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_scan_dpp(v);
    if (lane == 63) tot16[wave] = x;
    __syncthreads();
    const uint4* p = reinterpret_cast<const uint4*>(tot16);
    const uint4 q0 = p[0], q1 = p[1], q2 = p[2], q3 = p[3];
    const uint32_t t[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                            q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        before += w < wave ? t[w] : 0u;
        all += t[w];
    }
    *total = all;
    return before + x - v;
}

// Top-k of one (batch, head) row of scores sc[0, S) by the whole block, with
// the keys in registers (S <= kSelThreads * KPT): the kept indices in
// ascending order go to `kept` and, when given, to `kept_lds`.
template <int KPT>
__device__ __forceinline__ void select_reg(const float* sc, int S, int n_sink, int budget, int32_t* kept,
                                           int32_t* kept_lds) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_keep = min(budget, S);
    const int n_s = min(n_sink, n_keep);
    const int k = n_keep - n_s;
    const int C = S - n_s;
    auto emit = [&](uint32_t out, int j) {
        if (kept) kept[out] = j;
        if (kept_lds) kept_lds[out] = j;
    };
    if (k == C || k == 0) {                       // all candidates, or sinks only
        for (int i = tid; i < n_keep; i += blockDim.x) emit((uint32_t)i, i);
        return;
    }
    __shared__ __align__(16) uint32_t hist[kSelBuckets];
    __shared__ __align__(16) uint32_t tot16[4][16];
    __shared__ uint32_t pick[2][3];             // bucket, keys above it, keys in it
    __shared__ uint32_t cand[64], cand_rank[64], cand_n, fin[2];
    uint32_t key[KPT];
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    {
        // bounds-checked buffer loads: positions past S read as 0
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sc), (short)0, S * 4, 0x00020000);
        uint32_t raw[KPT];
        if ((S & 3) == 0) {
            // every 16-byte group is wholly inside or wholly past the end
#pragma unroll
            for (int i = 0; i < KPT; i += 4) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, (tid * KPT + i) * 4, 0, 0);
                raw[i] = x.x; raw[i + 1] = x.y; raw[i + 2] = x.z; raw[i + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < KPT; ++i) raw[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (tid * KPT + i) * 4, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int j = tid * KPT + i;
            key[i] = (j >= n_s && j < S) ? order_key(__uint_as_float(raw[i])) : 0u;
            if (key[i] != 0u) { kmin = min(kmin, key[i]); kmax = max(kmax, key[i]); }
        }
    }
    // zero the histogram while the keys load
    uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) h4[tid * (kSelPer / 4) + q] = make_uint4(0u, 0u, 0u, 0u);
    kmin = lane_reduce<true>(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
    kmax = lane_reduce<true>(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
    if (lane == 0) { tot16[0][wave] = kmin; tot16[1][wave] = kmax; }
    if (tid < 64) cand_rank[tid] = 0u;
    if (tid == 0) cand_n = 0u;
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int w = 0; w < 16; ++w) { lo = min(lo, tot16[0][w]); hi = max(hi, tot16[1][w]); }
    // bucket search over the keys in [base, base + lim): bucket (key - base) >> shift
    uint32_t base = lo, krem = (uint32_t)k;       // krem: rank of tau from the top of the range
    const uint32_t range = hi - lo;               // <= 0xFFFFFFFE: real keys are >= 0x007FFFFF
    uint32_t lim = range + 1u;
    int shift = range == 0u ? 0 : max(0, 32 - __clz((int)range) - kSelBits);   // range < 2^(shift + kSelBits)
    // Three barriers per level: after the histogram, inside the scan, after
    // the pick.  Each thread reads (and then clears) only its own buckets, so
    // clearing them for the next level needs no barrier of its own; the pick
    // and the scan's wave totals alternate between two slots.
    for (int level = 0;; ++level) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const uint32_t off = key[i] - base;       // keys below base wrap to large values
            if (key[i] != 0u && off < lim) atomicAdd(&hist[off >> shift], 1u);
        }
        __syncthreads();
        // thread t owns the buckets kSelBuckets-1-kSelPer*t downwards (scan from the top)
        const int top = kSelBuckets - kSelPer * (tid + 1);     // lowest bucket of this thread
        uint32_t cnt[kSelPer];
#pragma unroll
        for (int q = 0; q < kSelPer / 4; ++q) {
            const uint4 x = h4[top / 4 + q];
            cnt[4 * q] = x.x; cnt[4 * q + 1] = x.y; cnt[4 * q + 2] = x.z; cnt[4 * q + 3] = x.w;
            h4[top / 4 + q] = make_uint4(0u, 0u, 0u, 0u);
        }
        uint32_t v = 0;
#pragma unroll
        for (int q = 0; q < kSelPer; ++q) v += cnt[q];
        uint32_t tot;
        const uint32_t excl = scan1024(v, tot16[2 + (level & 1)], &tot);
        if (excl < krem && excl + v >= krem) {
            uint32_t run = excl;
#pragma unroll
            for (int q = kSelPer - 1; q >= 0; --q) {      // descending buckets
                if (run < krem && run + cnt[q] >= krem) {
                    pick[level & 1][0] = (uint32_t)(top + q);
                    pick[level & 1][1] = run;
                    pick[level & 1][2] = cnt[q];
                }
                run += cnt[q];
            }
        }
        __syncthreads();
        const uint32_t bucket = pick[level & 1][0], above = pick[level & 1][1], n_in = pick[level & 1][2];
        base += bucket << shift;
        krem -= above;
        if (shift == 0) break;                    // the bucket is one key value
        if (n_in <= 64u) {
            // Few keys in the bucket [base, base + 2^shift): gather them and
            // rank them directly.  Wave w compares every candidate with
            // candidates 4w .. 4w+3; the counts (greater | equal << 16) meet
            // in LDS, and tau is the candidate with greater < krem <= greater + equal.
            const uint32_t width = 1u << shift;
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                if (key[i] != 0u && key[i] - base < width) {
                    const uint32_t slot = atomicAdd(&cand_n, 1u);
                    if (slot < 64u) cand[slot] = key[i];
                }
            }
            __syncthreads();
            const uint32_t ci = (uint32_t)lane, j0 = 4u * (uint32_t)wave;
            if (ci < n_in && j0 < n_in) {
                const uint32_t x = cand[ci];
                uint32_t gt = 0, eq = 0;
#pragma unroll
                for (uint32_t u = 0; u < 4; ++u) {
                    if (j0 + u < n_in) {
                        const uint32_t y = cand[j0 + u];
                        gt += (y > x);
                        eq += (y == x);
                    }
                }
                atomicAdd(&cand_rank[ci], gt | (eq << 16));
            }
            __syncthreads();
            if ((uint32_t)tid < n_in) {
                const uint32_t r = cand_rank[tid], gt = r & 0xFFFFu, eq = r >> 16;
                if (gt < krem && gt + eq >= krem) { fin[0] = cand[tid]; fin[1] = krem - gt; }
            }
            __syncthreads();
            base = fin[0];
            krem = fin[1];
            break;
        }
        lim = 1u << shift;
        shift = max(0, shift - kSelBits);
    }
    const uint32_t tau = base;                    // k-th largest key; krem keys equal to it are kept
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int j = tid * KPT + i;
        n_gt += (j < n_s || key[i] > tau);
        n_eq += (key[i] == tau);
    }
    uint32_t tot;
    const uint32_t packed = n_gt | (n_eq << 16);
    // tot16[0] (the key minima) was last read before the first level
    const uint32_t excl = scan1024(packed, tot16[0], &tot);
    uint32_t a_run = excl & 0xFFFFu, e_run = excl >> 16;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int j = tid * KPT + i;
        if (j >= S) break;
        if (j < n_s || key[i] > tau) {
            const uint32_t out = a_run + min(e_run, krem);
            if (out < (uint32_t)n_keep) emit(out, j);
            ++a_run;
        } else if (key[i] == tau) {
            if (e_run < krem) {
                const uint32_t out = a_run + e_run;
                if (out < (uint32_t)n_keep) emit(out, j);
            }
            ++e_run;
        }
    }
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void snap_select_reg_kernel(const float* scores, int S, int n_sink,
                                                                      int budget, int32_t* kept_all) {
    const int64_t bh = blockIdx.x;
    const int n_keep = min(budget, S);
    select_reg<KPT>(scores + bh * S, S, n_sink, budget, kept_all + bh * n_keep, nullptr);
}

// Select and gather in one launch: n_rep blocks per (batch, head) each run
// the same selection (block rep 0 writes the kept indices), then copy their
// share of the kept K and V rows (and positions).  The selection is
// latency-bound and the copy is short, so the repeats cost nothing and the
// gather's own launch disappears.
constexpr int kFuseMaxKeep = 4096;
// Blocks go to the XCDs in turn (block x on XCD x % 8), so block x =
// ((bh / 8) n_rep + rep) 8 + bh % 8 puts the n_rep blocks of one (batch,
// head) on one XCD, where they share its L2 copy of the head's scores; the
// grid is padded to whole groups of 8 heads.
constexpr int kXcds = 8;
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void snap_select_gather_kernel(SnapArgs a, const float* rank, int n_rep) {
    __shared__ int32_t keptl[kFuseMaxKeep];
    const int xcd = (int)(blockIdx.x % kXcds), jx = (int)(blockIdx.x / kXcds);
    const int rep = jx % n_rep;
    const int64_t bh = (int64_t)(jx / n_rep) * kXcds + xcd;
    if (bh >= (int64_t)a.B * a.H) return;         // padding block
    const int n_keep = min(a.budget, a.S);
    select_reg<KPT>(rank + bh * a.S, a.S, a.n_sink, a.budget, rep == 0 ? a.kept + bh * n_keep : nullptr, keptl);
    if (a.flags && rep == 0)                      // the one-read scores' ready flags, for the next call
        for (int t = (int)threadIdx.x; t < a.n_one; t += kSelThreads) a.flags[bh * a.n_one + t] = 0u;
    __syncthreads();
    const int upr = a.D / 8;                      // 16-byte units per fp16 row
    const int units = n_keep * upr;
    const int per = (units + n_rep - 1) / n_rep;
    const int u1 = min(units, (rep + 1) * per);
    for (int x = rep * per + (int)threadIdx.x; x < u1; x += kSelThreads) {
        const int rl = x / upr, u = x - rl * upr;
        const int j = keptl[rl];
        const int64_t src = (bh * a.kv_stride + (int64_t)j * a.D) / 8 + u;
        const int64_t dst = (bh * a.out_stride + (int64_t)rl * a.D) / 8 + u;
        reinterpret_cast<uint4*>(a.k_out)[dst] = reinterpret_cast<const uint4*>(a.k)[src];
        reinterpret_cast<uint4*>(a.v_out)[dst] = reinterpret_cast<const uint4*>(a.v)[src];
        if (u == 0 && a.pos_out)
            a.pos_out[bh * a.pos_out_rows + rl] = a.pos_in ? a.pos_in[bh * a.pos_in_rows + j] : j;
    }
}

__global__ __launch_bounds__(256) void snap_gather_kernel(SnapArgs a, int n_keep) {
    const int upr = a.D / 8;                      // 16-byte units per fp16 row
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)a.B * a.H * n_keep;
    if (idx >= rows * upr) return;
    const int64_t r = idx / upr;
    const int u = (int)(idx - r * upr);
    const int64_t bh = r / n_keep;
    const int rl = (int)(r - bh * n_keep);
    const int j = a.kept[r];
    if (j < 0 || j >= a.S) return;
    const int64_t src = (bh * a.kv_stride + (int64_t)j * a.D) / 8 + u;
    const int64_t dst = (bh * a.out_stride + (int64_t)rl * a.D) / 8 + u;
    reinterpret_cast<uint4*>(a.k_out)[dst] = reinterpret_cast<const uint4*>(a.k)[src];
    reinterpret_cast<uint4*>(a.v_out)[dst] = reinterpret_cast<const uint4*>(a.v)[src];
    if (u == 0 && a.pos_out)
        a.pos_out[bh * a.pos_out_rows + rl] = a.pos_in ? a.pos_in[bh * a.pos_in_rows + j] : j;
}

// Chunk rows into a kept-row state: thread (row, unit) copies one 16-byte
// unit of K and V; unit 0 also writes the row's position.
__global__ __launch_bounds__(256) void snap_chunk_copy_kernel(const uint4* __restrict__ kc, const uint4* __restrict__ vc,
                                                              uint4* __restrict__ ks, uint4* __restrict__ vs,
                                                              int32_t* __restrict__ ps, int64_t rows, int n, int upr,
                                                              int cap, int row0, int first_pos) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * upr) return;
    const int64_t r = idx / upr;
    const int u = (int)(idx - r * upr);
    const int64_t bh = r / n;
    const int i = (int)(r - bh * n);
    const int64_t dst = (bh * cap + row0 + i) * upr + u;
    ks[dst] = kc[idx];
    vs[dst] = vc[idx];
    if (u == 0) ps[bh * cap + row0 + i] = first_pos + i;
}

// Max-pool smoothing of a score row: out[r][j] = max of in[r][j'] over
// |j' - j| <= half, clipped to [0, S).
__global__ __launch_bounds__(256) void snap_pool_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                        int64_t rows, int S, int half) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * S) return;
    const int64_t r = idx / S;
    const int j = (int)(idx - r * S);
    const float* x = in + r * S;
    const int lo = max(0, j - half), hi = min(S - 1, j + half);
    float m = x[lo];
    for (int t = lo + 1; t <= hi; ++t) m = fmaxf(m, x[t]);
    out[idx] = m;
}

}  // namespace

// Workspace: chunk statistics, then scores (used when the caller passes no
// scores buffer), then pooled scores (when pooling).
// Ready flags of the one-read scores: one per (b, h, 128-key chunk), which
// covers every chunking the one-read kernel uses (and grows with S, so a
// workspace sized for a capacity also holds a call over fewer rows).
size_t snapkv_flag_bytes(int B, int H, int S, int n_rows) {
    (void)n_rows;
    const int n_chunks = (S + kChunk - 1) / kChunk;
    return ((size_t)B * H * n_chunks * sizeof(uint64_t) + 255) & ~(size_t)255;
}

size_t snapkv_ws_bytes(int B, int H, int S, int D, int n_rows, bool pooled) {
    (void)D;
    const int n_chunks = (S + kChunk - 1) / kChunk;
    size_t stats = (size_t)B * H * n_chunks * n_rows * 2 * sizeof(float);
    stats = (stats + 255) & ~(size_t)255;
    size_t sc = (size_t)B * H * S * sizeof(float);
    sc = (sc + 255) & ~(size_t)255;
    return stats + sc + (pooled ? sc : 0) + snapkv_flag_bytes(B, H, S, n_rows);
}

int g_snap_wait_us = 200;

// One-read chunking: 256 keys per workgroup (two 32-key sub-chunks per wave)
// for up to 32 observation rows, 128 keys for more (their logits take 2 or 4
// row tiles of registers).
static int one_read_f(int rows) { return rows <= 32 ? 2 : 1; }
static int one_read_nt(int rows) { return rows <= 32 ? 1 : (rows <= 64 ? 2 : 4); }

template <int D, int F, int NT>
static int one_read_resident() {
    // workgroups of this kernel that the whole device holds at once
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] > 0) return cached[dev];
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, snap_one_read_kernel<D, F, NT>, 256, 0) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = per_cu * cus;
    return cached[dev];
}

template <int D>
static int one_read_resident_d(int F, int NT) {
    if (F == 2) return one_read_resident<D, 2, 1>();
    return NT == 2 ? one_read_resident<D, 1, 2>() : one_read_resident<D, 1, 4>();
}

bool snapkv_one_read_applies(const SnapArgs& a) {
    if (!a.flags) return false;
    const int n_keep = a.budget < a.S ? a.budget : a.S;
    // the select-gather launch clears the flags: it must be the fused one
    if (n_keep > kFuseMaxKeep || a.S > kSelThreads * 32) return false;
    const int F = one_read_f(a.n_rows), NT = one_read_nt(a.n_rows);
    const int n_c = (a.S + 128 * F - 1) / (128 * F);
    if (n_c > 256) return false;
    const int cap = a.D == 128 ? one_read_resident_d<128>(F, NT)
                               : (a.D == 64 ? one_read_resident_d<64>(F, NT) : one_read_resident_d<32>(F, NT));
    return (int64_t)a.B * a.H * n_c <= cap;
}

template <int D>
static hipError_t launch_one_read_d(const SnapArgs& a, int F, int NT, hipStream_t s) {
    const dim3 grid((unsigned)a.n_one, (unsigned)a.H, (unsigned)a.B);
    if (F == 2) hipLaunchKernelGGL((snap_one_read_kernel<D, 2, 1>), grid, dim3(256), 0, s, a);
    else if (NT == 2) hipLaunchKernelGGL((snap_one_read_kernel<D, 1, 2>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((snap_one_read_kernel<D, 1, 4>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_snapkv_scores_one_read(SnapArgs& a, hipStream_t s) {
    const int F = one_read_f(a.n_rows), NT = one_read_nt(a.n_rows);
    a.one_chunk = 128 * F;
    a.n_one = (a.S + a.one_chunk - 1) / a.one_chunk;
    if (a.D == 128) return launch_one_read_d<128>(a, F, NT, s);
    if (a.D == 64) return launch_one_read_d<64>(a, F, NT, s);
    return launch_one_read_d<32>(a, F, NT, s);
}

hipError_t launch_snapkv_pool(const float* in, float* out, int64_t rows, int S, int kernel, hipStream_t s) {
    const int64_t n = rows * S;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(snap_pool_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in, out, rows, S,
                       (kernel - 1) / 2);
    return hipGetLastError();
}

// Stats chunking: F 128-key sub-chunks per step and stat_reps steps per
// workgroup, so that at most kStatTarget partials per window row are left
// for the scores pass to merge (F <= 4 keeps the fragments in registers).
static void stat_plan(SnapArgs& a) {
    const int n128 = a.n_chunks;
    int f = 1;
    while (f < 4 && (n128 + f - 1) / f > kStatTarget) f *= 2;
    const int per = f * kStatTarget;                          // sub-chunks covered by one rep
    a.stat_f = f;
    a.stat_reps = n128 > per ? (n128 + per - 1) / per : 1;
    a.n_stat = (n128 + f * a.stat_reps - 1) / (f * a.stat_reps);
}

template <int D>
static hipError_t launch_scores_d(SnapArgs a, hipStream_t s) {
    stat_plan(a);
    dim3 sgrid((unsigned)a.n_stat, (unsigned)a.H, (unsigned)a.B);
    if (a.stat_f == 1) hipLaunchKernelGGL((snap_stats_kernel<D, 1>), sgrid, dim3(256), 0, s, a);
    else if (a.stat_f == 2) hipLaunchKernelGGL((snap_stats_kernel<D, 2>), sgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((snap_stats_kernel<D, 4>), sgrid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)a.n_chunks, (unsigned)a.H, (unsigned)a.B);
    hipLaunchKernelGGL((snap_scores_kernel<D>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_snapkv_scores(const SnapArgs& a, hipStream_t s) {
    if (a.D == 128) return launch_scores_d<128>(a, s);
    if (a.D == 64) return launch_scores_d<64>(a, s);
    return launch_scores_d<32>(a, s);
}

hipError_t launch_snapkv_select(const float* scores, int B, int H, int S, int n_sink, int budget,
                                int32_t* kept, hipStream_t s) {
    if (S <= kSelThreads * 8)
        hipLaunchKernelGGL((snap_select_reg_kernel<8>), dim3((unsigned)(B * H)), dim3(kSelThreads), 0, s, scores, S,
                           n_sink, budget, kept);
    else if (S <= kSelThreads * 16)
        hipLaunchKernelGGL((snap_select_reg_kernel<16>), dim3((unsigned)(B * H)), dim3(kSelThreads), 0, s, scores, S,
                           n_sink, budget, kept);
    else if (S <= kSelThreads * 32)
        hipLaunchKernelGGL((snap_select_reg_kernel<32>), dim3((unsigned)(B * H)), dim3(kSelThreads), 0, s, scores, S,
                           n_sink, budget, kept);
    else
        hipLaunchKernelGGL(snap_select_radix_kernel, dim3((unsigned)(B * H)), dim3(1024), 0, s, scores, S,
                           n_sink, budget, kept);
    return hipGetLastError();
}

hipError_t launch_snapkv_chunk_copy(const void* k_chunk, const void* v_chunk, void* k_state, void* v_state,
                                    int32_t* pos_state, int B, int H, int D, int n, int cap, int row0,
                                    int first_pos, hipStream_t s) {
    const int upr = D / 8;
    const int64_t rows = (int64_t)B * H * n;
    const int64_t total = rows * upr;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(snap_chunk_copy_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint4*>(k_chunk), static_cast<const uint4*>(v_chunk),
                       static_cast<uint4*>(k_state), static_cast<uint4*>(v_state), pos_state, rows, n, upr, cap,
                       row0, first_pos);
    return hipGetLastError();
}

hipError_t launch_snapkv_select_gather(const SnapArgs& a, const float* rank, hipStream_t s) {
    const int n_keep = a.budget < a.S ? a.budget : a.S;
    if (n_keep > kFuseMaxKeep || a.S > kSelThreads * 32) {
        const hipError_t e = launch_snapkv_select(rank, a.B, a.H, a.S, a.n_sink, a.budget, a.kept, s);
        if (e != hipSuccess) return e;
        return launch_snapkv_gather(a, s);
    }
    // about one 16-byte unit of K and of V per thread and block
    int n_rep = (n_keep * (a.D / 8) + kSelThreads - 1) / kSelThreads;
    n_rep = n_rep < 1 ? 1 : (n_rep > 32 ? 32 : n_rep);
    const dim3 grid((unsigned)((a.B * a.H + kXcds - 1) / kXcds * n_rep * kXcds));
    if (a.S <= kSelThreads * 8)
        hipLaunchKernelGGL((snap_select_gather_kernel<8>), grid, dim3(kSelThreads), 0, s, a, rank, n_rep);
    else if (a.S <= kSelThreads * 16)
        hipLaunchKernelGGL((snap_select_gather_kernel<16>), grid, dim3(kSelThreads), 0, s, a, rank, n_rep);
    else
        hipLaunchKernelGGL((snap_select_gather_kernel<32>), grid, dim3(kSelThreads), 0, s, a, rank, n_rep);
    return hipGetLastError();
}

hipError_t launch_snapkv_gather(const SnapArgs& a, hipStream_t s) {
    const int n_keep = a.budget < a.S ? a.budget : a.S;
    const int64_t total = (int64_t)a.B * a.H * n_keep * (a.D / 8);
    hipLaunchKernelGGL(snap_gather_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, n_keep);
    return hipGetLastError();
}

}  // namespace kvq

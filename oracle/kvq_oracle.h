/*
 * kvq_oracle.h -- plain CPU reference for the compressed-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no source with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [P1] "StreamingLLM + KIVI -- long-context decode without growing the KV
 *        cache" (posttrainllm.com): sections "Affine quantisation formula",
 *        "Implementation", "The bug class the previous attempt hit".
 *   [P2] "SnapKV -- Prefill Observation-Window Token Eviction"
 *        (veloxquant-mlx): section "How it works", "Evidence".
 *   [P3] "kv-cache: optional per-channel K-cache mean-centering for Q4_0"
 *        (llama.cpp PR #51): sections "The idea", "Why this is safe".
 *   [P4] "Low-bit KV caches on MLX: what exists and what is missing":
 *        sections 1 ("What mlx-lm ships today") and 3 (KIVI residual buffer).
 *
 * Precision: quantization runs in IEEE fp32 exactly as the specification
 * fixes it (codes must match bit-for-bit); attention and SnapKV scores run in
 * fp64 as ground truth.  Codes are held one per byte ("canonical" layout);
 * packing into nibbles is a storage detail checked separately.
 *
 * Parity pins: every function here is checked in tests/test_oracle_pins.py
 * against closed forms, brute force, library routines or the pages' numbers.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats (IEEE 754 binary16 / bfloat16) ---------------------- */
uint16_t kvo_f32_to_f16(float x);      /* round to nearest, ties to even; keeps subnormals */
float    kvo_f16_to_f32(uint16_t h);   /* exact */
float    kvo_bf16_to_f32(uint16_t b);  /* exact */
void     kvo_f32_to_f16_n(const float* x, int64_t n, uint16_t* out);
void     kvo_f16_to_f32_n(const uint16_t* h, int64_t n, float* out);

/* ---- A2 / A4: per-token asymmetric group quantization ------------------- *
 * [P1] "Affine quantisation formula" applied along head_dim in groups of G
 * channels ([P4] s.1: mx.quantize groups the last axis).
 * x: [rows][D] fp32.  u: [rows][D] codes in [0, 2^bits-1].
 * meta: [rows][D/G][2] fp16 bit patterns (scale, zero).                       */
void kvo_quant_tok_affine(const float* x, int64_t rows, int D, int G, int bits,
                          uint8_t* u, uint16_t* meta);

/* ---- A1: KIVI per-channel quantization of one closed group of Gt tokens --- *
 * [P1] "KIVI" (K per channel) with scales frozen per token group ([P1]
 * caveats: the KIVI group-size idea; [P4] s.3: keys quantize in closed blocks).
 * x: [Gt][D] fp32.  u: [Gt][D].  meta: [D][2] fp16 (scale, zero) per channel. */
void kvo_quant_channel_group(const float* x, int Gt, int D, int bits,
                             uint8_t* u, uint16_t* meta);

/* ---- A3: symmetric 4-bit blocks of 32 channels with optional centering ---- *
 * [P3] "The idea": subtract a fixed per-(kv-head, channel) mean before a
 * symmetric (zero-point-free) 4-bit block quantizer.
 * x: [rows][D] fp32; bias: [D] fp32 or NULL.  u: [rows][D] codes q+8 in [0,15].
 * scale: [rows][D/32] fp16.                                                   */
void kvo_quant_sym4(const float* x, int64_t rows, int D, const float* bias,
                    uint8_t* u, uint16_t* scale);

/* ---- B: decode attention over a dequantized view (fp64) ----------------- */
enum { KVO_PLAIN = 0, KVO_CHANNEL = 1, KVO_TOK_AFFINE = 2, KVO_SYM4 = 3 };

typedef struct {
    int kind;                 /* KVO_* */
    int D;                    /* head_dim */
    int G;                    /* channels per group (TOK_AFFINE) */
    const uint8_t* u;         /* [T][D] codes (CHANNEL, TOK_AFFINE, SYM4) */
    const uint16_t* meta;     /* TOK_AFFINE [T][D/G][2]; SYM4 [T][D/32];
                                 CHANNEL table [rows][D][2] */
    const int32_t* row;       /* CHANNEL: [T] table row of each slot */
    const float* plain;       /* PLAIN: [T][D] values; CHANNEL: residual rows */
    int n_coded;              /* CHANNEL: slots [0,n_coded) are coded; slot t >= n_coded
                                 reads plain[(t - n_coded)*D + d] */
} kvo_view;

double kvo_dequant(const kvo_view* v, int t, int d);

/* One query head: out[d] = sum_t softmax_t(scale * q.k_t) v_t[d] in fp64.
 * T == 0 gives out = 0.                                                       */
void kvo_decode_head(const kvo_view* K, const kvo_view* V, int T,
                     const float* q, double scale, double* out);

/* ---- RoPE applied on read ("StreamingLLM + KIVI", "RoPE caveat") -------- *
 * Keys stored before the rotary embedding are rotated when read, at their
 * slot index in the compressed cache.  Rotation in the half-split form: for
 * j < D/2 the pair (x_j, x_{j+D/2}) turns by the angle pos * base^(-2j/D).
 * x: [D] fp64, rotated in place.                                             */
void kvo_rope_rotate(double* x, int D, double base, int pos);

/* kvo_decode_head with RoPE on read: the query is rotated at q_pos, the key
 * of slot t at position t, then attention as kvo_decode_head (fp64).         */
void kvo_decode_head_rope(const kvo_view* K, const kvo_view* V, int T,
                          const float* q, double scale, double base, int q_pos,
                          double* out);

/* ---- D1: SnapKV observation-window scores (fp64) ------------------------ *
 * [P2] "How it works" step 1: the row softmax of the last w keys against all keys (scaled by 1/sqrt(D)), averaged over
 * the window; w clamped to S.  K: [S][D] fp32.  score: [S].                   */
void kvo_snapkv_scores(const float* K, int S, int D, int w, double* score);

/* ---- SnapKV with given observation rows (fp64) ---------------------------- *
 * [P2] "Proxy limitation": the SnapKV paper scores with the prompt's final
 * query vectors rather than the trailing key rows.  score[j] = mean over the
 * n_rows rows r of softmax_j(Q[r] . K[j] / sqrt(D)), no mask.
 * Q: [n_rows][D] fp32, K: [S][D] fp32, score: [S].                          */
void kvo_snapkv_scores_rows(const float* Q, int n_rows, const float* K, int S, int D, double* score);

/* ---- max-pool smoothing of scores ------------------------------------------ *
 * [P2] "Proxy limitation": the paper smooths the scores with a max-pool of
 * width kernel > 1 before ranking.  out[j] = max of in[j'] over
 * j - (kernel-1)/2 <= j' <= j + (kernel-1)/2, 0 <= j' < S.  kernel odd.     */
void kvo_maxpool1d(const float* in, int S, int kernel, float* out);

/* ---- D2: sink guarantee + top-k + sorted union -------------------------- *
 * [P2] "How it works" steps 2-3.  Ties are broken by the lower index.
 * kept: [min(budget, S)] ascending positions.  Returns the count.           */
int kvo_snapkv_select(const float* score, int S, int n_sink, int budget, int32_t* kept);

#ifdef __cplusplus
}
#endif
#endif
